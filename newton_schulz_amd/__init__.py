"""Python binding of the NVFP4 Newton–Schulz library (libnvfp4ns.so).

Argument marshalling only: every step runs in the HIP kernels behind the C
ABI declared in ``include/nvfp4ns.h``.  torch supplies device memory and the
current stream.  There is no fallback: if the library is missing this
module raises ImportError.

Functions carry the C names:
    nvfp4_quantize, nvfp4_quantize_noalloc, nvfp4_quantize_rht, nvfp4_dequantize,
    nvfp4_gemm_workspace_bytes, nvfp4_gemm, ns_workspace_bytes, ns_workspace_layout,
    ns_orthogonalize, ns_orthogonalize_rht, ns_orthogonalize_ex,
    ns_abs_quantile_workspace_bytes, ns_abs_quantile,
    ns_grouped_workspace_bytes, ns_orthogonalize_grouped, ns_orthogonalize_grouped_ex,
    ns_orthogonalize_grouped_on
"""
import ctypes
import os

# torch first: the library must bind to the HIP runtime torch has loaded (the
# one that owns the devices, streams and memory it is handed), not bring in
# a second copy ahead of it.
import torch  # noqa: F401

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libnvfp4ns.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python newton_schulz_amd/build.py` "
        "(or __graft_entry__.build()) first")

_lib = ctypes.CDLL(LIB_PATH)

NS_OK, NS_ERR_ARG, NS_ERR_SHAPE, NS_ERR_WORKSPACE, NS_ERR_HIP = 0, -1, -2, -3, -4
NS_F32, NS_BF16 = 0, 1
NVFP4_ROWS, NVFP4_COLS = 0, 1
STATUS_NAMES = {0: "NS_OK", -1: "NS_ERR_ARG", -2: "NS_ERR_SHAPE",
                -3: "NS_ERR_WORKSPACE", -4: "NS_ERR_HIP"}

_i64, _sz, _vp, _f, _i = ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float, ctypes.c_int
_u16 = ctypes.c_uint16
_d = ctypes.c_double


class NsOptions(ctypes.Structure):
    """ns_options of the C ABI."""
    _fields_ = [("clip", ctypes.c_float), ("clip_quantile", ctypes.c_double),
                ("rht_masks", ctypes.POINTER(ctypes.c_uint16)), ("adaptive46", ctypes.c_int)]

class NsWorkspaceMap(ctypes.Structure):
    """ns_workspace_map of the C ABI (byte offsets into an NS workspace)."""
    _fields_ = [("xm", ctypes.c_int64), ("xn", ctypes.c_int64),
                ("x", ctypes.c_size_t), ("a", ctypes.c_size_t), ("b", ctypes.c_size_t),
                ("qx_codes", ctypes.c_size_t), ("qx_scales", ctypes.c_size_t),
                ("qt_codes", ctypes.c_size_t), ("qt_scales", ctypes.c_size_t),
                ("qa_codes", ctypes.c_size_t), ("qa_scales", ctypes.c_size_t),
                ("qb_codes", ctypes.c_size_t), ("qb_scales", ctypes.c_size_t),
                ("global_scales", ctypes.c_size_t), ("total", ctypes.c_size_t)]


_SIGS = {
    "nvfp4_quantize_workspace_bytes": (_sz, [_i64, _i64]),
    "nvfp4_quantize": (_i, [_vp, _i, _i64, _i64, _i, _vp, _vp, _vp, _vp, _sz, _vp]),
    "nvfp4_quantize_noalloc": (_i, [_vp, _i, _i64, _i64, _i, _vp, _vp, _vp, _vp]),
    "nvfp4_quantize_rht": (_i, [_vp, _i, _i64, _i64, _i, _u16, _vp, _vp, _vp, _vp, _sz, _vp]),
    "nvfp4_quantize_46": (_i, [_vp, _i, _i64, _i64, _i, _vp, _vp, _vp, _vp, _sz, _vp]),
    "nvfp4_dequantize": (_i, [_vp, _vp, _vp, _i64, _i64, _i, _vp, _i, _vp]),
    "nvfp4_gemm_workspace_bytes": (_sz, [_i64, _i64, _i64, _i]),
    "nvfp4_gemm": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i, _f, _f, _vp, _vp, _vp,
                        _vp, _sz, _vp]),
    "ns_workspace_bytes": (_sz, [_i64, _i64]),
    "ns_workspace_layout": (_i, [_i64, _i64, _vp]),
    "ns_orthogonalize": (_i, [_vp, _i, _i64, _i64, _vp, _i, _f, _vp, _i, _vp, _sz, _vp]),
    "ns_orthogonalize_rht": (_i, [_vp, _i, _i64, _i64, _vp, _i, _f, _vp, _vp, _i, _vp, _sz, _vp]),
    "ns_orthogonalize_ex": (_i, [_vp, _i, _i64, _i64, _vp, _i, _vp, _vp, _i, _vp, _sz, _vp]),
    "ns_abs_quantile_workspace_bytes": (_sz, []),
    "ns_abs_quantile": (_i, [_vp, _i, _i64, _d, _vp, _vp, _sz, _vp]),
    "ns_grouped_workspace_bytes": (_sz, [_i, _vp, _vp]),
    "ns_orthogonalize_grouped": (_i, [_i, _vp, _vp, _vp, _i, _vp, _i, _vp, _vp, _i, _vp, _sz, _vp]),
    "ns_orthogonalize_grouped_ex": (_i, [_i, _vp, _vp, _vp, _i, _vp, _i, _vp, _vp, _vp, _i, _vp, _sz,
                                         _vp]),
    "ns_orthogonalize_grouped_on": (_i, [_i, _vp, _vp, _vp, _i, _vp, _i, _vp, _vp, _vp, _i, _vp, _sz,
                                         _vp, _i, _vp]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTED = tuple(_SIGS)


class NSError(RuntimeError):
    def __init__(self, status, where):
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}")
        self.status = status


def _check(status, where):
    if status != NS_OK:
        raise NSError(status, where)


def _torch():
    import torch
    return torch


def _stream(stream, device=None):
    """The stream to enqueue on: `stream`, else the current stream of the
    tensors' device."""
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _dt(t):
    torch = _torch()
    if t.dtype == torch.float32:
        return NS_F32
    if t.dtype == torch.bfloat16:
        return NS_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _out_dtype(code):
    torch = _torch()
    return torch.float32 if code == NS_F32 else torch.bfloat16


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need_cuda(*ts):
    ts = [t for t in ts if t is not None]
    for t in ts:
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("tensors must be contiguous device tensors")
    if any(t.device != ts[0].device for t in ts):
        raise ValueError("tensors must be on one device")


def _need(t, name, dtypes, numel):
    """A caller-supplied tensor: one of `dtypes` and at least `numel`
    elements, so that no kernel reads or writes past its end."""
    if t is None:
        return
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype}, expected one of {dtypes}")
    if t.numel() < numel:
        raise ValueError(f"{name}: {t.numel()} elements, at least {numel} needed")


def _need_shape(t, name, shape):
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")


def _floats():
    torch = _torch()
    return (torch.float32, torch.bfloat16)


# ------------------------------------------------------------- quantizer --

def nvfp4_quantize(x, axis=NVFP4_ROWS, codes=None, scales=None, global_scale=None,
                   workspace=None, stream=None, adaptive46=False):
    """NVFP4 quantization of a 2-D float32/bfloat16 device tensor.

    Returns (codes uint8 [r][c/2], scales uint8 [r][c/16], s_g float32 [1]),
    in the layout of x (NVFP4_ROWS) or of x^T (NVFP4_COLS).  adaptive46=True
    calls nvfp4_quantize_46 (adaptive 4/6 block scaling).
    """
    torch = _torch()
    _need_cuda(x)
    rows, cols = x.shape
    r, c = (rows, cols) if axis == NVFP4_ROWS else (cols, rows)
    dev = x.device
    if codes is None:
        codes = torch.empty((r, c // 2), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((r, c // 16), dtype=torch.uint8, device=dev)
    if global_scale is None:
        global_scale = torch.empty(1, dtype=torch.float32, device=dev)
    wsb = _lib.nvfp4_quantize_workspace_bytes(rows, cols)
    if workspace is None:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=dev)
    _need_quant_outputs(x, rows, cols, codes, scales, global_scale, workspace)
    fn, name = ((_lib.nvfp4_quantize_46, "nvfp4_quantize_46") if adaptive46
                else (_lib.nvfp4_quantize, "nvfp4_quantize"))
    with torch.cuda.device(dev):
        _check(fn(_ptr(x), _dt(x), rows, cols, axis, _ptr(codes), _ptr(scales), _ptr(global_scale),
                  _ptr(workspace), workspace.numel(), _stream(stream, dev)), name)
    return codes, scales, global_scale


def nvfp4_quantize_noalloc(x, axis=NVFP4_ROWS, codes=None, scales=None, global_scale=None,
                           stream=None):
    """nvfp4_quantize through the allocation-free entry point (its scratch is
    the library's static device array); outputs as nvfp4_quantize."""
    torch = _torch()
    _need_cuda(x)
    rows, cols = x.shape
    r, c = (rows, cols) if axis == NVFP4_ROWS else (cols, rows)
    dev = x.device
    if codes is None:
        codes = torch.empty((r, c // 2), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((r, c // 16), dtype=torch.uint8, device=dev)
    if global_scale is None:
        global_scale = torch.empty(1, dtype=torch.float32, device=dev)
    _need_quant_outputs(x, rows, cols, codes, scales, global_scale, None)
    with torch.cuda.device(dev):
        _check(_lib.nvfp4_quantize_noalloc(_ptr(x), _dt(x), rows, cols, axis, _ptr(codes),
                                           _ptr(scales), _ptr(global_scale),
                                           _stream(stream, dev)), "nvfp4_quantize_noalloc")
    return codes, scales, global_scale


def _need_quant_outputs(x, rows, cols, codes, scales, global_scale, workspace):
    torch = _torch()
    _need_cuda(x, codes, scales, global_scale, workspace)
    _need(codes, "codes", (torch.uint8,), rows * cols // 2)
    _need(scales, "scales", (torch.uint8,), rows * cols // 16)
    _need(global_scale, "global_scale", (torch.float32,), 1)
    _need(workspace, "workspace", (torch.uint8,), 0)


def nvfp4_quantize_rht(x, mask, axis=NVFP4_ROWS, codes=None, scales=None, global_scale=None,
                       workspace=None, stream=None):
    """Q_1x16(x H) (NVFP4_ROWS) or Q_16x1(H^T x) (NVFP4_COLS) with the random
    Hadamard transform H_16^r of the 16-bit sign mask; outputs as
    nvfp4_quantize."""
    torch = _torch()
    _need_cuda(x)
    rows, cols = x.shape
    r, c = (rows, cols) if axis == NVFP4_ROWS else (cols, rows)
    dev = x.device
    if codes is None:
        codes = torch.empty((r, c // 2), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((r, c // 16), dtype=torch.uint8, device=dev)
    if global_scale is None:
        global_scale = torch.empty(1, dtype=torch.float32, device=dev)
    wsb = _lib.nvfp4_quantize_workspace_bytes(rows, cols)
    if workspace is None:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=dev)
    _need_quant_outputs(x, rows, cols, codes, scales, global_scale, workspace)
    with torch.cuda.device(dev):
        _check(_lib.nvfp4_quantize_rht(_ptr(x), _dt(x), rows, cols, axis, int(mask) & 0xFFFF,
                                       _ptr(codes), _ptr(scales), _ptr(global_scale),
                                       _ptr(workspace), workspace.numel(), _stream(stream, dev)),
               "nvfp4_quantize_rht")
    return codes, scales, global_scale


def nvfp4_dequantize(codes, scales, global_scale, rows, cols, axis=NVFP4_ROWS,
                     out_dtype=NS_F32, out=None, stream=None):
    """x_hat = x_E2M1 * s * s_g, in the original rows x cols orientation."""
    torch = _torch()
    _need_cuda(codes, scales, global_scale, out)
    if out is None:
        out = torch.empty((rows, cols), dtype=_out_dtype(out_dtype), device=codes.device)
    _need(codes, "codes", (torch.uint8,), rows * cols // 2)
    _need(scales, "scales", (torch.uint8,), rows * cols // 16)
    _need(global_scale, "global_scale", (torch.float32,), 1)
    _need(out, "out", (_out_dtype(out_dtype),), rows * cols)
    with torch.cuda.device(codes.device):
        _check(_lib.nvfp4_dequantize(_ptr(codes), _ptr(scales), _ptr(global_scale), rows, cols,
                                     axis, _ptr(out), out_dtype, _stream(stream, codes.device)),
               "nvfp4_dequantize")
    return out


def nvfp4_quantize_workspace_bytes(rows, cols):
    return int(_lib.nvfp4_quantize_workspace_bytes(rows, cols))


def nvfp4_gemm_workspace_bytes(M, N, K, symmetric=False):
    return int(_lib.nvfp4_gemm_workspace_bytes(M, N, K, 1 if symmetric else 0))


def nvfp4_gemm(p, q, M, N, K, symmetric=False, alpha=1.0, beta=0.0, addend=None, out=None,
               amax_out=None, workspace=None, split=True, stream=None):
    """out = beta*addend + alpha*s_gP*s_gQ*(P Q^T); p, q = (codes, scales, s_g).

    With split=True (default) a workspace of nvfp4_gemm_workspace_bytes() is
    allocated when none is given, so the product runs with the same launch
    schedule as inside ns_orthogonalize.
    """
    torch = _torch()
    (pc, ps, pg), (qc, qs, qg) = p, q
    _need_cuda(pc, ps, pg, qc, qs, qg, addend, out, amax_out)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=pc.device)
    if workspace is None and split:
        nb = nvfp4_gemm_workspace_bytes(M, N, K, symmetric)
        workspace = torch.empty(max(nb, 1), dtype=torch.uint8, device=pc.device)
    _need_cuda(pc, workspace)
    u8 = (torch.uint8,)
    _need(pc, "p codes", u8, M * K // 2)
    _need(ps, "p scales", u8, M * K // 16)
    _need(qc, "q codes", u8, N * K // 2)
    _need(qs, "q scales", u8, N * K // 16)
    _need(pg, "p s_g", (torch.float32,), 1)
    _need(qg, "q s_g", (torch.float32,), 1)
    _need(out, "out", (torch.float32,), M * N)
    if float(beta) != 0.0:
        _need(addend, "addend", (torch.float32,), M * N)
    _need(amax_out, "amax_out", (torch.int32, torch.uint32), 1)
    _need(workspace, "workspace", u8, 0)
    wsp, wsn = (_ptr(workspace), workspace.numel()) if workspace is not None else (_ptr(None), 0)
    with torch.cuda.device(pc.device):
        _check(_lib.nvfp4_gemm(_ptr(pc), _ptr(ps), _ptr(pg), _ptr(qc), _ptr(qs), _ptr(qg),
                               M, N, K, 1 if symmetric else 0, float(alpha), float(beta),
                               _ptr(addend), _ptr(out), _ptr(amax_out), wsp, wsn,
                               _stream(stream, pc.device)),
               "nvfp4_gemm")
    return out


# ---------------------------------------------------------- Newton–Schulz --

def ns_workspace_bytes(m, n):
    return int(_lib.ns_workspace_bytes(m, n))


def ns_workspace_layout(m, n):
    """ns_workspace_layout: dict of the byte offsets (and xm, xn, total) of
    the iteration's operands inside an ns_orthogonalize workspace."""
    mp = NsWorkspaceMap()
    _check(_lib.ns_workspace_layout(m, n, ctypes.byref(mp)), "ns_workspace_layout")
    return {name: int(getattr(mp, name)) for name, _ in NsWorkspaceMap._fields_}


def ns_workspace_views(ws, m, n):
    """Views of the operands inside an NS workspace (uint8 device tensor):
    X, A, B as float32 matrices, the four NVFP4 operands as (codes, scales)
    uint8 matrices, and the four tensor scales as float32[4]."""
    torch = _torch()
    L = ns_workspace_layout(m, n)
    xm, xn = L["xm"], L["xn"]

    def f32(off, r, c):
        return ws[off:off + 4 * r * c].view(torch.float32).view(r, c)

    def u8(off, r, c):
        return ws[off:off + r * c].view(r, c)

    return {"X": f32(L["x"], xm, xn), "A": f32(L["a"], xm, xm), "B": f32(L["b"], xm, xm),
            "qX": (u8(L["qx_codes"], xm, xn // 2), u8(L["qx_scales"], xm, xn // 16)),
            "qX16": (u8(L["qt_codes"], xn, xm // 2), u8(L["qt_scales"], xn, xm // 16)),
            "qA": (u8(L["qa_codes"], xm, xm // 2), u8(L["qa_scales"], xm, xm // 16)),
            "qB": (u8(L["qb_codes"], xm, xm // 2), u8(L["qb_scales"], xm, xm // 16)),
            "sg": ws[L["global_scales"]:L["global_scales"] + 16].view(torch.float32)}


def _need_ns(G, out, workspace):
    torch = _torch()
    _need_cuda(G, out, workspace)
    _need_shape(out, "out", G.shape)
    _need(out, "out", _floats(), G.numel())
    _need(workspace, "workspace", (torch.uint8,), 0)


def _coeff_array(coeffs):
    flat = [float(v) for abc in coeffs for v in abc]
    return (ctypes.c_float * len(flat))(*flat), len(flat) // 3


def ns_orthogonalize(G, coeffs, clip=float("inf"), out_dtype=NS_F32, out=None, workspace=None,
                     stream=None):
    """k NVFP4 Newton–Schulz steps on one m x n float32/bfloat16 matrix."""
    torch = _torch()
    _need_cuda(G, out)
    m, n = G.shape
    if out is None:
        out = torch.empty((m, n), dtype=_out_dtype(out_dtype), device=G.device)
    if workspace is None:
        workspace = torch.empty(ns_workspace_bytes(m, n), dtype=torch.uint8, device=G.device)
    _need_ns(G, out, workspace)
    carr, k = _coeff_array(coeffs)
    with torch.cuda.device(G.device):
        _check(_lib.ns_orthogonalize(_ptr(G), _dt(G), m, n, carr, k, float(clip), _ptr(out),
                                     _dt(out), _ptr(workspace), workspace.numel(),
                                     _stream(stream, G.device)), "ns_orthogonalize")
    return out


def ns_orthogonalize_rht(G, coeffs, masks, clip=float("inf"), out_dtype=NS_F32, out=None,
                         workspace=None, stream=None):
    """ns_orthogonalize with the random Hadamard transform of each step
    (one 16-bit sign mask per coefficient triple)."""
    torch = _torch()
    _need_cuda(G, out)
    m, n = G.shape
    if out is None:
        out = torch.empty((m, n), dtype=_out_dtype(out_dtype), device=G.device)
    if workspace is None:
        workspace = torch.empty(ns_workspace_bytes(m, n), dtype=torch.uint8, device=G.device)
    _need_ns(G, out, workspace)
    carr, k = _coeff_array(coeffs)
    if len(masks) != k:
        raise ValueError("one Hadamard mask per step")
    marr = (ctypes.c_uint16 * k)(*[int(v) & 0xFFFF for v in masks])
    with torch.cuda.device(G.device):
        _check(_lib.ns_orthogonalize_rht(_ptr(G), _dt(G), m, n, carr, k, float(clip), marr,
                                         _ptr(out), _dt(out), _ptr(workspace), workspace.numel(),
                                         _stream(stream, G.device)), "ns_orthogonalize_rht")
    return out


def ns_orthogonalize_ex(G, coeffs, clip=float("inf"), clip_quantile=0.0, rht_masks=None,
                        out_dtype=NS_F32, out=None, workspace=None, stream=None, adaptive46=False):
    """ns_orthogonalize with an on-device quantile clip (clip_quantile in
    (0, 1]; 0 uses `clip`), the random Hadamard transform (one 16-bit mask
    per step) and/or adaptive 4/6 block scaling on every quantization."""
    torch = _torch()
    _need_cuda(G, out)
    m, n = G.shape
    if out is None:
        out = torch.empty((m, n), dtype=_out_dtype(out_dtype), device=G.device)
    if workspace is None:
        workspace = torch.empty(ns_workspace_bytes(m, n), dtype=torch.uint8, device=G.device)
    _need_ns(G, out, workspace)
    carr, k = _coeff_array(coeffs)
    opt = NsOptions(float(clip), float(clip_quantile), None, 1 if adaptive46 else 0)
    marr = None
    if rht_masks is not None:
        if len(rht_masks) != k:
            raise ValueError("one Hadamard mask per step")
        marr = (ctypes.c_uint16 * k)(*[int(v) & 0xFFFF for v in rht_masks])
        opt.rht_masks = ctypes.cast(marr, ctypes.POINTER(ctypes.c_uint16))
    with torch.cuda.device(G.device):
        _check(_lib.ns_orthogonalize_ex(_ptr(G), _dt(G), m, n, carr, k, ctypes.byref(opt),
                                        _ptr(out), _dt(out), _ptr(workspace), workspace.numel(),
                                        _stream(stream, G.device)), "ns_orthogonalize_ex")
    return out


def ns_abs_quantile_workspace_bytes():
    return int(_lib.ns_abs_quantile_workspace_bytes())


def ns_abs_quantile(x, q, out=None, workspace=None, stream=None):
    """The q-quantile of |x| (k-th smallest magnitude, k = ceil(q N)) as a
    one-element float32 device tensor."""
    torch = _torch()
    _need_cuda(x)
    if out is None:
        out = torch.empty(1, dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = torch.empty(ns_abs_quantile_workspace_bytes(), dtype=torch.uint8, device=x.device)
    _need_cuda(x, out, workspace)
    _need(out, "out", (torch.float32,), 1)
    _need(workspace, "workspace", (torch.uint8,), 0)
    with torch.cuda.device(x.device):
        _check(_lib.ns_abs_quantile(_ptr(x), _dt(x), x.numel(), float(q), _ptr(out),
                                    _ptr(workspace), workspace.numel(), _stream(stream, x.device)),
               "ns_abs_quantile")
    return out


def ns_grouped_workspace_bytes(shapes):
    cnt = len(shapes)
    ms = (ctypes.c_int64 * cnt)(*[s[0] for s in shapes])
    ns = (ctypes.c_int64 * cnt)(*[s[1] for s in shapes])
    return int(_lib.ns_grouped_workspace_bytes(cnt, ms, ns))


def ns_orthogonalize_grouped(Gs, coeffs, clips, out_dtype=NS_F32, outs=None, workspace=None,
                             stream=None):
    """ns_orthogonalize over a list of matrices with one schedule."""
    torch = _torch()
    cnt = len(Gs)
    _need_cuda(*Gs)
    dt = _dt(Gs[0])
    if any(_dt(g) != dt for g in Gs):
        raise TypeError("all inputs must share one dtype")
    shapes = [tuple(g.shape) for g in Gs]
    if outs is None:
        outs = [torch.empty(s, dtype=_out_dtype(out_dtype), device=Gs[0].device) for s in shapes]
    if workspace is None:
        workspace = torch.empty(ns_grouped_workspace_bytes(shapes), dtype=torch.uint8,
                                device=Gs[0].device)
    _need_group(Gs, outs, workspace)
    if len(clips) != cnt:
        raise ValueError("one clip per matrix")
    gp = (ctypes.c_void_p * cnt)(*[g.data_ptr() for g in Gs])
    op = (ctypes.c_void_p * cnt)(*[o.data_ptr() for o in outs])
    ms = (ctypes.c_int64 * cnt)(*[s[0] for s in shapes])
    ns = (ctypes.c_int64 * cnt)(*[s[1] for s in shapes])
    cl = (ctypes.c_float * cnt)(*[float(c) for c in clips])
    carr, k = _coeff_array(coeffs)
    dev = Gs[0].device
    with torch.cuda.device(dev):
        _check(_lib.ns_orthogonalize_grouped(cnt, gp, ms, ns, dt, carr, k, cl, op, _dt(outs[0]),
                                             _ptr(workspace), workspace.numel(),
                                             _stream(stream, dev)), "ns_orthogonalize_grouped")
    return outs


def _need_group(Gs, outs, workspace):
    torch = _torch()
    if len(Gs) == 0 or len(outs) != len(Gs):
        raise ValueError("one output per matrix, at least one matrix")
    _need_cuda(*Gs, *outs, workspace)
    for i, (g, o) in enumerate(zip(Gs, outs)):
        _need_shape(o, f"outs[{i}]", g.shape)
        _need(o, f"outs[{i}]", (outs[0].dtype,), g.numel())
    _need(outs[0], "outs[0]", _floats(), 0)
    _need(workspace, "workspace", (torch.uint8,), 0)


def ns_orthogonalize_grouped_ex(Gs, coeffs, clips=None, clip_quantile=0.0, rht_masks=None,
                                out_dtype=NS_F32, outs=None, workspace=None, stream=None,
                                adaptive46=False):
    """ns_orthogonalize_grouped with a per-matrix quantile clip, the random
    Hadamard transform and/or adaptive 4/6 scaling (options shared by every
    matrix)."""
    torch = _torch()
    cnt = len(Gs)
    _need_cuda(*Gs)
    dt = _dt(Gs[0])
    if any(_dt(g) != dt for g in Gs):
        raise TypeError("all inputs must share one dtype")
    shapes = [tuple(g.shape) for g in Gs]
    if outs is None:
        outs = [torch.empty(s, dtype=_out_dtype(out_dtype), device=Gs[0].device) for s in shapes]
    if workspace is None:
        workspace = torch.empty(ns_grouped_workspace_bytes(shapes), dtype=torch.uint8,
                                device=Gs[0].device)
    _need_group(Gs, outs, workspace)
    if clips is not None and len(clips) != cnt:
        raise ValueError("one clip per matrix")
    gp = (ctypes.c_void_p * cnt)(*[g.data_ptr() for g in Gs])
    op = (ctypes.c_void_p * cnt)(*[o.data_ptr() for o in outs])
    ms = (ctypes.c_int64 * cnt)(*[s[0] for s in shapes])
    ns_ = (ctypes.c_int64 * cnt)(*[s[1] for s in shapes])
    cl = (ctypes.c_float * cnt)(*[float(c) for c in clips]) if clips is not None else None
    carr, k = _coeff_array(coeffs)
    opt = NsOptions(float("inf"), float(clip_quantile), None, 1 if adaptive46 else 0)
    marr = None
    if rht_masks is not None:
        if len(rht_masks) != k:
            raise ValueError("one Hadamard mask per step")
        marr = (ctypes.c_uint16 * k)(*[int(v) & 0xFFFF for v in rht_masks])
        opt.rht_masks = ctypes.cast(marr, ctypes.POINTER(ctypes.c_uint16))
    dev = Gs[0].device
    with torch.cuda.device(dev):
        _check(_lib.ns_orthogonalize_grouped_ex(cnt, gp, ms, ns_, dt, carr, k, cl,
                                                ctypes.byref(opt), op, _dt(outs[0]),
                                                _ptr(workspace), workspace.numel(),
                                                _stream(stream, dev)),
               "ns_orthogonalize_grouped_ex")
    return outs


def ns_orthogonalize_grouped_on(Gs, coeffs, streams, clips=None, clip_quantile=0.0,
                                rht_masks=None, adaptive46=False, out_dtype=NS_F32, outs=None,
                                workspace=None, stream=None):
    """ns_orthogonalize_grouped_ex on the caller's streams (a list of
    torch.cuda.Stream, 1 to 16): the library keeps nothing between calls."""
    torch = _torch()
    cnt = len(Gs)
    _need_cuda(*Gs)
    dt = _dt(Gs[0])
    if any(_dt(g) != dt for g in Gs):
        raise TypeError("all inputs must share one dtype")
    shapes = [tuple(g.shape) for g in Gs]
    if outs is None:
        outs = [torch.empty(s, dtype=_out_dtype(out_dtype), device=Gs[0].device) for s in shapes]
    if workspace is None:
        workspace = torch.empty(ns_grouped_workspace_bytes(shapes), dtype=torch.uint8,
                                device=Gs[0].device)
    _need_group(Gs, outs, workspace)
    if clips is not None and len(clips) != cnt:
        raise ValueError("one clip per matrix")
    gp = (ctypes.c_void_p * cnt)(*[g.data_ptr() for g in Gs])
    op = (ctypes.c_void_p * cnt)(*[o.data_ptr() for o in outs])
    ms = (ctypes.c_int64 * cnt)(*[s[0] for s in shapes])
    ns_ = (ctypes.c_int64 * cnt)(*[s[1] for s in shapes])
    cl = (ctypes.c_float * cnt)(*[float(c) for c in clips]) if clips is not None else None
    carr, k = _coeff_array(coeffs)
    opt = NsOptions(float("inf"), float(clip_quantile), None, 1 if adaptive46 else 0)
    marr = None
    if rht_masks is not None:
        if len(rht_masks) != k:
            raise ValueError("one Hadamard mask per step")
        marr = (ctypes.c_uint16 * k)(*[int(v) & 0xFFFF for v in rht_masks])
        opt.rht_masks = ctypes.cast(marr, ctypes.POINTER(ctypes.c_uint16))
    sarr = (ctypes.c_void_p * max(len(streams), 1))(*[s.cuda_stream for s in streams])
    dev = Gs[0].device
    with torch.cuda.device(dev):
        _check(_lib.ns_orthogonalize_grouped_on(cnt, gp, ms, ns_, dt, carr, k, cl,
                                                ctypes.byref(opt), op, _dt(outs[0]),
                                                _ptr(workspace), workspace.numel(), sarr,
                                                len(streams), _stream(stream, dev)),
               "ns_orthogonalize_grouped_on")
    return outs
