"""The C-ABI library loads and exports what include/nvfp4ns.h declares;
host-side validation answers without touching a GPU (CPU only)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4ns.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(?:ns_status|size_t)\s+(\w+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = _declared()
    for want in ("nvfp4_quantize", "nvfp4_dequantize", "nvfp4_gemm", "ns_workspace_bytes",
                 "ns_orthogonalize", "ns_orthogonalize_grouped"):
        assert want in names


def test_library_exports_every_declared_symbol():
    ns = pytest.importorskip("newton_schulz_amd")
    lib = ctypes.CDLL(ns.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name
        assert name in ns.EXPORTED, name


def test_workspace_sizes_and_validation_on_host():
    ns = pytest.importorskip("newton_schulz_amd")
    lib = ns._lib
    assert lib.ns_workspace_bytes(3072, 8192) == lib.ns_workspace_bytes(8192, 3072)
    wb = lib.ns_workspace_bytes(3072, 8192)
    # X, A, B in fp32 and four packed NVFP4 tensors (215 MB)
    assert 215e6 < wb < 320e6 and wb % 256 == 0
    assert lib.ns_workspace_bytes(3072, 8190) == 0
    assert lib.nvfp4_quantize_workspace_bytes(16, 16) >= 4
    coeffs = (ctypes.c_float * 3)(3.4445, -4.775, 2.0315)
    fake = ctypes.c_void_p(0x1000)          # never dereferenced: validation fails first
    other = ctypes.c_void_p(0x100000000)
    # null input
    assert lib.ns_orthogonalize(None, 0, 32, 32, coeffs, 1, 1.0, other, 0, fake, wb, None) == ns.NS_ERR_ARG
    # shape not a multiple of 16
    assert lib.ns_orthogonalize(fake, 0, 30, 32, coeffs, 1, 1.0, other, 0, fake, wb, None) == ns.NS_ERR_SHAPE
    # k <= 0, clip <= 0, clip NaN
    assert lib.ns_orthogonalize(fake, 0, 32, 32, coeffs, 0, 1.0, other, 0, fake, wb, None) == ns.NS_ERR_ARG
    assert lib.ns_orthogonalize(fake, 0, 32, 32, coeffs, 1, 0.0, other, 0, fake, wb, None) == ns.NS_ERR_ARG
    assert lib.ns_orthogonalize(fake, 0, 32, 32, coeffs, 1, float("nan"), other, 0, fake, wb, None) == ns.NS_ERR_ARG
    # out overlapping G
    assert lib.ns_orthogonalize(fake, 0, 32, 32, coeffs, 1, 1.0, fake, 0, fake, wb, None) == ns.NS_ERR_ARG
    # workspace too small
    assert lib.ns_orthogonalize(fake, 0, 32, 32, coeffs, 1, 1.0, other, 0, fake, 16, None) == ns.NS_ERR_WORKSPACE
    # quantizer: bad axis, bad shape, no workspace
    assert lib.nvfp4_quantize(fake, 0, 16, 16, 7, fake, fake, fake, fake, 256, None) == ns.NS_ERR_ARG
    assert lib.nvfp4_quantize(fake, 0, 16, 24, 0, fake, fake, fake, fake, 256, None) == ns.NS_ERR_SHAPE
    assert lib.nvfp4_quantize(fake, 0, 16, 16, 0, fake, fake, fake, None, 256, None) == ns.NS_ERR_WORKSPACE
    # symmetric GEMM with different operands
    assert lib.nvfp4_gemm(fake, fake, fake, other, fake, fake, 32, 32, 32, 1, 1.0, 0.0,
                          None, fake, None, None, 0, None) == ns.NS_ERR_ARG
    # beta != 0 without an addend
    assert lib.nvfp4_gemm(fake, fake, fake, fake, fake, fake, 32, 32, 32, 0, 1.0, 2.0,
                          None, fake, None, None, 0, None) == ns.NS_ERR_ARG
    # the 3072^2 x 8192 Gram product has 300 tiles for 8 XCDs of 32 CUs: the
    # tiles left over after one per CU are split along K, which needs a
    # workspace, and a too-small one is refused
    wsg = lib.nvfp4_gemm_workspace_bytes(3072, 3072, 8192, 1)
    assert wsg > 0
    assert lib.nvfp4_gemm(fake, fake, fake, fake, fake, fake, 3072, 3072, 8192, 1, 1.0, 0.0,
                          None, other, None, fake, wsg - 1, None) == ns.NS_ERR_WORKSPACE
    # 3072 x 8192 x 3072 has 1536 tiles, six per CU: nothing is split
    assert lib.nvfp4_gemm_workspace_bytes(3072, 8192, 3072, 0) == 0


# Distinct fake device addresses, 1 TiB apart (never dereferenced: each call
# below fails validation before anything is enqueued).
def _addr(i, off=0):
    return ctypes.c_void_p((i + 1) * (1 << 40) + off)


def test_alignment_and_overlap_are_refused_on_host():
    ns = pytest.importorskip("newton_schulz_amd")
    lib = ns._lib
    qws = lib.nvfp4_quantize_workspace_bytes(64, 64)
    x, codes, scales, sg, ws = (_addr(i) for i in range(5))
    # misaligned input / codes / tensor scale
    assert lib.nvfp4_quantize(_addr(0, 4), 0, 64, 64, 0, codes, scales, sg, ws, qws, None) == ns.NS_ERR_ARG
    assert lib.nvfp4_quantize(x, 0, 64, 64, 0, _addr(1, 8), scales, sg, ws, qws, None) == ns.NS_ERR_ARG
    assert lib.nvfp4_quantize_46(x, 0, 64, 64, 1, codes, scales, _addr(3, 2), ws, qws, None) == ns.NS_ERR_ARG
    # codes inside the input, scales inside the codes, workspace inside the input
    assert lib.nvfp4_quantize(x, 0, 64, 64, 0, _addr(0, 256), scales, sg, ws, qws, None) == ns.NS_ERR_ARG
    assert lib.nvfp4_quantize_rht(x, 0, 64, 64, 0, 0x1234, codes, _addr(1, 64), sg, ws, qws,
                                  None) == ns.NS_ERR_ARG
    assert lib.nvfp4_quantize(x, 0, 64, 64, 0, codes, scales, sg, _addr(0, 1024), qws, None) == ns.NS_ERR_ARG
    # dequantize into its own codes
    assert lib.nvfp4_dequantize(codes, scales, sg, 64, 64, 0, _addr(1, 512), 0, None) == ns.NS_ERR_ARG
    # GEMM: output over an operand, amax word inside the output, misaligned addend
    P, PS, Q, QS, SP, SQ, O = (_addr(i) for i in range(7))
    assert lib.nvfp4_gemm(P, PS, SP, Q, QS, SQ, 64, 64, 256, 0, 1.0, 0.0, None, _addr(2, 4096),
                          None, None, 0, None) == ns.NS_ERR_ARG
    assert lib.nvfp4_gemm(P, PS, SP, Q, QS, SQ, 64, 64, 256, 0, 1.0, 0.0, None, O, _addr(6, 64),
                          None, 0, None) == ns.NS_ERR_ARG
    assert lib.nvfp4_gemm(P, PS, SP, Q, QS, SQ, 64, 64, 256, 0, 1.0, 1.0, _addr(7, 8), O,
                          None, None, 0, None) == ns.NS_ERR_ARG
    # addend partly over the output (equal is allowed, a shifted one is not)
    assert lib.nvfp4_gemm(P, PS, SP, Q, QS, SQ, 64, 64, 256, 0, 1.0, 1.0, _addr(6, 256), O,
                          None, None, 0, None) == ns.NS_ERR_ARG
    # NS: misaligned G, workspace over G
    coeffs = (ctypes.c_float * 3)(3.4445, -4.775, 2.0315)
    nws = lib.ns_workspace_bytes(64, 128)
    assert lib.ns_orthogonalize(_addr(0, 2), 1, 64, 128, coeffs, 1, 1.0, _addr(1), 0, _addr(2), nws,
                                None) == ns.NS_ERR_ARG
    assert lib.ns_orthogonalize(_addr(0), 1, 64, 128, coeffs, 1, 1.0, _addr(1), 0, _addr(0, 4096), nws,
                                None) == ns.NS_ERR_ARG
    # quantile: misaligned output word
    aws = lib.ns_abs_quantile_workspace_bytes()
    assert lib.ns_abs_quantile(_addr(0), 0, 1024, ctypes.c_double(0.99), _addr(1, 1), _addr(2), aws,
                               None) == ns.NS_ERR_ARG


def test_grouped_outputs_must_not_touch_other_problems():
    ns = pytest.importorskip("newton_schulz_amd")
    lib = ns._lib
    coeffs = (ctypes.c_float * 3)(3.4445, -4.775, 2.0315)
    m = (ctypes.c_int64 * 2)(64, 64)
    n = (ctypes.c_int64 * 2)(128, 128)
    clip = (ctypes.c_float * 2)(1.0, 1.0)
    wsb = lib.ns_grouped_workspace_bytes(2, m, n)
    G = (ctypes.c_void_p * 2)(_addr(0).value, _addr(1).value)
    # problem 0 writes over problem 1's input
    out = (ctypes.c_void_p * 2)(_addr(1).value, _addr(3).value)
    assert lib.ns_orthogonalize_grouped(2, G, m, n, 1, coeffs, 1, clip, out, 0, _addr(4), wsb,
                                        None) == ns.NS_ERR_ARG
    # both problems write the same output
    out = (ctypes.c_void_p * 2)(_addr(2).value, _addr(2).value)
    assert lib.ns_orthogonalize_grouped(2, G, m, n, 1, coeffs, 1, clip, out, 0, _addr(4), wsb,
                                        None) == ns.NS_ERR_ARG


def test_grouped_on_stream_list_is_validated_on_host():
    ns = pytest.importorskip("newton_schulz_amd")
    lib = ns._lib
    coeffs = (ctypes.c_float * 3)(3.4445, -4.775, 2.0315)
    m = (ctypes.c_int64 * 2)(64, 64)
    n = (ctypes.c_int64 * 2)(128, 128)
    clip = (ctypes.c_float * 2)(1.0, 1.0)
    wsb = lib.ns_grouped_workspace_bytes(2, m, n)
    G = (ctypes.c_void_p * 2)(_addr(0).value, _addr(1).value)
    out = (ctypes.c_void_p * 2)(_addr(2).value, _addr(3).value)

    def call(streams, count):
        return lib.ns_orthogonalize_grouped_on(2, G, m, n, 1, coeffs, 1, clip, None, out, 0,
                                               _addr(4), wsb, streams, count, None)
    s1 = (ctypes.c_void_p * 1)(_addr(5).value)
    assert call(None, 1) == ns.NS_ERR_ARG                       # no list
    assert call(s1, 0) == ns.NS_ERR_ARG                         # empty list
    s17 = (ctypes.c_void_p * 17)(*[_addr(5).value] * 17)
    assert call(s17, 17) == ns.NS_ERR_ARG                       # more than 16
    s2 = (ctypes.c_void_p * 2)(_addr(5).value, None)
    assert call(s2, 2) == ns.NS_ERR_ARG                         # a NULL stream
    # a valid list reaches the other checks: problem 0 writes over problem 1's input
    bad = (ctypes.c_void_p * 2)(_addr(1).value, _addr(3).value)
    assert lib.ns_orthogonalize_grouped_on(2, G, m, n, 1, coeffs, 1, clip, None, bad, 0, _addr(4),
                                           wsb, s1, 1, None) == ns.NS_ERR_ARG
    # opt = NULL needs the per-matrix clips
    assert lib.ns_orthogonalize_grouped_on(2, G, m, n, 1, coeffs, 1, None, None, out, 0, _addr(4),
                                           wsb, s1, 1, None) == ns.NS_ERR_ARG


def test_empty_shapes_are_refused_on_host():
    """Zero-sized matrices have no NVFP4 blocks: every entry point answers
    NS_ERR_SHAPE without enqueuing anything."""
    ns = pytest.importorskip("newton_schulz_amd")
    lib = ns._lib
    coeffs = (ctypes.c_float * 3)(3.4445, -4.775, 2.0315)
    a, b, c, d, e = (_addr(i) for i in range(5))
    assert lib.ns_workspace_bytes(0, 64) == 0
    assert lib.ns_orthogonalize(a, 0, 0, 64, coeffs, 1, 1.0, b, 0, c, 1 << 20, None) == ns.NS_ERR_SHAPE
    assert lib.ns_orthogonalize(a, 0, 64, 0, coeffs, 1, 1.0, b, 0, c, 1 << 20, None) == ns.NS_ERR_SHAPE
    assert lib.nvfp4_quantize(a, 0, 0, 16, 0, b, c, d, e, 4096, None) == ns.NS_ERR_SHAPE
    assert lib.nvfp4_dequantize(a, b, c, 16, 0, 0, d, 0, None) == ns.NS_ERR_SHAPE
    assert lib.nvfp4_gemm(a, b, c, a, b, c, 0, 0, 32, 1, 1.0, 0.0, None, d, None, None, 0,
                          None) == ns.NS_ERR_SHAPE
    assert lib.nvfp4_gemm_workspace_bytes(16, 16, 0, 0) == 0
    assert lib.ns_abs_quantile(a, 0, 0, ctypes.c_double(0.5), b, c, 1 << 20, None) == ns.NS_ERR_SHAPE
    m = (ctypes.c_int64 * 1)(0)
    n = (ctypes.c_int64 * 1)(64)
    assert lib.ns_grouped_workspace_bytes(1, m, n) == 0


def test_workspace_layout_on_host():
    ns = pytest.importorskip("newton_schulz_amd")
    for m, n in [(3072, 8192), (8192, 3072), (144, 400), (16, 16)]:
        L = ns.ns_workspace_layout(m, n)
        xm, xn = min(m, n), max(m, n)
        assert (L["xm"], L["xn"]) == (xm, xn)
        assert L["total"] == ns.ns_workspace_bytes(m, n)
        # each operand's byte range, in layout order, inside the workspace
        spans = [("x", 4 * xm * xn), ("a", 4 * xm * xm), ("b", 4 * xm * xm),
                 ("qx_codes", xm * xn // 2), ("qx_scales", xm * xn // 16),
                 ("qt_codes", xm * xn // 2), ("qt_scales", xm * xn // 16),
                 ("qa_codes", xm * xm // 2), ("qa_scales", xm * xm // 16),
                 ("qb_codes", xm * xm // 2), ("qb_scales", xm * xm // 16),
                 ("global_scales", 16)]
        end = 0
        for name, size in spans:
            assert L[name] >= end and L[name] % 256 == 0, (m, n, name)
            end = L[name] + size
        assert end <= L["total"]
    with pytest.raises(ns.NSError) as e:
        ns.ns_workspace_layout(30, 32)
    assert e.value.status == ns.NS_ERR_SHAPE
    assert ns._lib.ns_workspace_layout(32, 32, None) == ns.NS_ERR_ARG
