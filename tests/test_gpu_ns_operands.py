"""The quantize passes that ns_orthogonalize runs inside its iteration,
checked byte for byte: after a call, the workspace holds the last step's
input iterate X (untransposed calls with FP32 output write the last product
straight into `out`), the upper triangles of A and B, every quantized
operand of that step and the tensor scales (ns_workspace_layout).  The
oracle quantizer applied to the GPU's own X, A and B must give the same
codes, scale bytes and s_g (the format rules of §2 "NVFP4 format", RTN as in
§3.4).  This covers

  * the first step's pass that normalises G and quantizes X_0 both ways
    (quant_tile_kernel<..., NORM>),
  * the two-layout pass of later steps and of transposed calls,
  * the symmetric pass that quantizes A and B from their upper triangles
    (row blocks of tiles above the diagonal come from the column blocks of
    the mirrored tile),

and, on the same operands, each product of the step against float64
(relative Frobenius 1e-5): A = qX qX^T, B = b A + c qA qA^T with the
quintic's c != 0, and X' = a X + qB qX16.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import ns as N
from oracle import nvfp4 as Q

pytestmark = pytest.mark.gpu

import newton_schulz_amd as ns  # noqa: E402
from gpu_util import host, rel_fro, to_dev_bf16, to_dev_f32  # noqa: E402

QUINTIC = synth.QUINTIC
CUBIC = (1.5, -0.5, 0.0)
GEMM_TOL = 1e-5


def _run(Gd, coeffs, clip, adaptive46=False, rht_masks=None):
    """One NS call with FP32 output; returns (out, workspace views as host
    arrays)."""
    m, n = Gd.shape
    ws = torch.empty(ns.ns_workspace_bytes(m, n), dtype=torch.uint8, device=Gd.device)
    out = ns.ns_orthogonalize_ex(Gd, coeffs, clip=clip, adaptive46=adaptive46, rht_masks=rht_masks,
                                 workspace=ws)
    v = ns.ns_workspace_views(ws, m, n)
    torch.cuda.synchronize()
    h = {k: (host(t) if not isinstance(t, tuple) else tuple(x.cpu().numpy() for x in t))
         for k, t in v.items()}
    return host(out), h


def _sym(upper):
    """The symmetric matrix whose upper triangle (with the diagonal) is that
    of `upper` (the GPU stores only row <= col)."""
    u = np.triu(upper.astype(np.float64))
    return u + np.triu(u, 1).T


def _same(got, want, label):
    codes, scales = got
    assert codes.shape == want.codes.shape, label
    nc = int(np.count_nonzero(codes != want.codes))
    ns_ = int(np.count_nonzero(scales != want.scales))
    print(f"[operands] {label}: {nc} code bytes, {ns_} scale bytes differ "
          f"of {codes.size} / {scales.size}", flush=True)
    assert nc == 0 and ns_ == 0, label


def _sg_equal(got, want, label):
    assert np.float32(got).view(np.uint32) == np.float32(want).view(np.uint32), (label, got, want)


def _check_step(X, h, coeffs_last, adaptive46, rows=None, cols=None, label=""):
    """h holds the workspace after the call; X is the input iterate of its
    last step (float32, xm x xn).  rows / cols: None (whole tensors) or
    sampled row indices of X, A, B and sampled column indices of X."""
    a, b, c = coeffs_last
    xm, xn = X.shape
    X64 = X.astype(np.float64)
    amax_x = Q.tensor_amax(X64)
    rsel = slice(None) if rows is None else rows
    csel = slice(None) if cols is None else cols
    # qX = Q_1x16(X) and qX16 = Q_16x1(X), one s_g
    qx = Q.quantize_rows(X64[rsel], amax=amax_x, adaptive46=adaptive46)
    _same((h["qX"][0][rsel], h["qX"][1][rsel]), qx, f"{label} qX")
    qt = Q.quantize_rows(X64.T[csel], amax=amax_x, adaptive46=adaptive46)
    _same((h["qX16"][0][csel], h["qX16"][1][csel]), qt, f"{label} qX16")
    _sg_equal(h["sg"][0], Q.global_scale(amax_x), f"{label} s_g(X)")
    # A: upper triangle stored; the oracle quantizer on the GPU's own A
    A = _sym(h["A"])
    amax_a = Q.tensor_amax(A)
    qa = Q.quantize_rows(A[rsel], amax=amax_a, adaptive46=adaptive46)
    _same((h["qA"][0][rsel], h["qA"][1][rsel]), qa, f"{label} qA")
    _sg_equal(h["sg"][1], Q.global_scale(amax_a), f"{label} s_g(A)")
    B = _sym(h["B"])
    amax_b = Q.tensor_amax(B)
    qb = Q.quantize_rows(B[rsel], amax=amax_b, adaptive46=adaptive46)
    _same((h["qB"][0][rsel], h["qB"][1][rsel]), qb, f"{label} qB")
    _sg_equal(h["sg"][2], Q.global_scale(amax_b), f"{label} s_g(B)")
    # the products of the step on these operands, float64
    if rows is None:
        dx = Q.dequantize_rows(qx)
        A_want = N.gemm_nt(dx, dx)
        qa_full = qa
        B_want = b * A + c * N.gemm_nt(Q.dequantize_rows(qa_full), Q.dequantize_rows(qa_full))
        err_a, err_b = rel_fro(A, A_want), rel_fro(B, B_want)
    else:
        # sampled entries (i, j): float64 dot products of the dequantized rows
        rng = np.random.default_rng(11)
        i, j = rng.choice(rows, 256), rng.integers(0, xm, 256)
        qx_i = Q.quantize_rows(X64[i], amax=amax_x, adaptive46=adaptive46)
        qx_j = Q.quantize_rows(X64[j], amax=amax_x, adaptive46=adaptive46)
        want = np.sum(Q.dequantize_rows(qx_i) * Q.dequantize_rows(qx_j), axis=1)
        err_a = float(np.linalg.norm(A[i, j] - want) / np.linalg.norm(want))
        qa_i = Q.quantize_rows(A[i], amax=amax_a, adaptive46=adaptive46)
        qa_j = Q.quantize_rows(A[j], amax=amax_a, adaptive46=adaptive46)
        want = b * A[i, j] + c * np.sum(Q.dequantize_rows(qa_i) * Q.dequantize_rows(qa_j), axis=1)
        err_b = float(np.linalg.norm(B[i, j] - want) / np.linalg.norm(want))
    print(f"[operands] {label}: A rel {err_a:.3g}, B rel {err_b:.3g}", flush=True)
    assert err_a <= GEMM_TOL and err_b <= GEMM_TOL, (label, err_a, err_b)
    return qx, qt, qb


@pytest.mark.parametrize("adaptive46", [False, True])
@pytest.mark.parametrize("case", ["gauss256x512", "ragged144x400", "lowrank272x528_clip"])
def test_first_step_operands_bit_exact(case, adaptive46):
    """k = 1, untransposed, FP32 output: the workspace X is X_0 written by the
    fused normalise + quantize pass; every operand of the step is checked
    whole, and the update product against float64 from the GPU's qB, qX16."""
    if case == "gauss256x512":
        G = synth.gaussian(256, 512, seed=1)
        Gd, clip = to_dev_f32(G), np.inf
    elif case == "ragged144x400":
        G = synth.gaussian(144, 400, seed=5) * 3.0
        Gd, clip = to_dev_f32(G), 2.5
    else:
        G, bits, clip = synth.ns_matrix(dict(synth.ns_workload("ns2048"), shapes=[(272, 528)]), 0)
        Gd = to_dev_bf16(bits)
    out, h = _run(Gd, [QUINTIC], clip, adaptive46=adaptive46)
    X0 = h["X"]
    # X_0 itself: the float32 rounding of the normalised clamp (a different
    # summation order of the norm: a few float32 ulps at most)
    want0 = N.clip_and_normalize(G.astype(np.float64), clip)
    assert np.max(np.abs(X0 - want0)) <= 4 * np.finfo(np.float32).eps * np.max(np.abs(want0))
    qx, qt, qb = _check_step(X0, h, QUINTIC, adaptive46, label=f"{case} 46={adaptive46} step 1")
    a = QUINTIC[0]
    want = a * X0.astype(np.float64) + N.gemm_nt(Q.dequantize_rows(qb), Q.dequantize_rows(qt))
    err = rel_fro(out, want)
    print(f"[operands] {case}: X' rel {err:.3g}", flush=True)
    assert err <= GEMM_TOL


@pytest.mark.parametrize("shape,seed", [((256, 512), 2), ((400, 144), 3), ((208, 80), 4)])
def test_later_step_operands_bit_exact(shape, seed):
    """Step 2 (the two-layout pass on an FP32 iterate, and the symmetric
    pass again), also for transposed calls: X_1 comes from a one-step call
    (every call is deterministic), the operands from a two-step call."""
    G = synth.gaussian(*shape, seed=seed)
    Gd = to_dev_f32(G)
    coeffs = [QUINTIC, (3.0, -3.2, 1.2)]
    m, n = shape
    if m <= n:
        X1 = host(ns.ns_orthogonalize(Gd, coeffs[:1]))    # the one-step call's output
    else:
        _, h1 = _run(Gd, coeffs[:1], np.inf)
        X1 = h1["X"]                  # transposed calls keep X_k (iterate layout)
    _, h2 = _run(Gd, coeffs, np.inf)
    _check_step(X1.astype(np.float32), h2, coeffs[1], False, label=f"{shape} step 2")


def test_rht_operands_bit_exact():
    """With the Hadamard transform: qX = Q_1x16(X H) and qX16 = Q_16x1(H^T X)
    with separate tensor scales, qA = Q_1x16(A H), qB = Q_1x16(B H), all from
    the same FP32 butterfly as the standalone transformed quantizer."""
    from oracle.rht import rht_rows_f32
    G = synth.gaussian(144, 400, seed=9)
    masks = [0xA5C3]
    _, h = _run(to_dev_f32(G), [QUINTIC], np.inf, rht_masks=masks)

    def q(t):      # Q_1x16 of the FP32 butterfly transform of t's row blocks
        return Q.quantize_rows(rht_rows_f32(t, masks[0]).astype(np.float64))
    X0 = h["X"]                       # X_0 (the last product wrote `out`)
    qx, qt = q(X0), q(X0.T)           # Q_16x1(H^T X) is stored as rows of X^T H
    _same(h["qX"], qx, "rht qX")
    _same(h["qX16"], qt, "rht qX16")
    _sg_equal(h["sg"][0], qx.global_scale, "rht s_g(XH)")
    _sg_equal(h["sg"][3], qt.global_scale, "rht s_g(H^T X)")
    A = _sym(h["A"])                  # upper triangle stored, as without the transform
    qa = q(A)
    _same(h["qA"], qa, "rht qA")
    _sg_equal(h["sg"][1], qa.global_scale, "rht s_g(AH)")
    B = _sym(h["B"])
    qb = q(B)
    _same(h["qB"], qb, "rht qB")
    _sg_equal(h["sg"][2], qb.global_scale, "rht s_g(BH)")


@pytest.mark.parametrize("case,adaptive46", [("gauss256x512", False), ("gauss512x256", False),
                                             ("gauss256x512", True), ("gauss512x256", True),
                                             ("full3072x8192", False)])
def test_rht_fused_maxima_operands(case, adaptive46):
    """The transform on shapes whose three products run 128 x 128 row-line
    tiles: the maxima behind the last step's tensor scales are folded into
    the epilogues of the products that wrote X (the previous step's update
    product, under this step's transform), A and B (the Gram products; at
    3072 their split tiles are summed in the product kernel first).  Every
    s_g equals the oracle's on the GPU's own tensors and the codes of all
    rows (sampled rows at full size) match byte for byte; with adaptive 4/6
    too (the pages' route)."""
    from oracle.rht import rht_rows_f32
    if case == "full3072x8192":
        G, bits, clip = synth.ns_matrix(synth.ns_workload("ns3072x8192"), 0)
        Gd, k = to_dev_bf16(bits), 2
    else:
        m, n = (256, 512) if case == "gauss256x512" else (512, 256)
        G, clip, k = synth.gaussian(m, n, seed=21), np.inf, 3
        Gd = to_dev_f32(G)
    masks = [0xA5C3, 0x3C5A, 0x0FF1][:k]
    coeffs = [QUINTIC] * k
    print(f"[operands] rht {case} k={k}: GPU calls", flush=True)
    _, h = _run(Gd, coeffs, clip, adaptive46=adaptive46, rht_masks=masks)
    m, n = Gd.shape
    if m <= n:
        X = h["X"]                    # X_{k-1}: the last product wrote `out`
    else:                             # transposed calls keep X_k; X_{k-1} from k - 1 steps
        X = host(ns.ns_orthogonalize_ex(Gd, coeffs[:k - 1], clip=clip, rht_masks=masks[:k - 1],
                                        adaptive46=adaptive46)).T
    X = np.ascontiguousarray(X, dtype=np.float32)
    A, B = _sym(h["A"]), _sym(h["B"])
    mk = masks[-1]
    xm, xn = X.shape
    if case == "full3072x8192":
        rng = np.random.default_rng(31)
        rows = np.unique(np.concatenate([rng.integers(0, xm, 24), [0, 127, 128, 3071]]))
        cols = np.unique(np.concatenate([rng.integers(0, xn, 24), [0, 8191]]))
    else:
        rows, cols = np.arange(xm), np.arange(xn)
    print(f"[operands] rht {case}: oracle", flush=True)
    for label, t, got, sg_i, sel in (("qX", X, h["qX"], 0, rows), ("qX16", X.T, h["qX16"], 3, cols),
                                     ("qA", A, h["qA"], 1, rows), ("qB", B, h["qB"], 2, rows)):
        th = rht_rows_f32(t, mk).astype(np.float64)
        amax = Q.tensor_amax(th)
        _sg_equal(h["sg"][sg_i], Q.global_scale(amax), f"rht {case} s_g of {label}")
        want = Q.quantize_rows(th[sel], amax=amax, adaptive46=adaptive46)
        _same((got[0][sel], got[1][sel]), want, f"rht {case} a46={adaptive46} {label}")


@pytest.mark.parametrize("k", [1, 2])
def test_full_size_operands_sampled_rows(k):
    """3072 x 8192 BF16 gradient, the benchmark's call: sampled rows of every
    operand (each row of qA and qB crosses tiles above, on and below the
    diagonal), byte for byte; A and B (B with the quintic's c != 0, so the
    3072^2 x 3072 product and its in-kernel split-K sum count) on sampled
    entries against float64."""
    spec = synth.ns_workload("ns3072x8192")
    G, bits, clip = synth.ns_matrix(spec, 0)
    Gd = to_dev_bf16(bits)
    coeffs = [QUINTIC] * k
    print(f"[operands] 3072x8192 k={k}: GPU calls", flush=True)
    _, h = _run(Gd, coeffs, clip)
    if k == 1:
        X = h["X"]
    else:
        X = host(ns.ns_orthogonalize(Gd, coeffs[:k - 1], clip))
    rng = np.random.default_rng(100 + k)
    rows = np.unique(np.concatenate([rng.integers(0, 3072, 40), [0, 127, 128, 255, 1536, 3071]]))
    cols = np.unique(np.concatenate([rng.integers(0, 8192, 40), [0, 63, 64, 4095, 8191]]))
    print(f"[operands] 3072x8192 k={k}: oracle on {rows.size} rows, {cols.size} columns", flush=True)
    _check_step(X.astype(np.float32), h, QUINTIC, False, rows=rows, cols=cols,
                label=f"3072x8192 step {k}")
