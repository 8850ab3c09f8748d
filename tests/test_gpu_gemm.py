"""Each NVFP4 GEMM of the NS step, fed the oracle's own quantized operands,
against the oracle's float64 result: relative Frobenius error <= 1e-5
(FP32 accumulation of exact products).  Symmetric products must come out
exactly symmetric, and the fused amax must equal max |out|."""
import numpy as np
import pytest
import torch

import synth
from oracle import ns as N
from oracle import nvfp4 as Q

pytestmark = pytest.mark.gpu

import newton_schulz_amd as ns  # noqa: E402
from gpu_util import DEV, host, rel_fro, to_dev_f32  # noqa: E402

TOL = 1e-5
QUINTIC = synth.QUINTIC


def dev_q(q):
    """Oracle NVFP4Tensor -> device (codes, scales, s_g)."""
    return (torch.from_numpy(np.ascontiguousarray(q.codes)).to(DEV),
            torch.from_numpy(np.ascontiguousarray(q.scales)).to(DEV),
            torch.tensor([np.float32(q.global_scale)], dtype=torch.float32, device=DEV))


def _amax_slot():
    return torch.zeros(1, dtype=torch.int32, device=DEV)


def _check_amax(slot, out):
    got = int(host(slot)[0]) & 0xFFFFFFFF
    want = int(np.abs(out.astype(np.float32)).max().view(np.uint32))
    assert got == want


def _gemm_steps(G, coeffs, label):
    trace = []
    N.ns_nvfp4(G, coeffs, trace=trace)
    m, n = trace[0]["X"].shape
    for s, t in enumerate(trace):
        a, b, c = t["coeffs"]
        print(f"[gemm] {label} step {s} m={m} n={n}", flush=True)
        qx, qa, qb, qx16 = dev_q(t["qX"]), dev_q(t["qA"]), dev_q(t["qB"]), dev_q(t["qX16"])
        slot = _amax_slot()
        A = host(ns.nvfp4_gemm(qx, qx, m, m, n, symmetric=True, amax_out=slot))
        assert rel_fro(A, t["A"]) <= TOL, (s, rel_fro(A, t["A"]))
        assert np.array_equal(A, A.T)
        _check_amax(slot, A)
        slot = _amax_slot()
        A32 = to_dev_f32(t["A"])
        B = host(ns.nvfp4_gemm(qa, qa, m, m, m, symmetric=True, alpha=c, beta=b, addend=A32,
                               amax_out=slot))
        assert rel_fro(B, t["B"]) <= TOL, (s, rel_fro(B, t["B"]))
        assert np.array_equal(B, B.T)
        _check_amax(slot, B)
        slot = _amax_slot()
        X32 = to_dev_f32(t["X"])
        Xn = host(ns.nvfp4_gemm(qb, qx16, m, n, m, alpha=1.0, beta=a, addend=X32, out=X32,
                                amax_out=slot))                     # in place, as in NS
        assert rel_fro(Xn, t["X_next"]) <= TOL, (s, rel_fro(Xn, t["X_next"]))
        _check_amax(slot, Xn)


@pytest.mark.parametrize("shape", [(256, 512), (144, 400), (512, 256)])
def test_every_gemm_of_a_quintic_run(shape):
    G = synth.gaussian(*shape, seed=1)
    _gemm_steps(G.astype(np.float64), [QUINTIC] * 5, f"gaussian {shape}")


def test_every_gemm_of_a_clipped_lowrank_run():
    spec = synth.ns_workload("ns2048")
    G, _, clip = synth.ns_matrix(dict(spec, shapes=[(272, 528)]), 0)
    trace_G = N.clip_and_normalize(G, clip)      # the iterate the GEMMs see
    _gemm_steps(trace_G, [QUINTIC, (1.5, -0.5, 0.0)], "lowrank 272x528")


# K % 128 != 0 runs the general kernel, K % 256 == 128 the 128-wide stages,
# K % 256 == 0 the row-line stages; the ragged M and N cut partial tiles
@pytest.mark.parametrize("MNK", [(144, 80, 272), (16, 16, 16), (128, 384, 4096), (200 - 8, 64, 48),
                                 (208, 144, 384), (208, 272, 1152), (208, 144, 512), (304, 528, 1280)])
def test_general_gemm_ragged(MNK):
    M, Nn, K = MNK
    rng = np.random.default_rng(M + Nn + K)
    P = rng.standard_normal((M, K)) * np.exp2(rng.uniform(-3, 3, (M, 1)))
    Qm = rng.standard_normal((Nn, K))
    qp, qq = Q.quantize_rows(P), Q.quantize_rows(Qm)
    want = N.gemm_nt(Q.dequantize_rows(qp), Q.dequantize_rows(qq))
    got = host(ns.nvfp4_gemm(dev_q(qp), dev_q(qq), M, Nn, K))
    assert rel_fro(got, want) <= TOL
    add = rng.standard_normal((M, Nn))
    got2 = host(ns.nvfp4_gemm(dev_q(qp), dev_q(qq), M, Nn, K, alpha=-0.5, beta=2.0,
                              addend=to_dev_f32(add)))
    assert rel_fro(got2, 2.0 * add.astype(np.float32) - 0.5 * want) <= TOL


@pytest.mark.parametrize("M,K", [(144, 272), (400, 96), (208, 640), (336, 768), (528, 1536)])
def test_symmetric_gemm_ragged(M, K):
    rng = np.random.default_rng(M)
    X = rng.standard_normal((M, K))
    q = Q.quantize_rows(X)
    dq = Q.dequantize_rows(q)
    want = N.gemm_nt(dq, dq)
    dq_dev = dev_q(q)                       # one tensor for both operands
    got = host(ns.nvfp4_gemm(dq_dev, dq_dev, M, M, K, symmetric=True))
    assert np.array_equal(got, got.T)
    assert rel_fro(got, want) <= TOL


def test_full_size_gemms_sampled():
    """3072 x 8192 (the benchmark's shape): GEMM1 (3072^2, K=8192, symmetric)
    and GEMM3 (3072 x 8192, K=3072) on 512 sampled outputs each, every one
    computed by the oracle as a float64 dot product of dequantized rows."""
    m, n = 3072, 8192
    rng = np.random.default_rng(4)
    X = rng.standard_normal((m, n)).astype(np.float32)
    print("[gemm] oracle quantize of the 3072x8192 operands", flush=True)
    qx = Q.quantize_rows(X)
    qx16 = Q.quantize_cols(X, amax=Q.tensor_amax(X))
    Bm = rng.standard_normal((m, m)).astype(np.float32)
    Bm = (Bm + Bm.T).astype(np.float32)
    qb = Q.quantize_rows(Bm)
    print("[gemm] full-size GEMM1 / GEMM3 on the GPU", flush=True)
    qx_dev = dev_q(qx)
    A = host(ns.nvfp4_gemm(qx_dev, qx_dev, m, m, n, symmetric=True))
    Xg = host(ns.nvfp4_gemm(dev_q(qb), dev_q(qx16), m, n, m, alpha=1.0, beta=3.4445,
                            addend=to_dev_f32(X)))
    assert np.array_equal(A, A.T)
    ii, jj = rng.integers(0, m, 512), rng.integers(0, m, 512)
    dxi = Q.dequantize_rows(Q.NVFP4Tensor(qx.codes[ii], qx.scales[ii], qx.global_scale, 512, n))
    dxj = Q.dequantize_rows(Q.NVFP4Tensor(qx.codes[jj], qx.scales[jj], qx.global_scale, 512, n))
    want = np.sum(dxi * dxj, axis=1)
    got = A[ii, jj]
    assert np.linalg.norm(got - want) <= TOL * np.linalg.norm(want)
    ii, jj = rng.integers(0, m, 512), rng.integers(0, n, 512)
    dbi = Q.dequantize_rows(Q.NVFP4Tensor(qb.codes[ii], qb.scales[ii], qb.global_scale, 512, m))
    dxc = Q.dequantize_rows(Q.NVFP4Tensor(qx16.codes[jj], qx16.scales[jj], qx16.global_scale, 512, m))
    want = 3.4445 * X[ii, jj].astype(np.float64) + np.sum(dbi * dxc, axis=1)
    got = Xg[ii, jj]
    assert np.linalg.norm(got - want) <= TOL * np.linalg.norm(want)


def _within_fp32_sum_bound(got, exact, absdot, K, extra=0.0):
    """Every entry within the error of a float32 sum of K exact products:
    (K + 2) units of 2^-24 of the sum of the products' magnitudes, plus
    `extra` (the roundings of an addend term)."""
    err = np.abs(got.astype(np.float64) - exact)
    bound = (K + 2) * 2.0 ** -24 * absdot + extra
    bad = err > bound
    assert not bad.any(), f"{np.count_nonzero(bad)} entries outside the bound; worst {np.max(err / (bound + 1e-300)):.3g}x"


def test_full_size_gemms_whole():
    """3072 x 8192 (the benchmark's shape), every output entry: GEMM1 (3072^2,
    K = 8192, symmetric, split tiles summed in the kernel) and GEMM3 (3072 x
    8192, K = 3072, beta X + qB qX16) against float64 products of the
    dequantized operands (the C++ oracle), each entry within the float32
    summation bound of its own terms."""
    from oracle import native as C
    m, n = 3072, 8192
    rng = np.random.default_rng(14)
    X = rng.standard_normal((m, n)).astype(np.float32)
    qx = C.quantize_rows(X)
    qx16 = C.quantize_rows(np.ascontiguousarray(X.T), amax=Q.tensor_amax(X))
    Bm = rng.standard_normal((m, m)).astype(np.float32)
    Bm = (Bm + Bm.T).astype(np.float32)
    qb = C.quantize_rows(Bm)
    print("[gemm] whole GEMM1 / GEMM3 on the GPU", flush=True)
    qx_dev = dev_q(qx)
    A = host(ns.nvfp4_gemm(qx_dev, qx_dev, m, m, n, symmetric=True))
    Xg = host(ns.nvfp4_gemm(dev_q(qb), dev_q(qx16), m, n, m, alpha=1.0, beta=3.4445,
                            addend=to_dev_f32(X)))
    print("[gemm] C++ oracle products", flush=True)
    dx = C.dequantize_rows(qx)
    _within_fp32_sum_bound(A, C.gemm_nt(dx, dx, symmetric=True),
                           C.gemm_nt(np.abs(dx), np.abs(dx), symmetric=True), n)
    del dx, A
    db, dx16 = C.dequantize_rows(qb), C.dequantize_rows(qx16)
    prod = C.gemm_nt(db, dx16)
    absprod = C.gemm_nt(np.abs(db), np.abs(dx16))
    ax = 3.4445 * X.astype(np.float64)
    # the addend term: beta * x rounded once, then the fused add rounds once more
    _within_fp32_sum_bound(Xg, ax + prod, absprod, m, extra=2 * 2.0 ** -24 * (np.abs(ax) + absprod))
    print("[gemm] 3072x8192: every entry of both products within the float32 bound", flush=True)


def test_symmetric_gemm_split_k():
    """A symmetric product with fewer tiles than CUs: its tiles are split
    along K into eight parts whose FP32 partials the last part to finish
    sums in part order inside the product kernel."""
    M, K = 384, 8192
    assert ns.nvfp4_gemm_workspace_bytes(M, M, K, True) > 0       # split schedule
    rng = np.random.default_rng(8)
    X = rng.standard_normal((M, K))
    q = Q.quantize_rows(X)
    dq = Q.dequantize_rows(q)
    want = N.gemm_nt(dq, dq)
    qd = dev_q(q)
    add = rng.standard_normal((M, M))
    add = (add + add.T).astype(np.float32)
    slot = _amax_slot()
    got = host(ns.nvfp4_gemm(qd, qd, M, M, K, symmetric=True, alpha=0.75, beta=-1.5,
                             addend=to_dev_f32(add), amax_out=slot))
    assert np.array_equal(got, got.T)
    assert rel_fro(got, 0.75 * want - 1.5 * add.astype(np.float64)) <= TOL
    _check_amax(slot, got)
    # the same product unsplit (no workspace) agrees to accumulation order
    got1 = host(ns.nvfp4_gemm(qd, qd, M, M, K, symmetric=True, alpha=0.75, beta=-1.5,
                              addend=to_dev_f32(add), split=False))
    assert rel_fro(got1, got) <= 1e-6


@pytest.mark.parametrize("M,NC,sym", [(400, 400, True), (400, 272, False)])
def test_split_k_in_kernel_sum_ragged(M, NC, sym):
    """K = 8192 (32 K-stages): leftover tiles are summed by their last K-part
    inside the product kernel; ragged edge tiles, an addend and the fused
    amax on that path."""
    K = 8192
    assert ns.nvfp4_gemm_workspace_bytes(M, NC, K, sym) > 0
    rng = np.random.default_rng(M + NC)
    P = rng.standard_normal((M, K))
    qp = Q.quantize_rows(P)
    if sym:
        qq = qp
        add = rng.standard_normal((M, M))
        add = (add + add.T).astype(np.float32)
    else:
        qq = Q.quantize_rows(rng.standard_normal((NC, K)))
        add = rng.standard_normal((M, NC)).astype(np.float32)
    want = N.gemm_nt(Q.dequantize_rows(qp), Q.dequantize_rows(qq))
    pd = dev_q(qp)
    qd = pd if sym else dev_q(qq)
    slot = _amax_slot()
    got = host(ns.nvfp4_gemm(pd, qd, M, NC, K, symmetric=sym, alpha=0.5, beta=2.0,
                             addend=to_dev_f32(add), amax_out=slot))
    assert rel_fro(got, 0.5 * want + 2.0 * add.astype(np.float64)) <= TOL
    if sym:
        assert np.array_equal(got, got.T)
    _check_amax(slot, got)


@pytest.mark.parametrize("M,NC,sym", [(384, 384, True), (384, 640, False)])
def test_split_k_reduce_kernel_path(M, NC, sym):
    """K = 2048 (8 K-stages): too short for the in-kernel sum, the K-parts'
    partials go through gemm_reduce_kernel."""
    K = 2048
    assert ns.nvfp4_gemm_workspace_bytes(M, NC, K, sym) > 0
    rng = np.random.default_rng(M + NC + 1)
    qp = Q.quantize_rows(rng.standard_normal((M, K)))
    qq = qp if sym else Q.quantize_rows(rng.standard_normal((NC, K)))
    add = rng.standard_normal((M, NC))
    if sym:
        add = add + add.T
    add = add.astype(np.float32)
    want = N.gemm_nt(Q.dequantize_rows(qp), Q.dequantize_rows(qq))
    pd = dev_q(qp)
    qd = pd if sym else dev_q(qq)
    slot = _amax_slot()
    got = host(ns.nvfp4_gemm(pd, qd, M, NC, K, symmetric=sym, alpha=-1.0, beta=0.25,
                             addend=to_dev_f32(add), amax_out=slot))
    assert rel_fro(got, -want + 0.25 * add.astype(np.float64)) <= TOL
    if sym:
        assert np.array_equal(got, got.T)
    _check_amax(slot, got)


def test_split_k_sums_are_deterministic():
    """3072^2 x 8192 Gram product (the NS step's first product): 44 leftover
    tiles in five K-parts each, summed by the last part inside the product
    kernel.  Which part finishes last varies from launch to launch; the sum
    order does not, so every launch gives the same bits; they also match the
    oracle on sampled entries."""
    m, n = 3072, 8192
    x = synth.gaussian(m, n, seed=23) / np.sqrt(m * n)
    q = Q.quantize_rows(x)
    qd = dev_q(q)
    ws = torch.empty(ns.nvfp4_gemm_workspace_bytes(m, m, n, True), dtype=torch.uint8, device=DEV)
    out = torch.empty((m, m), dtype=torch.float32, device=DEV)
    first = host(ns.nvfp4_gemm(qd, qd, m, m, n, symmetric=True, out=out, workspace=ws)).copy()
    for r in range(12):
        out.fill_(float("nan"))
        got = host(ns.nvfp4_gemm(qd, qd, m, m, n, symmetric=True, out=out, workspace=ws))
        assert np.array_equal(got, first), r
    print("[gemm] 3072^2 x 8192 split-K: 13 launches bit-identical", flush=True)
    rng = np.random.default_rng(3)
    ii, jj = rng.integers(0, m, 256), rng.integers(0, m, 256)
    dq = Q.dequantize_rows(q)
    want = np.sum(dq[ii] * dq[jj], axis=1)
    assert np.linalg.norm(first[ii, jj] - want) <= TOL * np.linalg.norm(want)


def test_split_k_hand_off_reads_this_launchs_partials():
    """The K-parts of a split tile pass FP32 partials to the part that sums
    them through the workspace.  Launches that share the workspace alternate
    between X and D X, D a random diagonal of signs (the sign bit of each
    E2M1 code flipped on the rows where D is -1): the exact products are
    A and D A D, so every partial of a tile that mixes both kinds of rows
    changes sign from one launch to the next, and a part that read a partial
    left by the previous launch would break the bit-exact relation
    out(D X) == D out(X) D."""
    m, n = 3072, 8192
    x = synth.gaussian(m, n, seed=29) / np.sqrt(m * n)
    q = Q.quantize_rows(x)
    d = np.where(np.random.default_rng(5).random(m) < 0.5, -1.0, 1.0).astype(np.float32)
    c1, s1, g1 = dev_q(q)
    flip = torch.from_numpy(np.where(d < 0, 0x88, 0).astype(np.uint8)).to(DEV)
    c2 = torch.bitwise_xor(c1, flip[:, None])
    ws = torch.empty(ns.nvfp4_gemm_workspace_bytes(m, m, n, True), dtype=torch.uint8, device=DEV)
    out = torch.empty((m, m), dtype=torch.float32, device=DEV)
    want1 = host(ns.nvfp4_gemm((c1, s1, g1), (c1, s1, g1), m, m, n, symmetric=True, out=out,
                               workspace=ws)).copy()
    want2 = want1 * d[:, None] * d[None, :]
    assert np.count_nonzero(want2 != want1) > m * m // 4
    for r in range(6):
        for qd, want in (((c2, s1, g1), want2), ((c1, s1, g1), want1)):
            out.fill_(float("nan"))
            got = host(ns.nvfp4_gemm(qd, qd, m, m, n, symmetric=True, out=out, workspace=ws))
            assert np.array_equal(got, want), r
    print("[gemm] 3072^2 x 8192 split-K: 12 alternating launches exact", flush=True)


def test_general_gemm_leftover_tiles_split_k():
    """A non-symmetric product whose tiles do not divide evenly over the CUs:
    the leftover tiles run as K-parts (partials summed in order by the last
    part, 16 K-stages), the rest whole; it matches the oracle and the
    unsplit run."""
    M, NC, K = 384, 640, 4096
    assert ns.nvfp4_gemm_workspace_bytes(M, NC, K, False) > 0
    rng = np.random.default_rng(9)
    P, Qm = rng.standard_normal((M, K)), rng.standard_normal((NC, K))
    qp, qq = Q.quantize_rows(P), Q.quantize_rows(Qm)
    want = N.gemm_nt(Q.dequantize_rows(qp), Q.dequantize_rows(qq))
    add = rng.standard_normal((M, NC)).astype(np.float32)
    slot = _amax_slot()
    got = host(ns.nvfp4_gemm(dev_q(qp), dev_q(qq), M, NC, K, alpha=1.25, beta=0.5,
                             addend=to_dev_f32(add), amax_out=slot))
    assert rel_fro(got, 1.25 * want + 0.5 * add.astype(np.float64)) <= TOL
    _check_amax(slot, got)
    got1 = host(ns.nvfp4_gemm(dev_q(qp), dev_q(qq), M, NC, K, alpha=1.25, beta=0.5,
                              addend=to_dev_f32(add), split=False))
    assert rel_fro(got1, got) <= 1e-6


def test_full_size_gram_update_sampled():
    """B = b A + c qA qA^T at the benchmark's size (3072^2, K = 3072) with the
    quintic's b and c: the launch the NS step makes, whose leftover tiles are
    split into K-parts summed by their last part inside the product kernel.
    512 sampled entries against float64 dot products of dequantized rows;
    the result is exactly symmetric and three launches agree bit for bit."""
    m = 3072
    b, c = -4.775, 2.0315
    assert ns.nvfp4_gemm_workspace_bytes(m, m, m, True) > 0        # split schedule
    rng = np.random.default_rng(12)
    Xs = rng.standard_normal((m, 1024)) / 32.0
    A = (Xs @ Xs.T).astype(np.float32)          # a Gram matrix: large diagonal
    A = np.triu(A) + np.triu(A, 1).T
    qa = Q.quantize_rows(A)
    qd = dev_q(qa)
    Ad = to_dev_f32(A)
    ws = torch.empty(ns.nvfp4_gemm_workspace_bytes(m, m, m, True), dtype=torch.uint8, device=DEV)
    slot = _amax_slot()
    got = host(ns.nvfp4_gemm(qd, qd, m, m, m, symmetric=True, alpha=c, beta=b, addend=Ad,
                             amax_out=slot, workspace=ws)).copy()
    assert np.array_equal(got, got.T)
    _check_amax(slot, got)
    for _ in range(2):
        again = host(ns.nvfp4_gemm(qd, qd, m, m, m, symmetric=True, alpha=c, beta=b, addend=Ad,
                                   workspace=ws))
        assert np.array_equal(again, got)
    ii, jj = rng.integers(0, m, 512), rng.integers(0, m, 512)
    da_i = Q.dequantize_rows(Q.NVFP4Tensor(qa.codes[ii], qa.scales[ii], qa.global_scale, 512, m))
    da_j = Q.dequantize_rows(Q.NVFP4Tensor(qa.codes[jj], qa.scales[jj], qa.global_scale, 512, m))
    want = b * A[ii, jj].astype(np.float64) + c * np.sum(da_i * da_j, axis=1)
    err = np.linalg.norm(got[ii, jj] - want) / np.linalg.norm(want)
    print(f"[gemm] 3072^2 x 3072 quintic update: sampled rel {err:.3g}", flush=True)
    assert err <= TOL
