"""Seeded random sweep against the oracle: shapes (multiples of 16, ragged
against every tile size), value distributions, input types and axes that
the fixed-shape tests do not name.  The same bars as there: the quantizer
bit for bit (codes, scales, s_g, dequantized values), each product within
1e-5 relative Frobenius error of the float64 product of the dequantized
operands and every entry within the float32 summation bound of its own
terms, NS (a stable schedule) within 2e-2 and the singular-value band."""
import numpy as np
import pytest

import synth
from oracle import ns as N
from oracle import nvfp4 as Q

pytestmark = pytest.mark.gpu

import newton_schulz_amd as ns  # noqa: E402
from gpu_util import host, rel_fro, same_band, to_dev_bf16, to_dev_f32  # noqa: E402
from test_gpu_quant import _check_dequant, _check_quant, _device_input  # noqa: E402

CUBIC = (1.5, -0.5, 0.0)


def _values(rng, rows, cols):
    """One of several value models, chosen by the case's generator."""
    kind = int(rng.integers(0, 5))
    if kind == 0:
        x = rng.standard_normal((rows, cols)) * 10.0 ** rng.uniform(-6, 3)
    elif kind == 1:
        x = rng.standard_t(3, size=(rows, cols)) * 0.02
        idx = rng.random((rows, cols)) < 0.001
        x[idx] *= 50.0
    elif kind == 2:
        # blocks whose scales span 2^-30 .. 1 of the tensor maximum
        x = rng.standard_normal((rows, cols))
        x *= np.exp2(rng.uniform(-30, 0, size=(rows, cols // 16))).repeat(16, axis=1)
    elif kind == 3:
        # sparse: most entries zero, the rest uniform
        x = rng.uniform(-1, 1, (rows, cols)) * (rng.random((rows, cols)) < 0.1)
    else:
        # constant blocks and exact small integers
        x = rng.integers(-8, 9, size=(rows, cols // 16)).repeat(16, axis=1).astype(np.float64)
    return x.astype(np.float32), kind


def _dim(rng, lo, hi):
    return 16 * int(rng.integers(lo // 16, hi // 16 + 1))


@pytest.mark.parametrize("case", range(64))
def test_quantizer_random_cases(case):
    rng = np.random.default_rng(1000 + case)
    hi = 2048 if case % 8 == 0 else 768
    rows, cols = _dim(rng, 16, hi), _dim(rng, 16, hi)
    dtype = ["f32", "bf16"][int(rng.integers(0, 2))]
    axis = ["rows", "cols"][int(rng.integers(0, 2))]
    x, kind = _values(rng, rows, cols)
    xd, vals = _device_input(x, dtype)
    label = f"case {case} kind {kind} {dtype}"
    codes, scales, sg, oq = _check_quant(vals, xd, axis, label)
    _check_dequant(codes, scales, sg, oq, rows, cols, axis, label)


def _dev_q(q):
    import torch
    return (torch.from_numpy(np.ascontiguousarray(q.codes)).to("cuda"),
            torch.from_numpy(np.ascontiguousarray(q.scales)).to("cuda"),
            torch.tensor([np.float32(q.global_scale)], dtype=torch.float32, device="cuda"))


@pytest.mark.parametrize("case", range(40))
def test_gemm_random_cases(case):
    rng = np.random.default_rng(2000 + case)
    sym = bool(rng.integers(0, 2))
    M = _dim(rng, 16, 640)
    Nn = M if sym else _dim(rng, 16, 640)
    # K: multiples of 256 (row-line stages), of 128 only, and of 16 only
    K = [_dim(rng, 256, 4096) // 256 * 256 or 256, 128 * (2 * int(rng.integers(1, 16)) + 1),
         _dim(rng, 16, 2048)][case % 3]
    alpha = float(rng.uniform(-3, 3))
    beta = float(rng.uniform(-3, 3)) if rng.integers(0, 2) else 0.0
    P = rng.standard_normal((M, K))
    qp = Q.quantize_rows(P)
    qq = qp if sym else Q.quantize_rows(rng.standard_normal((Nn, K)))
    add = rng.standard_normal((M, Nn))
    if sym:
        add = add + add.T
    add = add.astype(np.float32)
    print(f"[gemm] case {case} M={M} N={Nn} K={K} sym={sym} alpha={alpha:.3f} beta={beta:.3f}",
          flush=True)
    pd = _dev_q(qp)
    qd = pd if sym else _dev_q(qq)
    got = host(ns.nvfp4_gemm(pd, qd, M, Nn, K, symmetric=sym, alpha=alpha, beta=beta,
                             addend=to_dev_f32(add) if beta != 0.0 else None))
    dp, dq = Q.dequantize_rows(qp), Q.dequantize_rows(qq)
    prod = alpha * N.gemm_nt(dp, dq)
    absprod = abs(alpha) * N.gemm_nt(np.abs(dp), np.abs(dq))
    u = 2.0 ** -24
    want, bound = prod, (K + 2) * u * absprod
    if beta != 0.0:
        badd = beta * add.astype(np.float64)
        want = want + badd
        bound = bound + 2 * u * (np.abs(badd) + absprod)
    assert rel_fro(got, want) <= 1e-5
    # every entry within the float32 summation bound of its own terms
    err = np.abs(got.astype(np.float64) - want)
    assert (err <= bound).all(), float(np.max(err / np.maximum(bound, 1e-300)))
    if sym:
        assert np.array_equal(got, got.T)


@pytest.mark.parametrize("case", range(12))
def test_ns_random_cases(case):
    rng = np.random.default_rng(3000 + case)
    m, n = _dim(rng, 16, 512), _dim(rng, 16, 512)
    G = rng.standard_normal((m, n)).astype(np.float32)
    clip = float(np.float32(rng.uniform(1.5, 4.0) * np.sqrt(np.mean(G.astype(np.float64) ** 2))))
    bf16 = bool(rng.integers(0, 2))
    if bf16:
        bits, G = synth.to_bf16(G)
        Gd = to_dev_bf16(bits)
    else:
        Gd = to_dev_f32(G)
    coeffs = [CUBIC] * 4
    print(f"[ns] case {case} {m}x{n} bf16={bf16} clip={clip:.3f}", flush=True)
    got = host(ns.ns_orthogonalize(Gd, coeffs, clip)).astype(np.float64)
    want = N.ns_nvfp4(G.astype(np.float64), coeffs, clip=clip)
    assert rel_fro(got, want) <= 2e-2
    assert same_band(got, want)
