"""Pins for the C++ oracle (oracle/cpp/nvfp4_oracle.cpp via oracle.native),
CPU only: the hand-worked golden example, the hand E2M1 table, exactly
representable round trips, brute-force round-to-nearest in exact rationals,
idempotence, the per-block error bound, special tensors, its GEMM against a
triple loop and its NS against the scalar map on benign inputs; and, as a
second check, agreement with the independently written numpy oracle."""
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats as F
from oracle import native as C
from oracle import ns as N
from oracle import nvfp4 as Q

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
QUINTIC = (3.4445, -4.7750, 2.0315)
CUBIC = (1.5, -0.5, 0.0)


def _read_worked():
    d = {}
    for line in open(os.path.join(GOLDEN, "nvfp4_worked_2x32.txt")):
        if line.strip() and not line.startswith("#"):
            k, *v = line.split()
            d[k] = v
    return d


def test_hand_worked_example():
    d = _read_worked()
    t = np.array([[float(v) for v in d["row0"]], [float(v) for v in d["row1"]]], dtype=np.float32)
    q = C.quantize_rows(t)
    assert float(q.global_scale) == float(d["sg"][0])
    for r in range(2):
        assert q.scales[r].tolist() == [int(x, 16) for x in d[f"scales{r}"]]
        assert q.codes[r].tolist() == [int(x, 16) for x in d[f"codes{r}"]]
    deq = C.dequantize_rows(q)
    for r in range(2):
        want = np.array([float(v) for v in d[f"deq{r}"]])
        assert np.array_equal(deq[r], want) and np.array_equal(np.signbit(deq[r]), np.signbit(want))


def test_e2m1_values_against_hand_table():
    # codes 0..15 under scale byte 0x38 (= 1.0) and s_g = 1 decode to the
    # E2M1 values themselves
    table = {}
    for line in open(os.path.join(GOLDEN, "e2m1_values.txt")):
        if line.strip() and not line.startswith("#"):
            code, value = line.split()[:2]
            table[int(code, 16)] = float(value)
    codes = np.arange(16, dtype=np.uint8)
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8).reshape(1, 8)
    q = Q.NVFP4Tensor(packed, np.array([[0x38]], np.uint8), np.float32(1.0), 1, 16)
    deq = C.dequantize_rows(q)[0]
    for c in range(16):
        assert deq[c] == table[c] and np.signbit(deq[c]) == (c >= 8)


def _representable(rng, rows, cols, e_sg):
    nb = cols // 16
    scale_bytes = rng.integers(0x08, 0x7F, size=(rows, nb))
    scale_bytes[rng.integers(rows), rng.integers(nb)] = 0x7E
    codes = rng.integers(0, 16, size=(rows, cols))
    for r in range(rows):
        for b in range(nb):
            codes[r, 16 * b + rng.integers(16)] = rng.choice([7, 15])
    s = np.repeat(F.e4m3fn_decode(scale_bytes), 16, axis=1)
    return F.e2m1_decode(codes) * s * 2.0 ** e_sg, codes, scale_bytes


@pytest.mark.parametrize("e_sg", [-7, -20, 3])
def test_exactly_representable_round_trip(e_sg):
    rng = np.random.default_rng(200 + e_sg)
    t, codes, scale_bytes = _representable(rng, 8, 64, e_sg)
    q = C.quantize_rows(t.astype(np.float32))
    assert float(q.global_scale) == 2.0 ** e_sg
    assert np.array_equal(q.scales, scale_bytes.astype(np.uint8))
    assert np.array_equal(q.codes, (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8))
    deq = C.dequantize_rows(q)
    assert np.array_equal(deq, t) and np.array_equal(np.signbit(deq), np.signbit(t))


def _nearest(q, grid):
    """Index of the grid value nearest to the rational q (ties: even index;
    above the grid: the last)."""
    best = None
    for i, g in enumerate(grid):
        d = abs(q - g)
        if best is None or d < best[0] or (d == best[0] and i % 2 == 0):
            best = (d, i)
    return best[1]


def test_round_to_nearest_brute_force():
    # blocks built around exact midpoints of both grids, and random ones;
    # every scale byte and element code against a nearest-grid search in
    # exact rationals (ties to the even code)
    rng = np.random.default_rng(7)
    e4m3 = [Fraction(float(v)) for v in F.e4m3fn_decode(np.arange(127))]
    e2m1 = [Fraction(float(v)) for v in F.E2M1_MAGNITUDES]
    sg = np.float32(2.0 ** -5)
    rows = []
    for trial in range(24):
        blk = rng.standard_normal(16) * np.exp2(rng.integers(-9, 5))
        if trial % 3 == 0:          # element ties at E2M1 midpoints times the block's unit
            blk[:7] = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]) * np.exp2(rng.integers(-8, 2))
        if trial % 4 == 1:          # block maximum on an E4M3 midpoint times 6 s_g
            j = rng.integers(0, 126)
            blk[0] = float((e4m3[j] + e4m3[j + 1]) / 2 * 6 * Fraction(float(sg)))
        rows.append(blk)
    x = np.array(rows).reshape(1, -1)
    amax = float(2688 * sg)               # fixes s_g = 2^-5 for every block
    q = C.quantize_rows(x, amax=amax)
    assert float(q.global_scale) == float(sg)
    for b in range(x.shape[1] // 16):
        v = x[0, 16 * b:16 * b + 16]
        amax_b = Fraction(float(np.abs(v).max()))
        s_code = _nearest(amax_b / (6 * Fraction(float(sg))), e4m3)
        assert q.scales[0, b] == s_code, b
        unit = e4m3[s_code] * Fraction(float(sg))
        for i in range(16):
            want = 0 if unit == 0 else _nearest(Fraction(float(abs(v[i]))) / unit, e2m1)
            byte = q.codes[0, (16 * b + i) // 2]
            got = (byte >> 4) if i % 2 else (byte & 15)
            assert got & 7 == want and (got >> 3) == int(np.signbit(v[i])), (b, i)


def test_idempotent_with_normal_scales():
    rng = np.random.default_rng(8)
    for _ in range(10):
        x = rng.standard_normal((16, 128)) * np.exp2(rng.uniform(-8, 8))
        blocks = x.reshape(16, 8, 16)
        bm = np.abs(blocks).max(axis=2, keepdims=True)
        blocks *= np.where(bm < np.abs(x).max() / 20000, np.abs(x).max() / 20000 / bm, 1.0)
        q1 = C.quantize_rows(x.astype(np.float32))
        q2 = C.quantize_rows(C.dequantize_rows(q1))
        assert q2.global_scale == q1.global_scale
        assert np.array_equal(q2.scales, q1.scales) and np.array_equal(q2.codes, q1.codes)


def test_per_block_error_bound():
    rng = np.random.default_rng(9)
    x = (rng.standard_t(3, size=(64, 256)) * 0.02).astype(np.float32)
    q = C.quantize_rows(x)
    deq = C.dequantize_rows(q)
    unit = np.repeat(F.e4m3fn_decode(q.scales), 16, axis=1) * float(q.global_scale)
    err = np.abs(deq - x.astype(np.float64))
    quot = np.abs(x.astype(np.float64)) / np.where(unit > 0, unit, 1)
    gap = np.where(quot < 2, 0.5, np.where(quot < 4, 1.0, 2.0))
    ok = (unit > 0) & (quot <= 6)
    assert np.all(err[ok] <= 0.5 * gap[ok] * unit[ok])


def test_zero_nan_inf_tensors():
    z = np.zeros((2, 32), np.float32)
    z[1, 3] = -0.0
    q = C.quantize_rows(z)
    assert float(q.global_scale) == 0.0 and not q.scales.any()
    assert q.codes[1, 1] == 0x80          # element 3: high nibble of byte 1, sign kept
    for bad in (np.nan, np.inf, -np.inf):
        t = np.ones((2, 32), np.float32)
        t[0, 5] = bad
        q = C.quantize_rows(t)
        assert np.isnan(q.global_scale) and np.all(q.scales == 0x7F)
        assert np.all(q.codes & 0x77 == 0)
        assert np.all(np.isnan(C.dequantize_rows(q)))


def test_gemm_against_triple_loop():
    rng = np.random.default_rng(10)
    P = rng.integers(-6, 7, size=(37, 48)) * 0.5
    Qm = rng.integers(-6, 7, size=(21, 48)) * 0.25
    Cm = C.gemm_nt(P, Qm)
    for i in range(37):
        for j in range(21):
            assert Cm[i, j] == sum(P[i, k] * Qm[j, k] for k in range(48))
    S = C.gemm_nt(P, None, symmetric=True)
    assert np.array_equal(S, S.T)
    assert np.array_equal(S, C.gemm_nt(P, P))    # small dyadic values: exact either way


def _equal_magnitude_rows(m, n, rng):
    H = np.array([[1.0]])
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    M = H[rng.permutation(n)[:m]][:, rng.permutation(n)]
    return M * rng.choice([-1.0, 1.0], size=n)


@pytest.mark.parametrize("abc", [QUINTIC, (3.0, -3.2, 1.2), (0.5, 2.0, -1.25)])
def test_ns_step_follows_scalar_map_when_benign(abc):
    rng = np.random.default_rng(11)
    M = _equal_magnitude_rows(16, 64, rng)
    a, b, c = abc
    for s in (0.125, 0.7, 1.3):
        X = M * (s / 8.0)                    # every singular value s
        got = C.ns_nvfp4_step(X, a, b, c)
        assert np.linalg.norm(got - (a + b * s ** 2 + c * s ** 4) * X) <= 1e-5 * np.linalg.norm(X)


def test_ns_orientation_and_scalar_map():
    rng = np.random.default_rng(12)
    M = _equal_magnitude_rows(16, 32, rng)
    coeffs = [QUINTIC, CUBIC, (3.0, -3.2, 1.2)]
    s = 0.25                                  # X_0 = M / ||M|| has singular values 1/4
    for G in (M, M.T):
        X = C.ns_nvfp4(G, coeffs)
        sv = s
        for a, b, c in coeffs:
            sv = a * sv + b * sv ** 3 + c * sv ** 5
        assert np.linalg.norm(X - (sv / s) * G / np.linalg.norm(G)) <= 1e-5 * np.linalg.norm(X)


# ---- agreement with the numpy oracle ---------------------------------------

@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_quantizer_agrees_with_numpy_oracle(dtype):
    rng = np.random.default_rng(13)
    x = (rng.standard_t(3, size=(96, 160)) * 0.02)
    x.reshape(-1)[rng.choice(x.size, 20, replace=False)] *= 50
    x = x.astype(dtype)
    for amax in (None, float(np.abs(x).max()) * 4):
        a, b = C.quantize_rows(x, amax=amax), Q.quantize_rows(x, amax=amax)
        assert np.float32(a.global_scale) == np.float32(b.global_scale)
        assert np.array_equal(a.scales, b.scales) and np.array_equal(a.codes, b.codes)
        assert np.array_equal(C.dequantize_rows(a), Q.dequantize_rows(b))


@pytest.mark.parametrize("shape,coeffs", [((64, 128), [CUBIC] * 5), ((128, 64), [QUINTIC] * 2),
                                          ((48, 48), [QUINTIC, CUBIC, CUBIC])])
def test_ns_agrees_with_numpy_oracle(shape, coeffs):
    rng = np.random.default_rng(sum(shape))
    G = rng.standard_normal(shape)
    a, b = C.ns_nvfp4(G, coeffs, clip=2.5), N.ns_nvfp4(G, coeffs, clip=2.5)
    # two float64 implementations: summation orders differ in the last bits
    assert np.linalg.norm(a - b) <= 1e-10 * np.linalg.norm(b)


def test_ns_step_agrees_with_numpy_oracle():
    rng = np.random.default_rng(14)
    X = rng.standard_normal((80, 144)) * 0.02
    a = C.ns_nvfp4_step(X, *QUINTIC)
    b = N.ns_nvfp4_step(X, *QUINTIC)
    assert np.linalg.norm(a - b) <= 1e-10 * np.linalg.norm(b)
