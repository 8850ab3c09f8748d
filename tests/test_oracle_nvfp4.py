"""Pins for the oracle's NVFP4 quantizer and dequantizer (CPU only)."""
import os

import numpy as np
import pytest

from oracle import formats as F
from oracle import nvfp4 as Q

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_worked():
    d = {}
    for line in open(os.path.join(GOLDEN, "nvfp4_worked_2x32.txt")):
        if line.strip() and not line.startswith("#"):
            k, *v = line.split()
            d[k] = v
    return d


def test_hand_worked_example():
    d = _read_worked()
    t = np.array([[float(v) for v in d["row0"]], [float(v) for v in d["row1"]]],
                 dtype=np.float32)
    q = Q.quantize_rows(t)
    assert float(q.global_scale) == float(d["sg"][0])
    for r in range(2):
        assert q.scales[r].tolist() == [int(x, 16) for x in d[f"scales{r}"]]
        assert q.codes[r].tolist() == [int(x, 16) for x in d[f"codes{r}"]]
    deq = Q.dequantize_rows(q)
    for r in range(2):
        want = np.array([float(v) for v in d[f"deq{r}"]])
        assert np.array_equal(deq[r], want)
        assert np.array_equal(np.signbit(deq[r]), np.signbit(want))


def _representable(rng, rows, cols, e_sg):
    """A tensor equal to q*s*s_g for chosen codes with s_g = 2^e_sg, normal
    scales, one block at scale 448 holding a +-6 and a +-6 in every block."""
    nb = cols // 16
    scale_bytes = rng.integers(0x08, 0x7F, size=(rows, nb))   # normal, finite
    scale_bytes[rng.integers(rows), rng.integers(nb)] = 0x7E   # 448
    codes = rng.integers(0, 16, size=(rows, cols))
    for r in range(rows):
        for b in range(nb):
            codes[r, 16 * b + rng.integers(16)] = rng.choice([7, 15])  # +-6
    s = np.repeat(F.e4m3fn_decode(scale_bytes), 16, axis=1)
    t = F.e2m1_decode(codes) * s * 2.0 ** e_sg
    return t, codes, scale_bytes


@pytest.mark.parametrize("e_sg", [-7, -20, 3])
def test_exactly_representable_round_trip(e_sg):
    rng = np.random.default_rng(100 + e_sg)
    t, codes, scale_bytes = _representable(rng, 8, 64, e_sg)
    t32 = t.astype(np.float32)
    assert np.array_equal(t32.astype(np.float64), t)    # exact in float32
    q = Q.quantize_rows(t32)
    assert float(q.global_scale) == 2.0 ** e_sg
    assert np.array_equal(q.scales, scale_bytes.astype(np.uint8))
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    assert np.array_equal(q.codes, packed)
    deq = Q.dequantize_rows(q)
    assert np.array_equal(deq, t) and np.array_equal(np.signbit(deq), np.signbit(t))
    # bf16 output: the values have <= 6 significant bits, so bf16 holds them
    assert np.array_equal(Q.round_to_bf16(deq), t)


def test_column_layout_is_rows_of_transpose():
    rng = np.random.default_rng(3)
    t, _, _ = _representable(rng, 64, 32, -5)     # 16x1 blocks need rows % 16
    tt = t.T.astype(np.float32)                    # 32 x 64: columns blocked by 16
    qc = Q.quantize_cols(tt)
    qr = Q.quantize_rows(tt.T)
    assert np.array_equal(qc.codes, qr.codes) and np.array_equal(qc.scales, qr.scales)
    assert np.array_equal(Q.dequantize_cols(qc), tt.astype(np.float64))


def test_idempotent_with_normal_scales():
    rng = np.random.default_rng(4)
    for trial in range(20):
        rows, cols = 16, 128
        x = rng.standard_normal((rows, cols)) * np.exp2(rng.uniform(-8, 8))
        # keep every block maximum within 28672x of the tensor maximum so
        # every scale is an E4M3 normal number
        blocks = x.reshape(rows, cols // 16, 16)
        amax = np.abs(x).max()
        bm = np.abs(blocks).max(axis=2, keepdims=True)
        blocks *= np.where(bm < amax / 20000, amax / 20000 / bm, 1.0)
        x = x.astype(np.float32)
        q1 = Q.quantize_rows(x)
        assert np.all((q1.scales & 0x7F) >= 0x08)
        q2 = Q.quantize_rows(Q.dequantize_rows(q1))
        assert q2.global_scale == q1.global_scale
        assert np.array_equal(q2.scales, q1.scales)
        assert np.array_equal(q2.codes, q1.codes)


def test_idempotence_can_fail_with_subnormal_scale():
    # documented limit of the idempotence pin: a block whose exact scale is
    # 1.6 * 2^-9 rounds up to the subnormal 2^-8; its maximum then decodes
    # below 6*s*s_g and re-encodes with a smaller scale.
    sg = 2.0 ** -7
    x = np.zeros((1, 32), dtype=np.float64)
    x[0, 0] = 2688 * sg                       # tensor max -> s_g = 2^-7
    x[0, 16] = 1.6 * 2 ** -9 * 6 * sg         # block 1 quotient 1.6*2^-9
    q1 = Q.quantize_rows(x)
    q2 = Q.quantize_rows(Q.dequantize_rows(q1))
    assert q1.scales[0, 1] == 0x02 and q2.scales[0, 1] != q1.scales[0, 1]


def test_per_block_error_bound():
    rng = np.random.default_rng(5)
    x = (rng.standard_t(3, size=(64, 256)) * 0.02).astype(np.float32)
    x.reshape(-1)[rng.choice(x.size, 30, replace=False)] *= 50
    q = Q.quantize_rows(x)
    deq = Q.dequantize_rows(q)
    s = np.repeat(F.e4m3fn_decode(q.scales), 16, axis=1)
    unit = s * float(q.global_scale)
    err = np.abs(deq - x.astype(np.float64))
    normal = np.repeat((q.scales & 0x7F) >= 0x08, 16, axis=1)
    # every element of a normal-scale block: error <= s * s_g
    assert np.all(err[normal] <= unit[normal])
    # unsaturated elements: half the grid gap of the quotient's binade
    quot = np.abs(x.astype(np.float64)) / np.where(unit > 0, unit, 1)
    gap = np.where(quot < 2, 0.5, np.where(quot < 4, 1.0, 2.0))
    ok = (unit > 0) & (quot <= 6)
    assert np.all(err[ok] <= 0.5 * gap[ok] * unit[ok])
    # zero-scale blocks hold only values at most 6 * s_g * 2^-10
    zero = unit == 0
    assert np.all(np.abs(x[zero]) <= 6 * float(q.global_scale) * 2.0 ** -10)


def test_global_scale_is_single_rounding():
    from fractions import Fraction
    rng = np.random.default_rng(6)
    for a in np.concatenate([rng.uniform(0, 1e6, 2000).astype(np.float32),
                             np.exp2(rng.uniform(-140, 120, 2000)).astype(np.float32)]):
        sg = Q.global_scale(float(a))
        exact = Fraction(float(a)) / 2688
        lo = np.nextafter(sg, np.float32(-np.inf))
        hi = np.nextafter(sg, np.float32(np.inf))
        d = abs(Fraction(float(sg)) - exact)
        assert d <= abs(Fraction(float(lo)) - exact)
        assert d <= abs(Fraction(float(hi)) - exact)


def test_zero_nan_inf_tensors():
    z = np.zeros((2, 32), np.float32)
    z[1, 3] = -0.0
    q = Q.quantize_rows(z)
    assert q.global_scale == 0 and not q.scales.any()
    assert q.codes[1, 1] == 0x80 and np.count_nonzero(q.codes) == 1
    for bad in (np.nan, np.inf, -np.inf):
        x = np.ones((1, 32), np.float32)
        x[0, 5] = bad
        q = Q.quantize_rows(x)
        assert np.isnan(q.global_scale)
        assert np.all(q.scales == 0x7F)
        assert np.all((q.codes & 0x77) == 0)
        assert np.all(np.isnan(Q.dequantize_rows(q)))


def test_round_to_bf16_against_torch_from_float32():
    import torch
    rng = np.random.default_rng(7)
    v = np.concatenate([rng.standard_normal(5000) * np.exp2(rng.uniform(-140, 127, 5000)),
                        [0.0, -0.0, 3.4e38, -3.4e38, 1e-45]]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    ours = Q.round_to_bf16(v.astype(np.float64))
    assert np.array_equal(ours, ref)
    assert np.array_equal(np.signbit(ours), np.signbit(ref))
