"""Pins of the oracle's adaptive 4/6 block scaling (oracle/nvfp4.py,
``adaptive46``): each block keeps whichever of the M = 6 and M = 4 encodings
has the smaller squared error.  The M = 4 candidate is rebuilt here by brute
force over every E4M3 scale and E2M1 code, independent of the oracle's
encoders."""
from fractions import Fraction

import numpy as np

from oracle import nvfp4 as Q
from oracle.formats import e2m1_decode, e4m3fn_decode

E4M3_FINITE = [(b, Fraction(float(e4m3fn_decode(b)))) for b in range(0x7F)]   # 0x00 .. 0x7E
E2M1_MAGS = [Fraction(float(v)) for v in e2m1_decode(np.arange(8))]


def _rne(value, table):
    """Index of the table entry nearest to value; ties to the even index,
    values beyond the last entry saturate."""
    best = None
    for i, v in enumerate(table):
        key = (abs(v - value), i & 1)
        if best is None or key < best[0]:
            best = (key, i)
    return best[1]


def _brute_block(x, sg, m_max):
    """(scale byte, decoded values) of one block with its maximum mapped to m_max."""
    amax_b = max(abs(Fraction(float(v))) for v in x)
    target = amax_b / (m_max * Fraction(float(sg)))
    sbyte = E4M3_FINITE[_rne(target, [v for _, v in E4M3_FINITE])][0]
    s = Fraction(float(e4m3fn_decode(sbyte)))
    out = []
    for v in x:
        fv = Fraction(float(v))
        if s == 0:
            out.append(0.0)
            continue
        mag = E2M1_MAGS[_rne(abs(fv) / (s * Fraction(float(sg))), E2M1_MAGS)]
        out.append(float(-mag * s * Fraction(float(sg)) if v < 0 else mag * s * Fraction(float(sg))))
    return sbyte, np.array(out)


def _seq_err(x, v):
    e = 0.0
    for a, b in zip(np.asarray(x, np.float64), v):
        d = a - b
        e = e + d * d
    return e


def test_each_block_keeps_the_better_candidate():
    rng = np.random.default_rng(5)
    t = np.concatenate([rng.standard_normal((6, 64)),
                        rng.standard_t(3, (6, 64)),
                        rng.uniform(-1, 1, (6, 64)) ** 5], axis=0).astype(np.float32)
    q = Q.quantize_rows(t, adaptive46=True)
    deq = Q.dequantize_rows(q)
    sg = q.global_scale
    picked4 = 0
    for r in range(t.shape[0]):
        for b in range(t.shape[1] // 16):
            x = t[r, 16 * b:16 * b + 16]
            s6, v6 = _brute_block(x, sg, 6)
            s4, v4 = _brute_block(x, sg, 4)
            e6, e4 = _seq_err(x, v6), _seq_err(x, v4)
            want_byte, want_v = (s4, v4) if e4 < e6 else (s6, v6)
            picked4 += e4 < e6
            assert q.scales[r, b] == want_byte, (r, b)
            assert np.array_equal(deq[r, 16 * b:16 * b + 16], want_v), (r, b)
    assert 0 < picked4 < t.shape[0] * t.shape[1] // 16   # both choices occur


def test_exact_on_four_and_not_on_six():
    # a block {4, 3, 2, 1} * s * s_g decodes exactly with M = 4 (scale s) but
    # with M = 6 its scale is RNE(2s/3) and 3 * s no longer lands on a code
    big = np.full(16, 2688.0, np.float32)           # fixes s_g = 1 (amax 2688)
    s = 6.0
    blk = np.array([4, 3, 2, 1] * 4, np.float32) * s
    t = np.stack([big, blk])
    q = Q.quantize_rows(t, adaptive46=True)
    assert q.global_scale == np.float32(1.0)
    assert np.array_equal(Q.dequantize_rows(q)[1], blk.astype(np.float64))
    plain = Q.quantize_rows(t)
    assert not np.array_equal(Q.dequantize_rows(plain)[1], blk.astype(np.float64))


def test_ties_keep_six():
    # one nonzero value x with x / (6 s_g) = 1: both candidates are exact
    # (6 * 1 and 4 * 1.5), so M = 6 keeps scale 1.0 (byte 0x38)
    big = np.full(16, 2688.0, np.float32)
    blk = np.zeros(16, np.float32)
    blk[3] = 6.0
    zero = np.zeros(16, np.float32)
    q = Q.quantize_rows(np.stack([big, blk, zero]), adaptive46=True)
    assert q.scales[1, 0] == 0x38 and q.scales[2, 0] == 0x00
    assert np.array_equal(q.codes, Q.quantize_rows(np.stack([big, blk, zero])).codes)


def test_never_worse_than_plain_and_same_special_cases():
    rng = np.random.default_rng(8)
    t = (rng.standard_t(3, (32, 128)) * 0.02).astype(np.float32)
    a = Q.quantize_rows(t, adaptive46=True)
    p = Q.quantize_rows(t)
    da, dp = Q.dequantize_rows(a), Q.dequantize_rows(p)
    x = t.astype(np.float64)
    ea = Q.block_sq_error(x, np.signbit(x).astype(np.int64), *_codes_and_den(a))
    ep = Q.block_sq_error(x, np.signbit(x).astype(np.int64), *_codes_and_den(p))
    assert np.all(ea <= ep)
    assert np.sum((x - da) ** 2) < np.sum((x - dp) ** 2)
    assert a.global_scale == p.global_scale
    # NaN and all-zero tensors encode as without the option
    for u in (np.zeros((2, 32), np.float32), np.where(np.arange(64).reshape(2, 32) == 5, np.nan, 1.0)):
        ua, up = Q.quantize_rows(u, adaptive46=True), Q.quantize_rows(u)
        assert np.array_equal(ua.codes, up.codes) and np.array_equal(ua.scales, up.scales)


def test_cols_layout_is_rows_of_the_transpose():
    rng = np.random.default_rng(9)
    t = rng.standard_normal((48, 32)).astype(np.float32)
    c = Q.quantize_cols(t, adaptive46=True)
    r = Q.quantize_rows(np.ascontiguousarray(t.T), adaptive46=True)
    assert np.array_equal(c.codes, r.codes) and np.array_equal(c.scales, r.scales)


def _codes_and_den(q):
    lo = (q.codes & 0x7).astype(np.int64)
    hi = ((q.codes >> 4) & 0x7).astype(np.int64)
    mag = np.empty((q.rows, q.cols), np.int64)
    mag[:, 0::2], mag[:, 1::2] = lo, hi
    den = np.repeat(e4m3fn_decode(q.scales) * float(q.global_scale), 16, axis=1)
    return mag, den
