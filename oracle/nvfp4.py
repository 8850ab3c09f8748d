"""NVFP4 1x16 / 16x1 quantizer and dequantizer — oracle (test infrastructure).

Source: Full-Stack FP4 (arXiv 2607.04422), §2 "NVFP4 format"
(x_hat = x_E2M1 * s * s_g; 1x16 blocks share an E4M3 scale s; one FP32 s_g
per tensor) and §3.4 (Q_1x16 and Q_16x1 in the NVFP4 NS iteration, all
quantizations RTN).

Readings (the page prints the decode rule only):
* s_g = RN_f32(amax / (6 * 448)): the tensor maximum maps to the largest
  element magnitude times the largest scale.
* s   = RNE_E4M3FN(amax_b / (6 * s_g)), exact quotient, saturating at 448.
* q   = sign(t) * RNE_E2M1(|t| / (s * s_g)), exact quotient, saturating at 6;
  when s == 0 or s_g == 0 every magnitude code is 0.
* Any NaN or infinity in the tensor makes amax NaN; then s_g is NaN, every
  scale byte is 0x7F (the E4M3FN NaN) and every magnitude code is 0, so the
  decoded tensor is all NaN.
* The sign bit of a code is the sign bit of t (so -0 and small negative
  values keep it).  Codes are packed two per byte, element 2i in the low
  nibble.  Scales are one byte per block, row-major [rows][cols/16].
* Q_16x1(T) is Q_1x16(T^T) and is stored in the layout of T^T.

Adaptive 4/6 block scaling (§3.4 says the Root quantizations use RTN and
adaptive 4/6 scaling; §5 names it adaptive M=4/M=6 block scaling after Four
Over Six [7], whose rule is not on the pages).  Readings, with ``adaptive46``:
* every block is encoded twice, with its maximum mapped to M = 6 (the rule
  above) and to M = 4 (s = RNE_E4M3FN(amax_b / (4 * s_g)), saturating at 448);
  the element codes follow from each scale by the same RTN rule;
* the block keeps the candidate with the smaller squared error
  sum (x - x_hat)^2, each difference, square and running sum rounded in
  float64 in element order (0..15); M = 6 wins ties;
* s_g is unchanged (amax / 2688), so a block whose M = 4 scale saturates
  simply loses the comparison.  The decode rule is unchanged: the scale byte
  alone says how a block decodes.
"""
from dataclasses import dataclass
from fractions import Fraction

import numpy as np

from .formats import (e2m1_decode, e4m3fn_decode, e2m1_encode_quotient,
                      e4m3fn_encode_quotient)

BLOCK = 16
AMAX_TO_SG = 6 * 448  # 2688


@dataclass
class NVFP4Tensor:
    """Packed NVFP4 tensor in the 1x16 layout of a rows x cols matrix."""
    codes: np.ndarray         # uint8 [rows, cols // 2]
    scales: np.ndarray        # uint8 [rows, cols // 16], E4M3FN bytes
    global_scale: np.float32  # s_g
    rows: int
    cols: int


def tensor_amax(t):
    """max |t| over the tensor as float64; NaN if any element is NaN or inf."""
    a = np.abs(np.asarray(t, dtype=np.float64))
    if a.size == 0:
        return 0.0
    if not np.all(np.isfinite(a)):
        return float("nan")
    return float(a.max())


def _round_fraction_to_f32(fr):
    """Round an exact rational to the nearest float32, ties to even."""
    approx = np.float32(float(fr))           # within one float32 ulp of fr
    if not np.isfinite(approx):
        return approx
    cands = [np.nextafter(approx, np.float32(-np.inf)), approx,
             np.nextafter(approx, np.float32(np.inf))]
    best = None
    for c in cands:
        if not np.isfinite(c):
            continue
        d = abs(Fraction(float(c)) - fr)
        key = (d, int(np.array(c, np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return np.float32(best[1])


def global_scale(amax):
    """s_g = RN_f32(amax / 2688), rounded once from the exact quotient."""
    if np.isnan(amax):
        return np.float32(np.nan)
    return _round_fraction_to_f32(Fraction(float(amax)) / AMAX_TO_SG)


def _encode_blocks(mag, amax_b, sg64, m_max):
    """Scale codes [rows, nblk] and magnitude codes [rows, cols] with the block
    maximum mapped to m_max (6, or 4 for the adaptive candidate), and the
    per-element unit s * s_g (float64, exact)."""
    scale_codes = e4m3fn_encode_quotient(amax_b, m_max * sg64)
    s = e4m3fn_decode(scale_codes)                        # exact float64
    den = np.repeat(s * sg64, BLOCK, axis=1)              # exact (<= 28 bits)
    mag_codes = e2m1_encode_quotient(mag, np.where(den > 0, den, 1.0))
    return scale_codes, np.where(den > 0, mag_codes, 0), den


def block_sq_error(x, neg, mag_codes, den):
    """Per block: sum over its 16 elements, in element order, of
    (x - x_hat)^2, every operation rounded in float64."""
    rows, cols = x.shape
    v = e2m1_decode(mag_codes) * den                       # exact magnitudes
    d = (x - np.where(neg == 1, -v, v)).reshape(rows, cols // BLOCK, BLOCK)
    e = np.zeros((rows, cols // BLOCK))
    for i in range(BLOCK):
        e = e + d[:, :, i] * d[:, :, i]
    return e


def quantize_rows(t, amax=None, adaptive46=False):
    """Q_1x16(t): blocks of 16 consecutive elements along each row.

    ``amax`` overrides the tensor maximum (used when ``t`` is a slice of a
    larger tensor whose maximum is known, or to share one s_g between the
    two layouts of the same tensor).  ``adaptive46`` selects M = 4 or 6 per
    block (module docstring).
    """
    t = np.asarray(t)
    if t.ndim != 2 or t.shape[1] % BLOCK:
        raise ValueError("quantize_rows needs a 2-D array with cols % 16 == 0")
    rows, cols = t.shape
    x = t.astype(np.float64)
    if amax is None:
        amax = tensor_amax(x)
    s_g = global_scale(amax)
    sg64 = float(s_g)

    mag = np.abs(x)
    blocks = mag.reshape(rows, cols // BLOCK, BLOCK)
    neg = np.signbit(x).astype(np.int64)

    if np.isnan(sg64):
        scale_codes = np.full((rows, cols // BLOCK), 0x7F, dtype=np.int64)
        mag_codes = np.zeros((rows, cols), dtype=np.int64)
    elif sg64 == 0.0:
        scale_codes = np.zeros((rows, cols // BLOCK), dtype=np.int64)
        mag_codes = np.zeros((rows, cols), dtype=np.int64)
    else:
        amax_b = blocks.max(axis=2)
        scale_codes, mag_codes, den = _encode_blocks(mag, amax_b, sg64, 6.0)
        if adaptive46:
            sc4, mc4, den4 = _encode_blocks(mag, amax_b, sg64, 4.0)
            pick4 = block_sq_error(x, neg, mc4, den4) < block_sq_error(x, neg, mag_codes, den)
            scale_codes = np.where(pick4, sc4, scale_codes)
            mag_codes = np.where(np.repeat(pick4, BLOCK, axis=1), mc4, mag_codes)

    codes4 = (neg << 3) | mag_codes
    packed = (codes4[:, 0::2] | (codes4[:, 1::2] << 4)).astype(np.uint8)
    return NVFP4Tensor(packed, scale_codes.astype(np.uint8), s_g, rows, cols)


def quantize_cols(t, amax=None, adaptive46=False):
    """Q_16x1(t) = Q_1x16(t^T): blocks of 16 down each column of t.

    The result is stored in the layout of t^T (cols rows of rows/2 bytes).
    """
    t = np.asarray(t)
    return quantize_rows(t.T, amax=tensor_amax(t) if amax is None else amax,
                         adaptive46=adaptive46)


def dequantize_rows(q):
    """Exact float64 values q * s * s_g of a 1x16 tensor, shape [rows, cols]."""
    lo = (q.codes & 0xF).astype(np.int64)
    hi = (q.codes >> 4).astype(np.int64)
    codes4 = np.empty((q.rows, q.cols), dtype=np.int64)
    codes4[:, 0::2] = lo
    codes4[:, 1::2] = hi
    s = np.repeat(e4m3fn_decode(q.scales), BLOCK, axis=1)
    return e2m1_decode(codes4) * s * float(q.global_scale)


def dequantize_cols(q):
    """Values of a 16x1 tensor in the original orientation (= rows-deq^T)."""
    return dequantize_rows(q).T


def round_to_bf16(v):
    """Round float64 values to bfloat16 (RNE, IEEE subnormals/overflow).

    Returns float64 values that are exactly bfloat16 numbers.  The rounding
    is done once from the float64 value: scale to an integer at the bf16
    ulp of the value's binade (a power-of-two scaling, exact) and round half
    to even there.
    """
    v = np.asarray(v, dtype=np.float64)
    out = v.copy()
    fin = np.isfinite(v) & (v != 0)
    a = np.abs(v[fin])
    e = np.floor(np.log2(a)).astype(np.int64)
    # guard log2 rounding at binade edges
    e = np.where(np.ldexp(1.0, e.astype(np.int32)) > a, e - 1, e)
    e = np.where(np.ldexp(1.0, (e + 1).astype(np.int32)) <= a, e + 1, e)
    ulp_exp = np.maximum(e, -126) - 7
    q = np.rint(np.ldexp(a, (-ulp_exp).astype(np.int32)))
    r = np.ldexp(q, ulp_exp.astype(np.int32))
    bf16_max = float(np.ldexp(255.0, 120))  # (2 - 2^-7) * 2^127
    r = np.where(r > bf16_max, np.inf, r)
    out[fin] = np.copysign(r, v[fin])
    return out


def bf16_bits(v):
    """uint16 bit patterns of values that are exactly bfloat16 numbers."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)
