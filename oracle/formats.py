"""Element and scale codes of NVFP4 — oracle side (test infrastructure only).

Source: Full-Stack FP4 (arXiv 2607.04422), §2 "Preliminaries", paragraph
"NVFP4 format": elements are E2M1 (1 sign, 2 exponent, 1 mantissa bit), each
16-element block carries one FP8 E4M3 scale s, the tensor one FP32 scale s_g,
and a value decodes as x_E2M1 * s * s_g.  §3.4 says every quantization on the
Newton–Schulz path uses RTN (round to nearest).

Readings taken where the page is silent:
* E4M3 is the OCP "E4M3FN" variant: exponent bias 7, no infinities, the one
  NaN pattern per sign is S.1111.111, largest finite 448, subnormal step 2^-9.
* E2M1 has exponent bias 1 and no NaN/Inf: magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6.
* RTN means round to nearest with ties to the even code (mantissa LSB 0), and
  saturation at the largest finite magnitude.

Encoding never divides.  The value to be rounded is an exact quotient
num/den of two FP64 numbers; the code is the number of grid midpoints that
num exceeds after each midpoint is multiplied by den.  The callers guarantee
that every product midpoint*den is exact in FP64 (few significant bits on
each side), so every decision is an exact comparison of reals.
"""
import numpy as np

# ---------------------------------------------------------------- E2M1 ----

def e2m1_decode(code):
    """Closed-form value of a 4-bit E2M1 code (array or scalar), as float64.

    Bit 3 is the sign, bits 2..1 the exponent e (bias 1), bit 0 the mantissa
    m; e == 0 encodes the subnormal m * 0.5, otherwise 2^(e-1) * (1 + m/2).
    """
    code = np.asarray(code, dtype=np.int64)
    sign = np.where((code >> 3) & 1, -1.0, 1.0)
    e = (code >> 1) & 3
    m = code & 1
    mag = np.where(e == 0, m * 0.5, np.ldexp(1.0 + m * 0.5, (e - 1).astype(np.int32)))
    return sign * mag


#: magnitudes of the eight non-negative E2M1 codes, code order 0..7
E2M1_MAGNITUDES = e2m1_decode(np.arange(8))
#: midpoints between neighbouring magnitudes (0.25, 0.75, ..., 5)
E2M1_MIDPOINTS = 0.5 * (E2M1_MAGNITUDES[:-1] + E2M1_MAGNITUDES[1:])


def e2m1_encode_quotient(num, den):
    """Magnitude code (0..7) of RNE_E2M1(num / den), num >= 0, den > 0.

    Midpoint k lies between codes k and k+1.  On an exact tie the even code
    wins: for even k the value must exceed the midpoint to move up, for odd
    k reaching it is enough.  Above the last midpoint the code saturates at
    7 (magnitude 6).  Requires mid*den exact in FP64 (the quantizer's den is
    s * s_g with at most 4 + 24 significant bits; midpoints have at most 3).
    """
    num = np.asarray(num, dtype=np.float64)
    den = np.asarray(den, dtype=np.float64)
    code = np.zeros(np.broadcast(num, den).shape, dtype=np.int64)
    for k, mid in enumerate(E2M1_MIDPOINTS):
        thr = mid * den
        if k % 2 == 0:
            code += num > thr
        else:
            code += num >= thr
    return code


# --------------------------------------------------------------- E4M3FN ---

def e4m3fn_decode(byte):
    """Closed-form value of an E4M3FN byte (array or scalar), as float64.

    Bit 7 sign, bits 6..3 exponent E (bias 7), bits 2..0 mantissa M.
    E == 0: M * 2^-9 (subnormal).  E == 15 and M == 7: NaN.
    Otherwise 2^(E-7) * (1 + M/8).
    """
    b = np.asarray(byte, dtype=np.int64)
    sign = np.where((b >> 7) & 1, -1.0, 1.0)
    E = (b >> 3) & 15
    M = b & 7
    mag = np.where(E == 0, M * 2.0 ** -9,
                   np.ldexp(1.0 + M / 8.0, (E - 7).astype(np.int32)))
    mag = np.where((E == 15) & (M == 7), np.nan, mag)
    return sign * mag


#: values of the 127 non-negative finite E4M3FN codes 0x00..0x7E, ascending
E4M3_GRID = e4m3fn_decode(np.arange(127))
#: the 126 midpoints between neighbouring grid values
E4M3_MIDPOINTS = 0.5 * (E4M3_GRID[:-1] + E4M3_GRID[1:])
E4M3_MAX = float(E4M3_GRID[-1])  # 448


def e4m3fn_encode_quotient(num, den):
    """Byte of RNE_E4M3FN(num / den) for num >= 0 and a scalar den > 0.

    Counts the midpoints (times den) that num exceeds; on an exact tie the
    even code is taken.  Quotients above 448 saturate to 0x7E (448); a
    quotient at or below 2^-10 (half the smallest subnormal) gives 0.
    Requires mid*den exact in FP64 (midpoints have at most 5 significant
    bits; the quantizer's den = 6*s_g has at most 26).
    """
    num = np.asarray(num, dtype=np.float64)
    thr = E4M3_MIDPOINTS * float(den)          # ascending, exact products
    below = np.searchsorted(thr, num, side="left")   # midpoints < num
    at = np.minimum(below, thr.size - 1)
    tie = (below < thr.size) & (thr[at] == num)
    # a tie sits between codes `below` and `below+1`: keep the even one
    return below + (tie & (below % 2 == 1))
