"""Pins for the oracle's NVFP4 codecs (CPU only).

Each check compares the oracle with something other than itself: a
hand-written table from the format definition, torch's float8_e4m3fn cast,
or a brute-force nearest-grid search in exact rationals.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_e2m1_decode_matches_hand_table():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "e2m1_values.txt"))
            if l.strip() and not l.startswith("#")]
    for code_hex, val in rows:
        got = float(F.e2m1_decode(int(code_hex, 16)))
        want = float(val)
        assert got == want and np.signbit(got) == np.signbit(want), code_hex


def test_e4m3fn_decode_all_256_against_torch():
    ours = F.e4m3fn_decode(np.arange(256))
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8) \
        .view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert sorted(np.nonzero(nan)[0].tolist()) == [0x7F, 0xFF]
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))
    assert F.E4M3_MAX == 448.0


def _nearest_even(q, grid):
    """Brute force: index of the grid value nearest to the rational q,
    ties to the even index; grid is ascending (values are exact floats)."""
    best = None
    for i, g in enumerate(grid):
        d = abs(Fraction(float(g)) - q)
        key = (d, i % 2)
        if best is None or key < best[0]:
            best = (key, i)
    return best[1]


def test_e4m3_rne_matches_torch_cast_on_float32_quotients():
    # den = 1: the quotient is the float32 value itself, which torch rounds
    # once (RNE) to float8_e4m3fn; torch does not saturate, so stay <= 448.
    rng = np.random.default_rng(0)
    v = np.concatenate([
        rng.uniform(0, 448, 20000),
        np.exp2(rng.uniform(-12, 8.8, 20000)),
        F.E4M3_MIDPOINTS,                      # exact ties
        np.nextafter(F.E4M3_MIDPOINTS, 0), np.nextafter(F.E4M3_MIDPOINTS, 1e9),
        F.E4M3_GRID,
    ]).astype(np.float32)
    v = v[v <= 448]
    ours = F.e4m3fn_encode_quotient(v.astype(np.float64), 1.0)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref.astype(np.int64))


def test_e4m3_rne_brute_force_with_scaled_denominator():
    rng = np.random.default_rng(1)
    grid = F.E4M3_GRID
    for _ in range(400):
        sg = np.float32(np.exp2(rng.uniform(-20, 5)) * rng.uniform(1, 2))
        den = 6.0 * float(sg)
        q = rng.choice([rng.uniform(0, 470), float(rng.choice(F.E4M3_MIDPOINTS)),
                        float(np.exp2(rng.uniform(-11, -5)))])
        num = float(np.float32(q * den))        # a float32 block maximum
        if rng.random() < 0.3:                  # an exact tie on purpose
            mid = float(rng.choice(F.E4M3_MIDPOINTS))
            num = mid * den
            if float(np.float32(num)) != num:
                continue
        want = _nearest_even(Fraction(num) / Fraction(den), grid)
        assert int(F.e4m3fn_encode_quotient(num, den)) == want, (num, den)


def test_e4m3_saturates_and_underflows():
    assert int(F.e4m3fn_encode_quotient(460.0, 1.0)) == 0x7E
    assert int(F.e4m3fn_encode_quotient(1e30, 1.0)) == 0x7E
    assert int(F.e4m3fn_encode_quotient(2.0 ** -10, 1.0)) == 0      # tie -> even 0
    assert int(F.e4m3fn_encode_quotient(np.nextafter(2.0 ** -10, 1), 1.0)) == 1
    assert int(F.e4m3fn_encode_quotient(0.0, 1.0)) == 0


def test_e2m1_rne_brute_force():
    rng = np.random.default_rng(2)
    mags = F.E2M1_MAGNITUDES
    for _ in range(3000):
        s = float(F.e4m3fn_decode(rng.integers(1, 0x7F)))
        sg = float(np.float32(np.exp2(rng.uniform(-30, 0)) * rng.uniform(1, 2)))
        den = s * sg
        kind = rng.integers(3)
        if kind == 0:
            num = float(np.float32(rng.uniform(0, 7) * den))
        elif kind == 1:                         # exact midpoint, if representable
            num = float(rng.choice(F.E2M1_MIDPOINTS)) * den
            if float(np.float32(num)) != num:
                num = float(np.float32(num))
        else:                                   # one float32 ulp off a midpoint
            mid = np.float32(float(rng.choice(F.E2M1_MIDPOINTS)) * den)
            num = float(np.nextafter(mid, np.float32(rng.choice([-1, 1]) * np.inf)))
        want = _nearest_even(Fraction(num) / Fraction(den), mags)
        assert int(F.e2m1_encode_quotient(num, den)) == want, (num, den)


def test_e2m1_ties_go_to_even_codes():
    got = F.e2m1_encode_quotient(F.E2M1_MIDPOINTS, 1.0)
    # 0.25->0, 0.75->1.0, 1.25->1.0, 1.75->2.0, 2.5->2.0, 3.5->4.0, 5->4.0
    assert got.tolist() == [0, 2, 2, 4, 4, 6, 6]
    assert int(F.e2m1_encode_quotient(6.5, 1.0)) == 7
    assert int(F.e2m1_encode_quotient(1e9, 1.0)) == 7
