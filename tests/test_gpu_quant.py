"""GPU quantizer / dequantizer against the oracle: bit-exact codes, scales,
s_g and dequantized values on identical inputs (through the C ABI)."""
import os

import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from oracle import nvfp4 as Q

pytestmark = pytest.mark.gpu

import newton_schulz_amd as ns  # noqa: E402  (fails loudly when the library is missing)
from gpu_util import DEV, host, to_dev_bf16, to_dev_f32  # noqa: E402

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
AXES = {"rows": ns.NVFP4_ROWS, "cols": ns.NVFP4_COLS}


def _device_input(x, dtype):
    if dtype == "bf16":
        bits, vals = synth.to_bf16(x)
        return to_dev_bf16(bits), vals
    x = np.ascontiguousarray(x, dtype=np.float32)
    return to_dev_f32(x), x


def _oracle(vals, axis):
    return Q.quantize_rows(vals) if axis == "rows" else Q.quantize_cols(vals)


def _check_quant(vals, xd, axis, label):
    print(f"[quant] {label} shape={vals.shape} axis={axis}", flush=True)
    codes, scales, sg = ns.nvfp4_quantize(xd, AXES[axis])
    oq = _oracle(vals, axis)
    gsg = host(sg)[0]
    assert (np.isnan(gsg) and np.isnan(oq.global_scale)) or \
        np.float32(gsg).view(np.uint32) == np.float32(oq.global_scale).view(np.uint32), label
    gc, gs = host(codes), host(scales)
    assert np.array_equal(gs, oq.scales), f"{label}: {np.count_nonzero(gs != oq.scales)} scale bytes differ"
    assert np.array_equal(gc, oq.codes), f"{label}: {np.count_nonzero(gc != oq.codes)} code bytes differ"
    return codes, scales, sg, oq


def _check_dequant(codes, scales, sg, oq, rows, cols, axis, label):
    want = Q.dequantize_rows(oq)
    if axis == "cols":
        want = want.T
    for od, rnd in ((ns.NS_F32, lambda v: v.astype(np.float32).astype(np.float64)),
                    (ns.NS_BF16, Q.round_to_bf16)):
        out = ns.nvfp4_dequantize(codes, scales, sg, rows, cols, AXES[axis], od)
        got = host(out)
        ref = rnd(want)
        same = (got == ref) | (np.isnan(got) & np.isnan(ref))
        assert same.all(), f"{label} dequant dtype={od}: {np.count_nonzero(~same)} differ"
        assert np.array_equal(np.signbit(got[~np.isnan(got)]), np.signbit(ref[~np.isnan(ref)]))


SHAPES = [(16, 16), (64, 128), (80, 48), (144, 272), (256, 512), (1040, 208)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("axis", ["rows", "cols"])
@pytest.mark.parametrize("shape", SHAPES)
def test_quantize_dequantize_bit_exact(shape, axis, dtype):
    rows, cols = shape
    x = synth.student_t(rows, cols, seed=rows * 7 + cols)
    xd, vals = _device_input(x, dtype)
    label = f"student_t {dtype}"
    codes, scales, sg, oq = _check_quant(vals, xd, axis, label)
    _check_dequant(codes, scales, sg, oq, rows, cols, axis, label)


def test_hand_worked_fixture_on_gpu():
    d = {}
    for line in open(os.path.join(GOLDEN, "nvfp4_worked_2x32.txt")):
        if line.strip() and not line.startswith("#"):
            k, *v = line.split()
            d[k] = v
    t = np.array([[float(v) for v in d["row0"]], [float(v) for v in d["row1"]]], np.float32)
    t = np.concatenate([t] * 8)                      # 16 rows so both axes are legal
    for axis in ("rows", "cols"):
        codes, scales, sg, oq = _check_quant(t, to_dev_f32(t), axis, "fixture")
        if axis == "rows":
            assert host(codes)[:2].tolist() == [[int(x, 16) for x in d["codes0"]],
                                                [int(x, 16) for x in d["codes1"]]]
            assert host(scales)[:2].tolist() == [[int(x, 16) for x in d["scales0"]],
                                                 [int(x, 16) for x in d["scales1"]]]
        _check_dequant(codes, scales, sg, oq, 16, 32, axis, "fixture")


def _ties_tensor(rng, rows, cols, e_sg):
    """Elements placed exactly on E2M1 midpoints of their block, or one
    float32 ulp either side, with exactly known scales."""
    sg = 2.0 ** e_sg
    nb = cols // 16
    sbytes = rng.integers(0x10, 0x7E, size=(rows, nb))
    sbytes[0, 0] = 0x7E
    s = F.e4m3fn_decode(sbytes)
    mids = F.E2M1_MIDPOINTS
    # magnitudes up to 5 (no 6): a nudged element never exceeds the pinned
    # block maximum 6*s*s_g, so every scale and s_g stay exact
    q = rng.choice(np.concatenate([mids, F.E2M1_MAGNITUDES[:-1]]), size=(rows, cols))
    t = q * np.repeat(s, 16, axis=1) * sg
    t = t.astype(np.float32)
    nudge = rng.integers(-1, 2, size=t.shape)
    t = np.where(nudge < 0, np.nextafter(t, np.float32(0)), np.where(nudge > 0, np.nextafter(t, np.float32(1e30)), t))
    t = t * np.where(rng.random(t.shape) < 0.5, -1, 1).astype(np.float32)
    t[:, ::16] = (6 * s * sg).astype(np.float32)        # pin every scale
    return t.astype(np.float32)


@pytest.mark.parametrize("e_sg", [-7, -40, 20])
@pytest.mark.parametrize("axis", ["rows", "cols"])
def test_exact_ties_and_neighbours(e_sg, axis):
    rng = np.random.default_rng(50 - e_sg)
    t = _ties_tensor(rng, 64, 96, e_sg)
    if axis == "cols":
        t = np.ascontiguousarray(t.T)
    codes, scales, sg, oq = _check_quant(t, to_dev_f32(t), axis, f"ties e_sg={e_sg}")
    _check_dequant(codes, scales, sg, oq, *t.shape, axis, "ties")


@pytest.mark.parametrize("scale", [2.0 ** -126, 2.0 ** -110, 2.0 ** 100])
def test_extreme_magnitudes(scale):
    x = synth.student_t(48, 64, seed=9) * np.float32(scale)
    x = x.astype(np.float32)
    for axis in ("rows", "cols"):
        codes, scales, sg, oq = _check_quant(x, to_dev_f32(x), axis, f"scale={scale}")
        _check_dequant(codes, scales, sg, oq, 48, 64, axis, f"scale={scale}")


def test_wide_dynamic_range_blocks():
    # block maxima spread over 2^-30 .. 1 of the tensor max: zero and
    # subnormal E4M3 scales and many saturated codes
    rng = np.random.default_rng(11)
    x = rng.standard_normal((64, 256)).astype(np.float64)
    x *= np.exp2(rng.uniform(-30, 0, size=(64, 16))).repeat(16, axis=1)
    x = x.astype(np.float32)
    for dtype in ("f32", "bf16"):
        for axis in ("rows", "cols"):
            xd, vals = _device_input(x, dtype)
            codes, scales, sg, oq = _check_quant(vals, xd, axis, f"range {dtype}")
            if axis == "rows":          # the spread is per row block
                assert np.any(oq.scales == 0) and np.any((oq.scales > 0) & (oq.scales < 8))
            _check_dequant(codes, scales, sg, oq, 64, 256, axis, "range")


def test_zero_nan_inf():
    z = np.zeros((32, 32), np.float32)
    z[3, 5] = -0.0
    _check_quant(z, to_dev_f32(z), "rows", "zeros")
    for bad in (np.nan, np.inf, -np.inf):
        x = synth.gaussian(32, 48, seed=1)
        x[7, 9] = bad
        for axis in ("rows", "cols"):
            codes, scales, sg, oq = _check_quant(x, to_dev_f32(x), axis, f"bad={bad}")
            assert np.isnan(host(sg)[0])
            out = host(ns.nvfp4_dequantize(codes, scales, sg, 32, 48, AXES[axis]))
            assert np.all(np.isnan(out))


def _bf16_midpoint_scales(u, rng, want):
    """float32 tensor scales s_g for which RN_f32(u * s_g) has low half 0x8000,
    a bf16 midpoint, with the exact product above it, below it, or on it."""
    from fractions import Fraction
    found = []
    while len(found) < want:
        hi = int(rng.integers(0x3000, 0x4F00))          # a normal bf16 value
        m = np.uint32((hi << 16) | 0x8000).view(np.float32)
        sg0 = np.float32(float(Fraction(float(m)) / Fraction(u)))
        for d in range(-3, 4):
            sg = np.float32(np.uint32(sg0.view(np.uint32) + np.uint32(d) if d >= 0
                                      else sg0.view(np.uint32) - np.uint32(-d)).view(np.float32))
            exact = Fraction(u) * Fraction(float(sg))         # <= 30 bits: exact in float64
            f32 = np.float32(float(exact))
            if int(f32.view(np.uint32)) & 0xFFFF == 0x8000:
                found.append((sg, (exact > Fraction(float(f32))) - (exact < Fraction(float(f32)))))
    return found


@pytest.mark.parametrize("dtype", [ns.NS_BF16, ns.NS_F32])
def test_decode_rounds_once_at_bf16_midpoints(dtype):
    """Dequantized values u * s_g rounded once to bf16 (or f32), where the
    float32 product lands exactly on a bf16 midpoint: with the exact product
    above it, below it (double rounding would go the wrong way) and on it
    (ties to even), each among random codes and scales of the same 8-value
    items; and a tensor scale below 2^-90, where products can be tiny."""
    rng = np.random.default_rng(11)
    rows, cols = 64, 64
    cases = []
    for u, want in ((1.5, 8), (3.0, 4), (0.75, 4)):
        cases += [(u, sg, side) for sg, side in _bf16_midpoint_scales(u, rng, want)]
    cases += [(1.0, np.float32((1.0 + 2.0 ** -8) * 2.0 ** -7), 0),   # exact ties: u a power of two
              (1.0, np.float32(1.0 + 2.0 ** -8), 0)]
    sides = {c[2] for c in cases}
    assert sides == {-1, 0, 1}, sides
    cases.append((1.5, np.float32(2.0 ** -120 * 1.2345), 0))  # tiny products
    q_of = {0.75: (1.5, 0x30), 1.5: (1.5, 0x38), 3.0: (3.0, 0x38), 1.0: (1.0, 0x38)}
    e2m1 = {0.5: 1, 1.0: 2, 1.5: 3, 2.0: 4, 3.0: 5, 4.0: 6, 6.0: 7}
    for n, (u, sg, side) in enumerate(cases):
        codes = rng.integers(0, 256, (rows, cols // 2), dtype=np.uint8)
        scales = rng.integers(0, 0x7F, (rows, cols // 16), dtype=np.uint8)
        q, sbyte = q_of[u]
        # the designed value at several positions, in both nibbles
        for r, c in ((0, 0), (5, 17), (63, 63), (31, 8), (31, 9)):
            scales[r, c // 16] = sbyte
            nib = e2m1[q] | (8 if (r + c) % 3 == 0 else 0)
            byte = codes[r, c // 2]
            codes[r, c // 2] = (byte & 0xF0) | nib if c % 2 == 0 else (byte & 0x0F) | (nib << 4)
        print(f"[dequant] case {n}: u={u} s_g={float(sg)!r} side={side}", flush=True)
        oq = Q.NVFP4Tensor(codes=codes, scales=scales, global_scale=np.float32(sg), rows=rows, cols=cols)
        exact = Q.dequantize_rows(oq)
        want = Q.round_to_bf16(exact) if dtype == ns.NS_BF16 else exact.astype(np.float32).astype(np.float64)
        got = host(ns.nvfp4_dequantize(torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV),
                                       torch.tensor([sg], dtype=torch.float32, device=DEV),
                                       rows, cols, ns.NVFP4_ROWS, dtype))
        same = (got == want) & (np.signbit(got) == np.signbit(want))
        assert same.all(), f"case {n}: {np.count_nonzero(~same)} values differ"


def test_full_size_quantizer_whole_tensor():
    """The same 2^28-element launch checked whole against the C++ oracle
    (pinned byte for byte to the numpy one): every code and scale byte of
    both layouts, s_g, and every dequantized BF16 value of the row layout."""
    from oracle import native as C
    rows = cols = 16384
    print("[quant] generating 2^28-element workload", flush=True)
    bits, vals = synth.quant_workload(rows, cols, seed=2)
    xd = to_dev_bf16(bits)
    codes, scales, sg = ns.nvfp4_quantize(xd, ns.NVFP4_ROWS)
    out = ns.nvfp4_dequantize(codes, scales, sg, rows, cols, ns.NVFP4_ROWS, ns.NS_BF16)
    print(f"[quant] C++ oracle on {C.threads()} threads", flush=True)
    oq = C.quantize_rows(vals)
    assert np.float32(host(sg)[0]).view(np.uint32) == np.float32(oq.global_scale).view(np.uint32)
    gs, gc = host(scales), host(codes)
    assert np.array_equal(gs, oq.scales), f"{np.count_nonzero(gs != oq.scales)} scale bytes differ"
    assert np.array_equal(gc, oq.codes), f"{np.count_nonzero(gc != oq.codes)} code bytes differ"
    del gs, gc
    print("[quant] rows: codes and scales equal; checking dequantized values", flush=True)
    got = host(out)
    deq = C.dequantize_rows(oq)
    for r0 in range(0, rows, 1024):                  # BF16 rounding in slices of 2^24 values
        want = Q.round_to_bf16(deq[r0:r0 + 1024])
        same = got[r0:r0 + 1024] == want
        assert same.all(), f"rows {r0}..: {np.count_nonzero(~same)} dequantized values differ"
        if r0 % 4096 == 0:
            print(f"[quant] dequantized rows {r0}..{r0 + 1023} equal", flush=True)
    del got, deq, out
    print("[quant] column layout", flush=True)
    ccodes, cscales, csg = ns.nvfp4_quantize(xd, ns.NVFP4_COLS)
    oqc = C.quantize_rows(np.ascontiguousarray(vals.T))
    assert np.float32(host(csg)[0]).view(np.uint32) == np.float32(oqc.global_scale).view(np.uint32)
    assert np.array_equal(host(cscales), oqc.scales)
    assert np.array_equal(host(ccodes), oqc.codes)
    print("[quant] 2^28 elements: both layouts bit-exact", flush=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tensor_maximum_on_either_side_of_the_cached_tail(dtype):
    """A 128 MB tensor, larger than the last 96 MB that the maximum pass
    reads last with allocating loads (and the encode pass first): the
    tensor maximum planted at the start, just before and at the first
    element of that tail, and at the end is found every time (s_g bit for
    bit), and the rows around the planted element and the boundary encode
    bit for bit."""
    rows, cols = (8192, 4096) if dtype == "f32" else (8192, 8192)
    esize = 4 if dtype == "f32" else 2
    boundary = (rows * cols * esize - (96 << 20)) // esize   # first element of the tail
    x = (np.random.default_rng(5).standard_normal((rows, cols)) * 1e-3).astype(np.float32)
    xd, vals = _device_input(x, dtype)
    big = 7.0                                    # exact in BF16, the unique maximum
    want_sg = Q.global_scale(big)
    for pos in (0, boundary - 1, boundary, rows * cols - 1):
        r, c = divmod(pos, cols)
        print(f"[quant] {dtype} maximum at element {pos} (row {r})", flush=True)
        old = float(vals[r, c])
        xd[r, c] = big
        codes, scales, sg = ns.nvfp4_quantize(xd, ns.NVFP4_ROWS)
        assert np.float32(host(sg)[0]).view(np.uint32) == np.float32(want_sg).view(np.uint32)
        sel = np.unique([0, r, boundary // cols - 1, boundary // cols, rows - 1])
        part = vals[sel].astype(np.float64)
        part[np.searchsorted(sel, r), c] = big
        oq = Q.quantize_rows(part, amax=big)
        assert np.array_equal(host(scales)[sel], oq.scales)
        assert np.array_equal(host(codes)[sel], oq.codes)
        xd[r, c] = old


def test_full_size_quantizer_sampled_rows():
    """16384 x 16384 BF16 Student-t tensor (2^28 elements), the launch the
    benchmark times: s_g from the whole tensor, 96 sampled rows bit-exact."""
    rows = cols = 16384
    print("[quant] generating 2^28-element workload", flush=True)
    bits, vals = synth.quant_workload(rows, cols, seed=2)
    xd = to_dev_bf16(bits)
    print("[quant] full-size quantize", flush=True)
    codes, scales, sg = ns.nvfp4_quantize(xd, ns.NVFP4_ROWS)
    out = ns.nvfp4_dequantize(codes, scales, sg, rows, cols, ns.NVFP4_ROWS, ns.NS_BF16)
    amax = Q.tensor_amax(vals)
    assert np.float32(host(sg)[0]) == Q.global_scale(amax)
    pick = np.random.default_rng(0).choice(rows, 96, replace=False)
    oq = Q.quantize_rows(vals[pick], amax=amax)
    gc = host(codes)[pick]
    gs = host(scales)[pick]
    assert np.array_equal(gs, oq.scales) and np.array_equal(gc, oq.codes)
    got = host(out)[pick]
    assert np.array_equal(got, Q.round_to_bf16(Q.dequantize_rows(oq)))
    # the column layout at full size, sampled output rows (= input columns)
    ccodes, cscales, csg = ns.nvfp4_quantize(xd, ns.NVFP4_COLS)
    pick_c = np.random.default_rng(1).choice(cols, 32, replace=False)
    oqc = Q.quantize_rows(np.ascontiguousarray(vals[:, pick_c].T), amax=amax)
    assert np.array_equal(host(cscales)[pick_c], oqc.scales)
    assert np.array_equal(host(ccodes)[pick_c], oqc.codes)
