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
