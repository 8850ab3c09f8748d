"""The random Hadamard transform of the NVFP4 NS iteration (Full-Stack FP4,
§3.4) on the GPU against the oracle: the transformed quantizers bit for bit
(codes, scales, s_g) on identical inputs, and the transformed NS iteration
end to end to the 2e-2 / singular-value-band bar (stable schedules, as for
the untransformed iteration in test_gpu_ns.py)."""
import numpy as np
import pytest

import synth
from oracle import ns as N
from oracle import nvfp4 as Q
from oracle import rht as R

pytestmark = pytest.mark.gpu

import newton_schulz_amd as ns  # noqa: E402
from gpu_util import host, rel_fro, same_band, to_dev_bf16, to_dev_f32  # noqa: E402

AXES = {"rows": ns.NVFP4_ROWS, "cols": ns.NVFP4_COLS}
CUBIC = (1.5, -0.5, 0.0)
QUINTIC = synth.QUINTIC


def _device_input(x, dtype):
    if dtype == "bf16":
        bits, vals = synth.to_bf16(x)
        return to_dev_bf16(bits), vals.astype(np.float32)
    x = np.ascontiguousarray(x, dtype=np.float32)
    return to_dev_f32(x), x


def _oracle(vals, axis, mask):
    # Q_1x16(x H) = rows of the FP32-transformed x; Q_16x1(H^T x) is stored
    # as the rows of its transpose, x^T H
    t = vals if axis == "rows" else vals.T
    return Q.quantize_rows(R.rht_rows_f32(t, mask).astype(np.float64))


def _check(vals, xd, axis, mask, label):
    print(f"[rht-quant] {label} shape={vals.shape} axis={axis} mask={mask:#06x}", flush=True)
    codes, scales, sg = ns.nvfp4_quantize_rht(xd, mask, AXES[axis])
    oq = _oracle(vals, axis, mask)
    gsg = host(sg)[0]
    assert (np.isnan(gsg) and np.isnan(oq.global_scale)) or \
        np.float32(gsg).view(np.uint32) == np.float32(oq.global_scale).view(np.uint32), label
    gc, gs = host(codes), host(scales)
    assert np.array_equal(gs, oq.scales), f"{label}: {np.count_nonzero(gs != oq.scales)} scale bytes differ"
    assert np.array_equal(gc, oq.codes), f"{label}: {np.count_nonzero(gc != oq.codes)} code bytes differ"


SHAPES = [(16, 16), (64, 128), (80, 48), (144, 272), (1040, 208)]
MASKS = [0x0000, 0xFFFF, 0xBEEF]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("axis", ["rows", "cols"])
@pytest.mark.parametrize("shape", SHAPES)
def test_quantize_rht_bit_exact(shape, axis, dtype):
    rows, cols = shape
    x = synth.student_t(rows, cols, seed=rows * 5 + cols)
    xd, vals = _device_input(x, dtype)
    for mask in MASKS:
        _check(vals, xd, axis, mask, f"{dtype} {shape} {axis}")


def test_quantize_rht_special_values():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((64, 64)).astype(np.float32)
    x[3, 5] = 0.0
    x[7, :16] = -0.0                      # a whole negative-zero block
    x[9, 20] = 1e-30                      # tiny next to normal values
    for axis in ("rows", "cols"):
        _check(x, to_dev_f32(x), axis, 0x1357, f"special {axis}")
    z = np.zeros((32, 48), np.float32)
    _check(z, to_dev_f32(z), "rows", 0xFFFF, "all zero")
    y = x.copy()
    y[10, 10] = np.inf
    _check(y, to_dev_f32(y), "rows", 0x00FF, "with inf")


def test_quantize_rht_full_size_sampled_rows():
    """The benchmark's iterate shape, 3072 x 8192 FP32, with the tensor-wide
    s_g of the transformed tensor; sampled rows compared byte for byte."""
    x = (synth.gaussian(3072, 8192, seed=21) / np.sqrt(3072 * 8192)).astype(np.float32)
    mask = 0xA5C3
    codes, scales, sg = ns.nvfp4_quantize_rht(to_dev_f32(x), mask, ns.NVFP4_ROWS)
    t = R.rht_rows_f32(x, mask).astype(np.float64)
    amax = Q.tensor_amax(t)
    rows = np.random.default_rng(1).choice(3072, 24, replace=False)
    oq = Q.quantize_rows(t[rows], amax=amax)
    assert np.float32(host(sg)[0]).view(np.uint32) == np.float32(oq.global_scale).view(np.uint32)
    assert np.array_equal(host(codes)[rows], oq.codes)
    assert np.array_equal(host(scales)[rows], oq.scales)


def _compare_ns(got, G, coeffs, clip, masks, label):
    want = N.ns_nvfp4(G.astype(np.float64), coeffs, clip=clip, rht_masks=masks)
    err = rel_fro(got, want)
    band, gb, ob = same_band(got, want)
    print(f"[ns-rht] {label}: rel_fro={err:.3g} band_dev={band:.3g} gpu={gb} oracle={ob}", flush=True)
    assert got.shape == want.shape
    assert err <= 2e-2, (label, err)
    assert band <= 0.05, (label, band)


@pytest.mark.parametrize("coeffs,label", [([CUBIC] * 5, "cubic x5"), ([QUINTIC] * 2, "quintic x2")])
def test_ns_rht_256x512(coeffs, label):
    spec = synth.ns_workload("ns256x512")
    G, bits, clip = synth.ns_matrix(spec, 0)
    masks = synth.rht_masks(len(coeffs), seed=17)
    got = host(ns.ns_orthogonalize_rht(to_dev_f32(G), coeffs, masks, clip))
    _compare_ns(got, G, coeffs, clip, masks, f"256x512 {label}")


@pytest.mark.parametrize("shape", [(400, 144), (64, 64)])
def test_ns_rht_orientations(shape):
    G = synth.gaussian(*shape, seed=sum(shape) + 1)
    coeffs = [CUBIC] * 5
    masks = synth.rht_masks(5, seed=shape[0])
    got = host(ns.ns_orthogonalize_rht(to_dev_f32(G), coeffs, masks))
    _compare_ns(got, G, coeffs, np.inf, masks, f"gaussian {shape}")


def test_ns_rht_bf16_lowrank_with_clip():
    spec = dict(synth.ns_workload("ns2048"), shapes=[(384, 640)])
    G, bits, clip = synth.ns_matrix(spec, 0)
    coeffs = [CUBIC] * 5
    masks = synth.rht_masks(5, seed=23)
    got = host(ns.ns_orthogonalize_rht(to_dev_bf16(bits), coeffs, masks, clip, out_dtype=ns.NS_BF16))
    _compare_ns(got, G, coeffs, clip, masks, "bf16 lowrank 384x640 clip")


def test_ns_rht_2048_full_size():
    """The 2048^2 BF16 low-rank workload with its 8 x RMS clip, transformed."""
    spec = synth.ns_workload("ns2048")
    G, bits, clip = synth.ns_matrix(spec, 0)
    coeffs = [CUBIC] * 5
    masks = synth.rht_masks(5, seed=3)
    got = host(ns.ns_orthogonalize_rht(to_dev_bf16(bits), coeffs, masks, clip))
    _compare_ns(got, G, coeffs, clip, masks, "2048^2 lowrank cubic")


def test_ns_rht_rejects_missing_masks():
    import ctypes
    fake = ctypes.c_void_p(0x1000)
    coeffs = (ctypes.c_float * 3)(*CUBIC)
    st = ns._lib.ns_orthogonalize_rht(fake, 0, 32, 32, coeffs, 1, 1.0, None, ctypes.c_void_p(0x100000000),
                                      0, fake, 1 << 20, None)
    assert st == ns.NS_ERR_ARG
