"""Adaptive 4/6 block scaling on the GPU against the oracle: the quantizer
bit for bit (codes, scales, s_g) in both layouts, and the NS iteration with
every quantization adaptive, end to end."""
import numpy as np
import pytest

import synth
from oracle import ns as N
from oracle import nvfp4 as Q

pytestmark = pytest.mark.gpu

import newton_schulz_amd as ns  # noqa: E402
from gpu_util import host, rel_fro, same_band, to_dev_bf16, to_dev_f32  # noqa: E402

AXES = {"rows": ns.NVFP4_ROWS, "cols": ns.NVFP4_COLS}
CUBIC = (1.5, -0.5, 0.0)


def _inputs():
    rng = np.random.default_rng(46)
    yield "gaussian 64x128", rng.standard_normal((64, 128))
    yield "t3 x0.02 208x80", rng.standard_t(3, (208, 80)) * 0.02
    yield "uniform^5 144x272", rng.uniform(-1, 1, (144, 272)) ** 5
    out = rng.standard_normal((96, 160))
    out[rng.random(out.shape) < 0.01] *= 50.0
    yield "outliers x50 96x160", out
    tiny = rng.standard_normal((32, 64)) * 1e-30                     # subnormal scales
    yield "tiny 32x64", tiny
    z = rng.standard_normal((48, 48))
    z[:16] = 0.0
    z[16:32, ::3] = -0.0
    yield "zero rows and signed zeros 48x48", z
    # s_g = 1 (one block of 2688) and blocks of values that both candidates
    # often encode exactly: equal errors, decided by the double sums, keep 6
    e = rng.choice([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, 8.0, 12.0], (64, 96))
    e *= rng.choice([-1.0, 1.0], e.shape)
    e[0, :16] = 2688.0
    yield "exactly representable values 64x96", e


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("axis", ["rows", "cols"])
def test_quantize_46_bit_exact(dtype, axis):
    for label, x in _inputs():
        if dtype == "bf16":
            bits, vals = synth.to_bf16(x)
            xd = to_dev_bf16(bits)
        else:
            vals = np.ascontiguousarray(x, dtype=np.float32)
            xd = to_dev_f32(vals)
        codes, scales, sg = ns.nvfp4_quantize(xd, AXES[axis], adaptive46=True)
        oq = (Q.quantize_rows(vals, adaptive46=True) if axis == "rows"
              else Q.quantize_cols(vals, adaptive46=True))
        gs, gc = host(scales), host(codes)
        print(f"[46] {label} {dtype} {axis}: scales differ {np.count_nonzero(gs != oq.scales)}, "
              f"codes differ {np.count_nonzero(gc != oq.codes)}", flush=True)
        assert np.float32(host(sg)[0]).view(np.uint32) == np.float32(oq.global_scale).view(np.uint32)
        assert np.array_equal(gs, oq.scales), label
        assert np.array_equal(gc, oq.codes), label


def test_quantize_46_nan_tensor_and_error_reduction():
    x = synth.student_t(64, 256, seed=3).astype(np.float32)
    x[7, 9] = np.nan
    codes, scales, sg = ns.nvfp4_quantize(to_dev_f32(x), ns.NVFP4_ROWS, adaptive46=True)
    oq = Q.quantize_rows(x, adaptive46=True)
    assert np.isnan(host(sg)[0]) and np.array_equal(host(scales), oq.scales)
    assert np.array_equal(host(codes), oq.codes)
    # on heavy tails the adaptive choice lowers the total error
    y = synth.student_t(128, 512, seed=4).astype(np.float32)
    q6 = ns.nvfp4_quantize(to_dev_f32(y), ns.NVFP4_ROWS)
    q46 = ns.nvfp4_quantize(to_dev_f32(y), ns.NVFP4_ROWS, adaptive46=True)
    d6 = host(ns.nvfp4_dequantize(*q6, 128, 512, ns.NVFP4_ROWS, ns.NS_F32))
    d46 = host(ns.nvfp4_dequantize(*q46, 128, 512, ns.NVFP4_ROWS, ns.NS_F32))
    e6, e46 = np.sum((d6 - y) ** 2), np.sum((d46 - y) ** 2)
    print(f"[46] error plain {e6:.4g} adaptive {e46:.4g}", flush=True)
    assert e46 < e6


def _compare(got, G, coeffs, label, **kw):
    want = N.ns_nvfp4(G.astype(np.float64), coeffs, adaptive46=True, **kw)
    err = rel_fro(got, want)
    band, gb, ob = same_band(got, want)
    print(f"[ns-46] {label}: rel_fro={err:.3g} band_dev={band:.3g}", flush=True)
    assert err <= 2e-2, (label, err)
    assert band <= 0.05, (label, band)


@pytest.mark.parametrize("shape", [(256, 512), (384, 640), (640, 256)])
def test_ns_with_adaptive46(shape):
    G = synth.student_t(*shape, seed=sum(shape))
    bits, vals = synth.to_bf16(G)
    coeffs = [CUBIC] * 4
    got = host(ns.ns_orthogonalize_ex(to_dev_bf16(bits), coeffs, clip=0.1, adaptive46=True))
    _compare(got, vals, coeffs, f"bf16 t3 {shape} clip 0.1", clip=0.1)


def test_ns_with_adaptive46_and_transform():
    G = synth.gaussian(384, 768, seed=12)
    coeffs = [synth.QUINTIC] * 3
    masks = synth.rht_masks(3, seed=12)
    got = host(ns.ns_orthogonalize_ex(to_dev_f32(G), coeffs, rht_masks=masks, adaptive46=True))
    _compare(got, G, coeffs, "f32 gaussian 384x768 + H", rht_masks=masks)


def test_grouped_with_adaptive46_equals_single_calls():
    shapes = [(128, 256), (256, 128), (64, 192)]
    Gs = [to_dev_bf16(synth.to_bf16(synth.student_t(r, c, seed=60 + i))[0])
          for i, (r, c) in enumerate(shapes)]
    coeffs = [CUBIC] * 3
    outs = ns.ns_orthogonalize_grouped_ex(Gs, coeffs, clips=[0.1] * len(shapes), adaptive46=True)
    for i, (g, o) in enumerate(zip(Gs, outs)):
        single = host(ns.ns_orthogonalize_ex(g, coeffs, clip=0.1, adaptive46=True))
        print(f"[ns-46] grouped {shapes[i]} equal to single: {np.array_equal(host(o), single)}",
              flush=True)
        assert np.array_equal(host(o), single), shapes[i]
