"""The on-device quantile clip threshold (p99 outlier clipping of the NVFP4
Root path; Full-Stack FP4 §3.4, App. F Table 8) against the oracle: the
threshold bit for bit, and the NS iteration clipped at it end to end."""
import numpy as np
import pytest

import synth
from oracle import ns as N
from oracle import quantile as QT

pytestmark = pytest.mark.gpu

import newton_schulz_amd as ns  # noqa: E402
from gpu_util import host, rel_fro, same_band, to_dev_bf16, to_dev_f32  # noqa: E402

QS = [0.01, 0.5, 0.9, 0.99, 0.999, 1.0]
CUBIC = (1.5, -0.5, 0.0)


def _check(vals, xd, label):
    for q in QS:
        got = np.float32(host(ns.ns_abs_quantile(xd, q))[0])
        want = QT.abs_quantile(vals, q)
        print(f"[quantile] {label} q={q} gpu={got!r} oracle={want!r}", flush=True)
        assert got.view(np.uint32) == np.float32(want).view(np.uint32), (label, q)


@pytest.mark.parametrize("n", [16, 256, 4096, 1 << 20])
def test_quantile_f32_bit_exact(n):
    x = synth.student_t(1, n, seed=n).astype(np.float32).reshape(-1)
    _check(x, to_dev_f32(x), f"f32 t3 n={n}")


@pytest.mark.parametrize("n", [16, 4096, 1 << 20])
def test_quantile_bf16_bit_exact(n):
    bits, vals = synth.to_bf16(synth.gaussian(1, n, seed=n + 1).reshape(-1))
    _check(vals.astype(np.float32), to_dev_bf16(bits), f"bf16 gaussian n={n}")


def test_quantile_ties_zeros_and_nonfinite():
    rng = np.random.default_rng(3)
    x = rng.integers(-3, 4, size=4096).astype(np.float32)       # heavy ties, signed zeros
    x[::7] = -0.0
    _check(x, to_dev_f32(x), "integer ties")
    z = np.zeros(1024, np.float32)
    _check(z, to_dev_f32(z), "all zero")
    y = rng.standard_normal(4096).astype(np.float32)
    y[:30] = np.nan
    y[30:60] = -np.inf
    _check(y, to_dev_f32(y), "1.5% non-finite")            # q >= 0.99 reaches NaN
    # the same inputs in BF16 (whose 15-bit keys are counted in one pass)
    for label, arr in (("integer ties", x), ("all zero", z), ("1.5% non-finite", y)):
        bits, vals = synth.to_bf16(arr)
        _check(vals, to_dev_bf16(bits), f"bf16 {label}")
    # BF16 magnitudes that differ only in their low mantissa bits
    bits, vals = synth.to_bf16(np.linspace(1.0, 1.0625, 4096, dtype=np.float32))
    _check(vals, to_dev_bf16(bits), "bf16 one binade")


def test_quantile_every_bf16_pattern():
    """All 65536 BF16 bit patterns (both signs, subnormals, infinities and
    NaNs) in a shuffled order: every one of the 2^15 magnitude keys occurs
    twice, so each quantile lands on a known key."""
    pats = np.random.default_rng(4).permutation(np.arange(1 << 16, dtype=np.uint32)).astype(np.uint16)
    vals = (pats.astype(np.uint32) << 16).view(np.float32)
    qs = [1 / 65536, 0.25, 0.5, 0.75, 0.9, 0.99, 0.999, 1.0]
    xd = to_dev_bf16(pats)
    for q in qs:
        got = np.float32(host(ns.ns_abs_quantile(xd, q))[0])
        want = QT.abs_quantile(vals, q)
        print(f"[quantile] every bf16 pattern q={q} gpu={got!r} oracle={want!r}", flush=True)
        assert got.view(np.uint32) == np.float32(want).view(np.uint32), q


def test_quantile_full_size_gradient():
    """The 3072 x 8192 BF16 gradient of the benchmark workload."""
    G, bits, _ = synth.ns_matrix(synth.ns_workload("ns3072x8192"), 0)
    got = np.float32(host(ns.ns_abs_quantile(to_dev_bf16(bits), 0.99))[0])
    assert got.view(np.uint32) == np.float32(QT.abs_quantile(G, 0.99)).view(np.uint32)


def _compare(got, G, coeffs, q, label, masks=None):
    clip = float(QT.abs_quantile(G, q))
    want = N.ns_nvfp4(G.astype(np.float64), coeffs, clip=clip, rht_masks=masks)
    err = rel_fro(got, want)
    band, gb, ob = same_band(got, want)
    print(f"[ns-qclip] {label}: clip={clip:.4g} rel_fro={err:.3g} band_dev={band:.3g}", flush=True)
    assert err <= 2e-2, (label, err)
    assert band <= 0.05, (label, band)


def test_ns_with_quantile_clip():
    spec = dict(synth.ns_workload("ns2048"), shapes=[(384, 640)])
    G, bits, _ = synth.ns_matrix(spec, 0)
    coeffs = [CUBIC] * 5
    got = host(ns.ns_orthogonalize_ex(to_dev_bf16(bits), coeffs, clip_quantile=0.99))
    _compare(got, G, coeffs, 0.99, "bf16 lowrank 384x640 p99")


def test_ns_with_quantile_clip_and_transform_transposed():
    G = synth.student_t(640, 256, seed=9)          # m > n: runs on G^T
    bits, vals = synth.to_bf16(G)
    coeffs = [CUBIC] * 5
    masks = synth.rht_masks(5, seed=9)
    got = host(ns.ns_orthogonalize_ex(to_dev_bf16(bits), coeffs, clip_quantile=0.99, rht_masks=masks))
    _compare(got, vals, coeffs, 0.99, "bf16 t3 640x256 p99 + H", masks=masks)


def test_ns_ex_without_options_matches_plain_call():
    G = synth.gaussian(128, 256, seed=4)
    Gd = to_dev_f32(G)
    coeffs = [CUBIC] * 3
    a = host(ns.ns_orthogonalize(Gd, coeffs, 2.0))
    b = host(ns.ns_orthogonalize_ex(Gd, coeffs, clip=2.0))
    assert np.array_equal(a, b)


def test_invalid_quantiles_are_rejected():
    x = to_dev_f32(np.ones(64, np.float32))
    for q in (0.0, -0.5, 1.5, float("nan")):
        with pytest.raises(ns.NSError) as e:
            ns.ns_abs_quantile(x, q)
        assert e.value.status == ns.NS_ERR_ARG
    G = to_dev_f32(synth.gaussian(32, 64, seed=1))
    with pytest.raises(ns.NSError) as e:
        ns.ns_orthogonalize_ex(G, [CUBIC], clip_quantile=2.0)
    assert e.value.status == ns.NS_ERR_ARG


def test_grouped_ex_matches_single_calls():
    shapes = [(128, 256), (256, 128), (96, 96)]
    Gs = [to_dev_f32(synth.student_t(r, c, seed=20 + i)) for i, (r, c) in enumerate(shapes)]
    coeffs = [CUBIC] * 3
    masks = synth.rht_masks(3, seed=2)
    outs = ns.ns_orthogonalize_grouped_ex(Gs, coeffs, clip_quantile=0.99, rht_masks=masks)
    for g, o in zip(Gs, outs):
        single = host(ns.ns_orthogonalize_ex(g, coeffs, clip_quantile=0.99, rht_masks=masks))
        assert np.array_equal(host(o), single)
    # without a quantile the per-matrix clips apply, as in ns_orthogonalize_grouped
    clips = [0.05, 1.0, 0.02]
    outs = ns.ns_orthogonalize_grouped_ex(Gs, coeffs, clips=clips)
    ref = ns.ns_orthogonalize_grouped(Gs, coeffs, clips)
    for a, b in zip(outs, ref):
        assert np.array_equal(host(a), host(b))
