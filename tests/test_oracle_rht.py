"""Pins of the oracle's random Hadamard transform (oracle/rht.py) and of its
place in the NVFP4 NS iteration (oracle/ns.py, §3.4 of Full-Stack FP4)."""
import numpy as np
import pytest

from oracle import ns as N
from oracle import rht as R

MASKS = [0x0000, 0xFFFF, 0x1234, 0xBEEF, 0x8001, 0x5A5A]


def _sylvester(n):
    # independent construction: H_1 = [1], H_2k = [[H_k, H_k], [H_k, -H_k]]
    h = np.array([[1]], dtype=np.int64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def test_hadamard16_is_the_sylvester_matrix():
    H = R.hadamard16()
    assert np.array_equal(H, _sylvester(16))
    assert np.array_equal(H @ H, 16 * np.eye(16, dtype=np.int64))
    assert np.array_equal(H, H.T)


@pytest.mark.parametrize("mask", MASKS)
def test_random_hadamard_is_orthogonal(mask):
    M = R.rht_matrix(mask)
    assert np.array_equal(M @ M.T, np.eye(16))      # exact: entries are +-1/4
    assert np.array_equal(np.abs(M), np.full((16, 16), 0.25))


@pytest.mark.parametrize("mask", MASKS)
def test_rht_rows_follows_its_definition_elementwise(mask):
    # y_j = sum_i x_i s_i (-1)^popcount(i & j) / 4 for every 16-block of a row,
    # written as plain loops
    rng = np.random.default_rng(mask)
    x = rng.standard_normal((3, 48))
    want = np.zeros_like(x)
    for r in range(3):
        for b in range(3):
            for j in range(16):
                acc = 0.0
                for i in range(16):
                    s = -1.0 if (mask >> i) & 1 else 1.0
                    sgn = -1.0 if bin(i & j).count("1") % 2 else 1.0
                    acc += x[r, 16 * b + i] * s * sgn
                want[r, 16 * b + j] = acc / 4.0
    got = R.rht_rows(x, mask)
    assert np.max(np.abs(got - want)) <= 1e-14 * np.max(np.abs(want))


def test_rht_cols_is_the_transpose_of_the_row_transform():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((32, 16))
    m = 0x0F0F
    # H^T X: each 16-block of a column multiplied by (H^r)^T
    want = np.vstack([R.rht_matrix(m).T @ x[16 * b:16 * b + 16] for b in range(2)])
    assert np.allclose(R.rht_cols(x, m), want, rtol=0, atol=1e-14)


@pytest.mark.parametrize("mask", MASKS)
def test_fp32_butterfly_exact_on_integers(mask):
    # integer inputs: every partial sum is exact in FP32, so the butterfly
    # equals the FP64 product bit for bit
    rng = np.random.default_rng(mask + 1)
    x = rng.integers(-4000, 4000, size=(8, 64)).astype(np.float32)
    assert np.array_equal(R.rht_rows_f32(x, mask), R.rht_rows(x, mask).astype(np.float32))


@pytest.mark.parametrize("mask", MASKS)
def test_fp32_butterfly_within_rounding_of_fp64(mask):
    rng = np.random.default_rng(mask + 2)
    x = (rng.standard_normal((16, 128)) * np.exp(rng.uniform(-8, 8, (16, 1)))).astype(np.float32)
    got = R.rht_rows_f32(x, mask).astype(np.float64)
    want = R.rht_rows(x, mask)
    # four rounded stages; each partial sum is bounded by the block's l1 norm / 4
    l1 = np.abs(x.astype(np.float64)).reshape(16, 8, 16).sum(-1, keepdims=True)
    bound = 4 * 2.0 ** -24 * np.repeat(l1, 16, axis=-1).reshape(16, 128)
    assert np.all(np.abs(got - want) <= bound)


def _identity_quantizers(monkeypatch):
    # quantize / dequantize as exact identities (the 16x1 layout stores the
    # transpose), leaving only the transforms and the products
    monkeypatch.setattr(N, "quantize_rows", lambda t, amax=None, adaptive46=False: np.array(t, np.float64))
    monkeypatch.setattr(N, "dequantize_rows", lambda q: q)
    monkeypatch.setattr(N, "quantize_cols", lambda t, amax=None, adaptive46=False: np.array(t, np.float64).T)
    monkeypatch.setattr(N, "dequantize_cols", lambda q: q.T)


def test_transform_cancels_in_every_product(monkeypatch):
    """With exact quantizers the transformed iteration must equal the plain
    NS: H H^T = I cancels along K only if each product's two operands are
    transformed on the correct sides."""
    _identity_quantizers(monkeypatch)
    rng = np.random.default_rng(11)
    G = rng.standard_normal((32, 80))
    coeffs = [(3.4445, -4.775, 2.0315)] * 3
    masks = [0x1234, 0xBEEF, 0x0F0F]
    got = N.ns_nvfp4(G, coeffs, rht_masks=masks)
    want = N.ns_exact(G, coeffs)
    assert np.linalg.norm(got - want) <= 1e-12 * np.linalg.norm(want)


def test_misplaced_transform_does_not_cancel(monkeypatch):
    """The pin above bites: a transform on the wrong side of one operand
    (planted here in the oracle, on the CPU) breaks the cancellation."""
    _identity_quantizers(monkeypatch)
    monkeypatch.setattr(N, "rht_cols", lambda t, m: R.rht_rows(t, m))   # X H instead of H^T X
    rng = np.random.default_rng(11)
    G = rng.standard_normal((32, 80))
    coeffs = [(3.4445, -4.775, 2.0315)] * 3
    got = N.ns_nvfp4(G, coeffs, rht_masks=[0x1234, 0xBEEF, 0x0F0F])
    want = N.ns_exact(G, coeffs)
    assert np.linalg.norm(got - want) > 1e-2 * np.linalg.norm(want)


def test_transformed_quantized_ns_tracks_exact_ns():
    # cubic schedule on a well-conditioned matrix: NVFP4 with the transform
    # stays within the quantization noise of the exact iteration
    rng = np.random.default_rng(5)
    G = rng.standard_normal((48, 96))
    coeffs = [(1.5, -0.5, 0.0)] * 5
    want = N.ns_exact(G, coeffs)
    got = N.ns_nvfp4(G, coeffs, rht_masks=[0x1111 * (i + 1) & 0xFFFF for i in range(5)])
    assert np.linalg.norm(got - want) <= 0.05 * np.linalg.norm(want)


def test_one_mask_per_step_is_required():
    with pytest.raises(ValueError):
        N.ns_nvfp4(np.ones((16, 16)), [(1.5, -0.5, 0.0)] * 2, rht_masks=[1])


@pytest.mark.parametrize("scale", [1.0, 2.0 ** -120, 2.0 ** -140, 2.0 ** 120])
def test_block_maximum_commutes_with_the_quarter_scaling(scale):
    """The tensor maximum of the transformed blocks may be taken before the
    butterfly's final multiplication by 1/4 and scaled once: x -> RN(x / 4)
    is monotone and odd in float32, subnormal results included, so
    max_i |RN(f_i / 4)| = RN(max_i |f_i| / 4).  Checked against the FP32
    butterfly of the transform on blocks whose values land in the normal,
    subnormal and near-overflow ranges."""
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((512, 64)) * scale).astype(np.float32)
    for mask in (0x0000, 0xA5C3, 0xFFFF):
        full = R.rht_rows_f32(x, mask)                       # includes the 1/4
        s = R.sign_vector(mask).astype(np.float32)
        v = (x.reshape(512, 4, 16) * s).astype(np.float32)
        h = 1
        while h < 16:                                         # the butterfly without the 1/4
            out = v.copy()
            for i in range(16):
                if i & h:
                    continue
                out[..., i] = v[..., i] + v[..., i + h]
                out[..., i + h] = v[..., i] - v[..., i + h]
            v = out
            h *= 2
        blockmax = np.abs(v).max(axis=-1).astype(np.float32)
        want = np.abs(full).reshape(512, 4, 16).max(axis=-1)
        got = (blockmax * np.float32(0.25)).astype(np.float32)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (scale, mask)
