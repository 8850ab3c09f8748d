"""Tensors with more 64-row tiles (or 128-row GEMM tiles) than a second grid
dimension can count (65535): the tiled quantizer, its dequantizer, the
transform's maxima pass and the general GEMM run on one-dimensional grids.
Sampled row ranges (the first, the one past 65535 tile rows, the last)
against the oracle."""
import numpy as np
import pytest

from oracle import nvfp4 as Q
from oracle import rht as R

pytestmark = pytest.mark.gpu

import newton_schulz_amd as ns  # noqa: E402
from gpu_util import host, to_dev_f32  # noqa: E402

ROWS = 64 * 65537           # 4,194,368 rows: one 64-row tile row past 65535


def _x(rows, cols, seed):
    return np.random.default_rng(seed).standard_normal((rows, cols)).astype(np.float32)


def _starts(rows, tile):
    return (0, tile * 65535, rows - tile)


def test_tall_column_layout_and_its_dequantization():
    x = _x(ROWS, 16, 7)
    print(f"[tall] quantize cols {x.shape}", flush=True)
    codes, scales, sg = ns.nvfp4_quantize(to_dev_f32(x), ns.NVFP4_COLS)
    amax = Q.tensor_amax(x)
    assert np.float32(host(sg)[0]) == Q.global_scale(amax)
    gc, gs = host(codes), host(scales)
    out = host(ns.nvfp4_dequantize(codes, scales, sg, ROWS, 16, ns.NVFP4_COLS))
    for r0 in _starts(ROWS, 64):
        oq = Q.quantize_cols(x[r0:r0 + 64], amax=amax)
        assert np.array_equal(gc[:, r0 // 2:r0 // 2 + 32], oq.codes), r0
        assert np.array_equal(gs[:, r0 // 16:r0 // 16 + 4], oq.scales), r0
        assert np.array_equal(out[r0:r0 + 64], Q.dequantize_cols(oq).astype(np.float32)), r0


def test_tall_transformed_rows():
    x = _x(ROWS, 16, 8)
    mask = 0xB00F
    print(f"[tall] quantize_rht rows {x.shape}", flush=True)
    codes, scales, sg = ns.nvfp4_quantize_rht(to_dev_f32(x), mask, ns.NVFP4_ROWS)
    t = R.rht_rows_f32(x, mask)
    amax = Q.tensor_amax(t)
    assert np.float32(host(sg)[0]) == Q.global_scale(amax)
    gc, gs = host(codes), host(scales)
    for r0 in _starts(ROWS, 64):
        oq = Q.quantize_rows(t[r0:r0 + 64].astype(np.float64), amax=amax)
        assert np.array_equal(gc[r0:r0 + 64], oq.codes), r0
        assert np.array_equal(gs[r0:r0 + 64], oq.scales), r0


def test_tall_general_gemm():
    M, N, K = 128 * 65537, 16, 16          # K % 128 != 0: the general kernel
    p = _x(M, K, 9)
    q = _x(N, K, 10)
    print(f"[tall] general gemm {M}x{N}x{K}", flush=True)
    pq = ns.nvfp4_quantize(to_dev_f32(p), ns.NVFP4_ROWS)
    qq = ns.nvfp4_quantize(to_dev_f32(q), ns.NVFP4_ROWS)
    out = host(ns.nvfp4_gemm(pq, qq, M, N, K))
    amax_p = Q.tensor_amax(p)
    qd = Q.dequantize_rows(Q.quantize_rows(q))
    for r0 in _starts(M, 128):
        pd = Q.dequantize_rows(Q.quantize_rows(p[r0:r0 + 128], amax=amax_p))
        want = pd @ qd.T                       # exact products, FP64 sums
        mag = np.abs(pd) @ np.abs(qd).T
        # 16 exact products summed in FP32 (at most 15 roundings of partial
        # sums) and the tensor scales applied in FP32: within 20 * 2^-24 of
        # the sum of magnitudes
        err = np.max(np.abs(out[r0:r0 + 128] - want) / np.maximum(mag, 1e-30))
        print(f"[tall] rows {r0}..: max error / sum|terms| {err:.2e}", flush=True)
        assert err <= 20 * 2.0 ** -24, (r0, err)
