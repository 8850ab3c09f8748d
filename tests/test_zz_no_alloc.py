"""The allocation-free quantizer (nvfp4_quantize_noalloc, scratch in a static
device array) against nvfp4_quantize with a caller workspace: the same codes,
scales and tensor scale, bit for bit, on two calls in a row (the second with
a smaller input, so that a stale scratch word from the first would show),
along both axes and for both input types."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

import newton_schulz_amd as ns  # noqa: E402
from gpu_util import DEV, host, to_dev_bf16, to_dev_f32  # noqa: E402


def _pair(xd, axis):
    ref = ns.nvfp4_quantize(xd, axis)
    got = ns.nvfp4_quantize_noalloc(xd, axis)
    return [host(t) for t in ref], [host(t) for t in got]


@pytest.mark.parametrize("axis", [ns.NVFP4_ROWS, ns.NVFP4_COLS])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_noalloc_matches_workspace_quantizer(axis, dtype):
    # the first tensor's maximum (x1000 outlier) is far above the second's, so
    # a scratch word left over from the first call would change s_g
    big = synth.student_t(512, 768, seed=31)
    big[7, 9] = 1000.0
    small = synth.student_t(64, 96, seed=32)
    for x in (big, small):
        if dtype == "bf16":
            bits, _ = synth.to_bf16(x)
            xd = to_dev_bf16(bits)
        else:
            xd = to_dev_f32(x)
        print(f"[noalloc] {dtype} axis={axis} shape={x.shape}", flush=True)
        ref, got = _pair(xd, axis)
        for r, g in zip(ref, got):
            assert np.array_equal(np.asarray(r).view(np.uint8), np.asarray(g).view(np.uint8))
    # the second call's s_g is the small tensor's own
    assert host(ns.nvfp4_quantize_noalloc(xd, axis)[2])[0] < 1000.0 / 2688.0


def test_noalloc_rejects_bad_shapes_before_launching():
    # through the C ABI (the binding refuses undersized outputs first);
    # every buffer is large enough, only the shape is wrong
    import ctypes
    x = torch.zeros((16, 32), dtype=torch.float32, device=DEV)
    codes = torch.zeros(256, dtype=torch.uint8, device=DEV)
    scales = torch.zeros(64, dtype=torch.uint8, device=DEV)
    sg = torch.zeros(1, dtype=torch.float32, device=DEV)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    for rows, cols in [(16, 24), (0, 32), (24, 16)]:
        st = ns._lib.nvfp4_quantize_noalloc(p(x), ns.NS_F32, rows, cols, ns.NVFP4_ROWS, p(codes),
                                            p(scales), p(sg), None)
        assert st == ns.NS_ERR_SHAPE, (rows, cols, st)
    assert ns._lib.nvfp4_quantize_noalloc(p(x), ns.NS_F32, 16, 32, 7, p(codes), p(scales), p(sg),
                                          None) == ns.NS_ERR_ARG
