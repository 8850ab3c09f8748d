"""Grouped NS calls run every class of matrices that share an iterate shape
(min(m, n) x max(m, n), either orientation) as one batch: the passes of a
step are one launch each for the whole class, with each matrix on the
kernels and tile schedule of its single call.  Every result must equal its
single call bit for bit: with both output types, with the on-device
quantile clip and adaptive 4/6, with split Gram products summed in the
product kernel and by the separate reduce kernel, for classes mixed with
matrices the batch does not take (one member, a K off the fast path), with
the random Hadamard transform, and on the benchmark's four-block batch and
the pages' d = 4096 decoder blocks at full size (also on their full route)."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

import newton_schulz_amd as ns  # noqa: E402
from gpu_util import DEV, to_dev_bf16, to_dev_f32  # noqa: E402

CUBIC = (1.5, -0.5, 0.0)

# classes: (256, 640) x3 in both orientations, (384, 384) x3, (128, 256) x1,
# (96, 96) x1 and (144, 400) x2, whose products are off the fast path
MIXED = [(256, 640), (640, 256), (256, 640), (384, 384), (384, 384), (384, 384), (128, 256),
         (96, 96), (144, 400), (400, 144)]


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


def _same(a, b):
    torch.cuda.synchronize()
    return bool(torch.equal(_bits(a), _bits(b)))


def _inputs(shapes, seed0, bf16=True):
    out = []
    for i, (r, c) in enumerate(shapes):
        x = synth.student_t(r, c, seed=seed0 + i)
        out.append(to_dev_bf16(synth.to_bf16(x)[0]) if bf16 else to_dev_f32(x))
    return out


@pytest.mark.parametrize("out_dtype", [ns.NS_F32, ns.NS_BF16])
def test_classes_equal_single_calls(out_dtype):
    Gs = _inputs(MIXED, 300)
    coeffs = [synth.QUINTIC] * 2 + [CUBIC] * 2
    clips = [0.05 + 0.01 * i for i in range(len(MIXED))]
    outs = ns.ns_orthogonalize_grouped(Gs, coeffs, clips, out_dtype=out_dtype)
    for i, (g, o, c) in enumerate(zip(Gs, outs, clips)):
        single = ns.ns_orthogonalize(g, coeffs, c, out_dtype=out_dtype)
        print(f"[batch] {MIXED[i]} out {out_dtype}", flush=True)
        assert _same(o, single), MIXED[i]


@pytest.mark.parametrize("opts", [dict(clip_quantile=0.99), dict(adaptive46=True),
                                  dict(clip_quantile=0.99, adaptive46=True)],
                         ids=["p99", "46", "p99+46"])
def test_class_options_equal_single_calls(opts):
    shapes = [(256, 512), (512, 256), (256, 512), (256, 512), (128, 384)]
    Gs = _inputs(shapes, 320, bf16=False)
    coeffs = [CUBIC] * 3
    clips = None if "clip_quantile" in opts else [0.1] * len(shapes)
    if clips is None:
        outs = ns.ns_orthogonalize_grouped_ex(Gs, coeffs, **opts)
    else:
        outs = ns.ns_orthogonalize_grouped_ex(Gs, coeffs, clips=clips, **opts)
    for i, (g, o) in enumerate(zip(Gs, outs)):
        kw = dict(opts)
        if clips is not None:
            kw["clip"] = clips[i]
        single = ns.ns_orthogonalize_ex(g, coeffs, **kw)
        assert _same(o, single), (shapes[i], opts)


def test_split_products_summed_by_the_reduce_kernel():
    """A class whose Gram product splits its tiles along K but is too short
    to sum them inside the product kernel (1024 x 2048: 36 tiles, K = 2048
    in two parts of four stages), so the batched reduce kernel sums them."""
    shapes = [(1024, 2048), (2048, 1024), (1024, 2048)]
    Gs = _inputs(shapes, 360)
    coeffs = [synth.QUINTIC] * 2 + [CUBIC]
    clips = [0.05, 0.07, 0.09]
    outs = ns.ns_orthogonalize_grouped(Gs, coeffs, clips)
    for i, (g, o, c) in enumerate(zip(Gs, outs, clips)):
        assert _same(o, ns.ns_orthogonalize(g, coeffs, c)), shapes[i]


@pytest.mark.parametrize("opts", ["rht", "route"])
def test_transform_batches_equal_single_calls(opts):
    """With the random Hadamard transform a class also runs as one batch
    when its products fold the transformed maxima (256- and 512-wide
    iterates here; (384, 384) with K = 384 does not, and runs matrix by
    matrix); every result equals its single call bit for bit, also on the
    pages' full route (transform, adaptive 4/6, quantile clip)."""
    shapes = [(256, 512), (512, 256), (256, 512), (512, 512), (512, 512), (384, 384), (384, 384)]
    Gs = _inputs(shapes, 340, bf16=False)
    coeffs = [synth.QUINTIC, synth.QUINTIC, CUBIC]
    masks = synth.rht_masks(3, seed=9)
    if opts == "rht":
        outs = ns.ns_orthogonalize_grouped_ex(Gs, coeffs, clips=[0.1] * len(shapes), rht_masks=masks)
        single = lambda g: ns.ns_orthogonalize_ex(g, coeffs, clip=0.1, rht_masks=masks)
    else:
        outs = ns.ns_orthogonalize_grouped_ex(Gs, coeffs, clip_quantile=0.99, rht_masks=masks,
                                              adaptive46=True)
        single = lambda g: ns.ns_orthogonalize_ex(g, coeffs, clip_quantile=0.99, rht_masks=masks,
                                                  adaptive46=True)
    for s_, g, o in zip(shapes, Gs, outs):
        assert _same(o, single(g)), (opts, s_)


def _device_batch(shapes, seed0):
    Gs, clips = [], []
    for i, (r, c) in enumerate(shapes):
        g = synth.device_lowrank_bf16(r, c, seed0 + i, DEV)
        rms = float(g.float().norm()) / float(np.sqrt(r * c))
        Gs.append(g)
        clips.append(float(np.float32(8.0 * rms)))
    return Gs, clips


@pytest.mark.parametrize("which", ["ns4blocks", "pages_d4096", "pages_d4096_route"])
def test_full_size_batches_equal_single_calls(which):
    if which == "ns4blocks":
        shapes = synth.ns_workload("ns4blocks")["shapes"]
    else:
        shapes = synth.pages_block_shapes(4096)
    Gs, clips = _device_batch(shapes, 7000)
    coeffs = [synth.QUINTIC] * 5
    print(f"[batch] {which}: {len(shapes)} matrices, grouped call", flush=True)
    ws = torch.empty(ns.ns_grouped_workspace_bytes(shapes), dtype=torch.uint8, device=DEV)
    if which == "pages_d4096_route":
        # the pages' full route: transform, adaptive 4/6, p99 clip
        masks = synth.rht_masks(5, seed=11)
        outs = ns.ns_orthogonalize_grouped_ex(Gs, coeffs, clip_quantile=0.99, rht_masks=masks,
                                              adaptive46=True, workspace=ws)
        single = lambda g, c: ns.ns_orthogonalize_ex(g, coeffs, clip_quantile=0.99, rht_masks=masks,
                                                     adaptive46=True)
    else:
        outs = ns.ns_orthogonalize_grouped(Gs, coeffs, clips, workspace=ws)
        single = lambda g, c: ns.ns_orthogonalize(g, coeffs, c)
    torch.cuda.synchronize()
    del ws
    for i, (g, o, c) in enumerate(zip(Gs, outs, clips)):
        assert _same(o, single(g, c)), (which, i, shapes[i])
    print(f"[batch] {which}: every matrix equal to its single call", flush=True)
