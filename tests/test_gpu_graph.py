"""The NS step captured into a HIP graph: every launch of the path is a
kernel (no memset or allocation inside the call), so a captured call replays
to the eager result bit for bit.  Each replay is checked, with eager work on
the same workspace between replays."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

import newton_schulz_amd as ns  # noqa: E402
from gpu_util import host, to_dev_bf16  # noqa: E402

CUBIC = (1.5, -0.5, 0.0)


def _capture(fn):
    """Warm up on a side stream, then capture fn() into a graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    return graph


# 384 x 8192: the Gram product's leftover tiles are split along K, so its
# K-parts and their reduce run on a side stream forked from the call's stream
# 256 x 512 with the transform: the products fold the transformed maxima
@pytest.mark.parametrize("variant,shape", [("plain", (384, 640)), ("plain", (384, 8192)),
                                           ("p99 clip + transform", (384, 640)),
                                           ("adaptive 4/6", (384, 640)),
                                           ("full route", (256, 512))])
def test_graph_replays_match_eager(variant, shape):
    G = synth.student_t(*shape, seed=31)
    bits, _ = synth.to_bf16(G)
    Gd = to_dev_bf16(bits)
    other = to_dev_bf16(synth.to_bf16(synth.gaussian(*shape, seed=32))[0])
    coeffs = [CUBIC] * 4
    ws = torch.empty(ns.ns_workspace_bytes(*shape), dtype=torch.uint8, device=Gd.device)
    out = torch.empty(shape, dtype=torch.float32, device=Gd.device)
    if variant == "plain":
        call = lambda g: ns.ns_orthogonalize(g, coeffs, 0.05, out=out, workspace=ws)
    elif variant == "adaptive 4/6":
        call = lambda g: ns.ns_orthogonalize_ex(g, coeffs, clip=0.05, adaptive46=True,
                                                out=out, workspace=ws)
    elif variant == "full route":
        masks = synth.rht_masks(len(coeffs), seed=3)
        call = lambda g: ns.ns_orthogonalize_ex(g, coeffs, clip_quantile=0.99, rht_masks=masks,
                                                adaptive46=True, out=out, workspace=ws)
    else:
        masks = synth.rht_masks(len(coeffs), seed=3)
        call = lambda g: ns.ns_orthogonalize_ex(g, coeffs, clip_quantile=0.99, rht_masks=masks,
                                                out=out, workspace=ws)
    call(Gd)
    want = host(out).copy()
    call(other)
    want_other = host(out).copy()
    graph = _capture(lambda: call(Gd))
    for r in range(3):
        out.fill_(float("nan"))
        call(other)                               # eager work on the same workspace
        assert np.array_equal(host(out), want_other)
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        got = host(out)
        print(f"[graph] {variant} {shape} replay {r}: equal={np.array_equal(got, want)}", flush=True)
        assert np.array_equal(got, want), (variant, shape, r)


@pytest.mark.parametrize("route", [False, True])
def test_grouped_call_captures_across_its_streams(route):
    """A grouped call forks onto internal streams and joins them back into
    the caller's stream; captured, it replays to the eager results (also on
    the pages' full route, whose 256 x 512 class runs as one transformed
    batch)."""
    shapes = [(256, 512), (512, 256), (128, 128), (384, 640), (64, 192)]
    Gs = [to_dev_bf16(synth.to_bf16(synth.student_t(r, c, seed=40 + i))[0])
          for i, (r, c) in enumerate(shapes)]
    coeffs = [CUBIC] * 3
    clips = [0.05] * len(shapes)
    outs = [torch.empty(s, dtype=torch.float32, device=Gs[0].device) for s in shapes]
    ws = torch.empty(ns.ns_grouped_workspace_bytes(shapes), dtype=torch.uint8, device=Gs[0].device)
    if route:
        masks = synth.rht_masks(len(coeffs), seed=5)
        opts = dict(clip_quantile=0.99, rht_masks=masks, adaptive46=True)
        call = lambda: ns.ns_orthogonalize_grouped_ex(Gs, coeffs, outs=outs, workspace=ws, **opts)
        single = lambda g, c: ns.ns_orthogonalize_ex(g, coeffs, **opts)
    else:
        call = lambda: ns.ns_orthogonalize_grouped(Gs, coeffs, clips, outs=outs, workspace=ws)
        single = lambda g, c: ns.ns_orthogonalize(g, coeffs, c)
    call()
    want = [host(o).copy() for o in outs]
    for g, w, c in zip(Gs, want, clips):                  # each equals its single call
        assert np.array_equal(host(single(g, c)), w)
    graph = _capture(call)
    for r in range(3):
        for o in outs:
            o.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for i, (o, w) in enumerate(zip(outs, want)):
            assert np.array_equal(host(o), w), (r, i)
    print("[graph] grouped: 3 replays equal", flush=True)


def test_grouped_call_on_caller_streams_captures():
    """The grouped call on two caller-owned streams, captured from the
    caller's stream, replays to the eager results."""
    shapes = [(256, 512), (128, 128), (384, 640)]
    Gs = [to_dev_bf16(synth.to_bf16(synth.student_t(r, c, seed=60 + i))[0])
          for i, (r, c) in enumerate(shapes)]
    coeffs = [CUBIC] * 3
    clips = [0.05] * len(shapes)
    outs = [torch.empty(s, dtype=torch.float32, device=Gs[0].device) for s in shapes]
    ws = torch.empty(ns.ns_grouped_workspace_bytes(shapes), dtype=torch.uint8, device=Gs[0].device)
    streams = [torch.cuda.Stream() for _ in range(2)]
    call = lambda: ns.ns_orthogonalize_grouped_on(Gs, coeffs, streams, clips=clips, outs=outs,
                                                  workspace=ws)
    call()
    torch.cuda.synchronize()
    want = [host(o).copy() for o in outs]
    graph = _capture(call)
    for r in range(3):
        for o in outs:
            o.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for i, (o, w) in enumerate(zip(outs, want)):
            assert np.array_equal(host(o), w), (r, i)
    print("[graph] grouped on caller streams: 3 replays equal", flush=True)
