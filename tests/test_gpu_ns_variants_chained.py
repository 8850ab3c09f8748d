"""The benchmark's NS variants, step by step from the GPU's own state (the
NVFP4 NS iteration of §3.4 with its options): the random Hadamard transform
on every quantized operand and adaptive 4/6 block scaling, each over the five
quintic steps of the 2048^2 low-rank gradient workload, and the on-device
0.99-quantile clip, whose effect is confined to the first step.

As in test_gpu_ns_chained.py, the call with j steps is compared with the
oracle from the GPU's X_{j-1}: sampled rows of every quantized operand byte
for byte (the oracle quantizer with the same transform sign mask or 4/6 rule
on the GPU's own X, A, B), and X_j against the oracle's float64 step within
STEP_TOL and the singular-value band."""
import numpy as np
import pytest
import torch

import synth
from oracle import ns as N
from oracle import nvfp4 as Q
from oracle.quantile import abs_quantile
from oracle.rht import rht_rows_f32

pytestmark = pytest.mark.gpu

import newton_schulz_amd as ns  # noqa: E402
from gpu_util import host, rel_fro, same_band, to_dev_bf16  # noqa: E402

QUINTIC = synth.QUINTIC
STEP_TOL = 1e-2
BAND = 0.05


def _views(ws, m, n):
    v = ns.ns_workspace_views(ws, m, n)
    torch.cuda.synchronize()
    return {k: (host(t) if not isinstance(t, tuple) else tuple(x.cpu().numpy() for x in t))
            for k, t in v.items()}


def _same_rows(got, want, rows, label):
    codes, scales = got
    assert np.array_equal(codes[rows], want.codes), f"{label}: code bytes differ"
    assert np.array_equal(scales[rows], want.scales), f"{label}: scale bytes differ"


def _sym(upper):
    u = np.triu(upper.astype(np.float64))
    return u + np.triu(u, 1).T


def _call(Gd, k, clip, masks, a46, q):
    m, n = Gd.shape
    ws = torch.empty(ns.ns_workspace_bytes(m, n), dtype=torch.uint8, device=Gd.device)
    out = ns.ns_orthogonalize_ex(Gd, [QUINTIC] * k, clip=clip, clip_quantile=q,
                                 rht_masks=None if masks is None else masks[:k], adaptive46=a46,
                                 workspace=ws)
    return host(out), _views(ws, m, n)


@pytest.mark.parametrize("j", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("variant", ["rht", "adaptive46"])
def test_variant_step_from_gpu_state(variant, j):
    G, bits, clip = synth.ns_matrix(synth.ns_workload("ns2048"), 0)
    Gd = to_dev_bf16(bits)
    m, n = G.shape
    masks = synth.rht_masks(5, seed=77) if variant == "rht" else None
    a46 = variant == "adaptive46"
    a, b, c = QUINTIC
    print(f"[variants] {variant} step {j}: GPU calls", flush=True)
    Xj, h = _call(Gd, j, clip, masks, a46, 0.0)
    Xp = h["X"] if j == 1 else _call(Gd, j - 1, clip, masks, a46, 0.0)[0]
    if j > 1:
        assert np.array_equal(h["X"], Xp)
    X64 = Xp.astype(np.float64)
    rows = np.unique(np.concatenate([np.random.default_rng(j).integers(0, m, 24), [0, m - 1]]))

    if variant == "rht":
        mask = masks[j - 1]

        def quant(T, sel):            # Q_1x16 of the FP32 butterfly transform, tensor-wide s_g
            t = rht_rows_f32(T, mask).astype(np.float64)
            return Q.quantize_rows(t[sel], amax=Q.tensor_amax(t))
    else:
        def quant(T, sel):
            return Q.quantize_rows(T[sel], amax=Q.tensor_amax(T), adaptive46=True)
    A, B = _sym(h["A"]), _sym(h["B"])             # upper triangles stored
    _same_rows(h["qX"], quant(X64, rows), rows, f"{variant} qX")
    _same_rows(h["qX16"], quant(np.ascontiguousarray(X64.T), rows), rows, f"{variant} qX16")
    _same_rows(h["qA"], quant(A, rows), rows, f"{variant} qA")
    _same_rows(h["qB"], quant(B, rows), rows, f"{variant} qB")
    print(f"[variants] {variant} step {j}: operand rows equal; oracle step", flush=True)
    if j == 1:
        want = N.ns_nvfp4(G.astype(np.float64), [QUINTIC], clip=clip,
                          rht_masks=None if masks is None else masks[:1], adaptive46=a46)
    else:
        want = N.ns_nvfp4_step(X64, a, b, c, rht_mask=None if masks is None else masks[j - 1],
                               adaptive46=a46)
    err = rel_fro(Xj, want)
    band, gb, ob = same_band(Xj, want)
    print(f"[variants] {variant} step {j}: rel_fro {err:.3g}, band {band:.3g}", flush=True)
    assert err <= STEP_TOL and band <= BAND


def test_p99_clip_first_step():
    """The on-device quantile clip: the clip value equals the oracle's
    order statistic bit for bit, and the first step (the only one it
    changes) matches the oracle's from G with that clip."""
    G, bits, _ = synth.ns_matrix(synth.ns_workload("ns2048"), 0)
    Gd = to_dev_bf16(bits)
    thr = np.float32(abs_quantile(G, 0.99))
    got_thr = ns.ns_abs_quantile(Gd, 0.99)
    assert np.float32(host(got_thr)[0]).view(np.uint32) == thr.view(np.uint32)
    X1, h = _call(Gd, 1, float("inf"), None, False, 0.99)
    want = N.ns_nvfp4(G.astype(np.float64), [QUINTIC], clip=float(thr))
    err = rel_fro(X1, want)
    band, _, _ = same_band(X1, want)
    print(f"[variants] p99 step 1: clip {thr:.6g}, rel_fro {err:.3g}, band {band:.3g}", flush=True)
    assert err <= STEP_TOL and band <= BAND
    # the clipped, normalised X_0 the first step quantized
    X0 = h["X"].astype(np.float64)
    assert rel_fro(X0, N.clip_and_normalize(G.astype(np.float64), float(thr))) <= 1e-6
