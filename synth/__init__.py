"""Seeded synthetic inputs for the NVFP4 Newton–Schulz workloads.

Shared by the tests (oracle side) and the benchmark (GPU side).  This module
holds none of the method's arithmetic: it only draws matrices and rounds them
to the storage dtype the workload names.  All draws use numpy's Philox
counter-based generator keyed by an integer seed, so a workload is the same
on every machine with the same numpy.

Value models (shapes and distributions of the workloads):
* ``gaussian``        — i.i.d. N(0, 1).
* ``student_t``       — t(nu=3) * 0.02, then 0.1% of the positions (chosen
  uniformly without replacement) multiplied by 50: a heavy-tailed tensor for
  the standalone quantizer.
* ``lowrank_gradient`` — a rank-32 signal S = P Q^T (Gaussian factors, scaled
  to ||S||_F = 1) plus N(0, 0.01^2) noise, then 0.1% of positions x50: the
  gradient model of the Newton–Schulz workloads.  Its clip threshold is
  8 x RMS(G) with RMS = ||G||_F / sqrt(m n) of the rounded matrix.
"""
import numpy as np

OUTLIER_FRACTION = 0.001
OUTLIER_FACTOR = 50.0


def rng(seed):
    return np.random.Generator(np.random.Philox(int(seed)))


def to_bf16(x):
    """Round float32/float64 values to bfloat16 (RNE via torch's cast).

    Returns (bits uint16 array, float32 array holding the same values).
    """
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    bits = t.view(torch.int16).numpy().view(np.uint16).copy()
    vals = (bits.astype(np.uint32) << 16).view(np.float32)
    return bits, vals


def _scale_outliers(x, g, frac=OUTLIER_FRACTION, factor=OUTLIER_FACTOR):
    flat = x.reshape(-1)
    count = int(round(frac * flat.size))
    if count:
        idx = g.choice(flat.size, size=count, replace=False)
        flat[idx] *= factor
    return x


def gaussian(rows, cols, seed):
    """i.i.d. N(0,1) float32 matrix."""
    return rng(seed).standard_normal((rows, cols), dtype=np.float32)


def student_t(rows, cols, seed, nu=3.0, scale=0.02):
    """t(nu) * scale with 0.1% of entries x50, float32."""
    g = rng(seed)
    x = (g.standard_t(nu, size=(rows, cols)) * scale).astype(np.float32)
    return _scale_outliers(x, g)


def lowrank_gradient(rows, cols, seed, rank=32, noise=0.01):
    """Rank-32 signal with ||S||_F = 1, plus N(0, noise^2), plus 0.1% x50."""
    g = rng(seed)
    P = g.standard_normal((rows, rank))
    Q = g.standard_normal((cols, rank))
    S = P @ Q.T
    S /= np.sqrt(np.sum(S * S))
    x = S + noise * g.standard_normal((rows, cols))
    return _scale_outliers(x, g).astype(np.float32)


def rms(x):
    x = np.asarray(x, dtype=np.float64)
    return float(np.sqrt(np.sum(x * x) / x.size))


# The Newton–Schulz workloads.  Coefficients: the quintic (3.4445, -4.7750,
# 2.0315) at every one of five steps.
QUINTIC = (3.4445, -4.7750, 2.0315)
STEPS = 5


def rht_masks(k, seed):
    """k 16-bit sign masks for the random Hadamard transform (one per NS
    step; bit j set = sign -1 on element j of every 16-block)."""
    return [int(v) for v in rng(seed).integers(0, 1 << 16, size=k)]


def ns_workload(name):
    """Return dict(G=list of (rows, cols) specs, dtype, coeffs, seeds).

    Matrices are produced lazily by ``ns_matrices``.
    """
    if name == "ns256x512":        # small FP32 case, N(0,1), no clip
        return dict(shapes=[(256, 512)], dtype="f32", model="gaussian",
                    seeds=[1], clip_rms=None)
    if name == "ns2048":           # square 2048^2 gradient
        return dict(shapes=[(2048, 2048)], dtype="bf16", model="lowrank",
                    seeds=[3], clip_rms=8.0)
    if name == "ns3072x8192":      # MLP up-projection shape
        return dict(shapes=[(3072, 8192)], dtype="bf16", model="lowrank",
                    seeds=[4], clip_rms=8.0)
    if name == "ns4blocks":        # four blocks: Q,K,V,O 3072^2, up 3072x8192, down 8192x3072
        shapes, seeds = [], []
        for b in range(4):
            for j, s in enumerate([(3072, 3072)] * 4 + [(3072, 8192), (8192, 3072)]):
                shapes.append(s)
                seeds.append(5 * 1000 + 6 * b + j)
        return dict(shapes=shapes, dtype="bf16", model="lowrank",
                    seeds=seeds, clip_rms=8.0)
    raise KeyError(name)


def pages_block_shapes(d):
    """Parameter shapes (out x in) of the pages' four decoder blocks at model
    width d = 4096 or 6144 (Full-Stack FP4 §4.4: d_ff = 11008 / 13824,
    32 / 48 query heads of width 128, 8 KV heads): per block Q, K, V, O, and
    the gate, up and down projections of the gated MLP; 28 matrices."""
    dff = {4096: 11008, 6144: 13824}[d]
    kv = 8 * 128
    block = [(d, d), (kv, d), (kv, d), (d, d), (dff, d), (dff, d), (d, dff)]
    return block * 4


def device_lowrank_bf16(rows, cols, seed, device, rank=32, noise=0.01):
    """``lowrank_gradient``'s value model drawn on the GPU with torch's
    seeded generator (for the large benchmark-only batches whose host
    generation would take minutes), rounded to bfloat16."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    P = torch.randn((rows, rank), generator=g, device=device)
    Q = torch.randn((cols, rank), generator=g, device=device)
    S = P @ Q.t()
    S /= S.norm()
    x = S + noise * torch.randn((rows, cols), generator=g, device=device)
    count = int(round(OUTLIER_FRACTION * rows * cols))
    idx = torch.randperm(rows * cols, generator=g, device=device)[:count]
    x.view(-1)[idx] *= OUTLIER_FACTOR
    return x.to(torch.bfloat16)


def ns_matrix(spec, i):
    """(values float32, bf16 bits or None, clip) of matrix i of a workload."""
    rows, cols = spec["shapes"][i]
    seed = spec["seeds"][i]
    if spec["model"] == "gaussian":
        x = gaussian(rows, cols, seed)
    else:
        x = lowrank_gradient(rows, cols, seed)
    bits = None
    if spec["dtype"] == "bf16":
        bits, x = to_bf16(x)
    clip = np.inf if spec["clip_rms"] is None else spec["clip_rms"] * rms(x)
    return x, bits, float(np.float32(clip))   # the clip the library receives


def quant_workload(rows=16384, cols=16384, seed=2):
    """The standalone quantizer tensor: Student-t, rounded to bf16."""
    return to_bf16(student_t(rows, cols, seed))
