"""Quantile clip threshold — oracle (test infrastructure only).

Source: Full-Stack FP4 (arXiv 2607.04422): §3.4 "NVFP4 Root Optimizer"
(p99 outlier clipping before the NVFP4 NS products), App. E (the Root rows
use p99 clipping) and App. F Table 8 (Root quantile ratio 0.99).

Readings (the pages give the ratio, not the estimator):
* The threshold is the q-quantile of |G| over all elements of the matrix,
  taken as an order statistic of the empirical distribution (inverted CDF):
  the k-th smallest magnitude, k = ceil(q * N) in 1-based order, i.e. the
  smallest magnitude with at least q N elements at or below it.  It is an
  element of |G|, so the GPU can find it exactly by radix selection.
* k is computed in float64 as ceil(q * N) and clamped to [1, N]; q must lie
  in (0, 1] (q = 1 gives max |G|).
* Magnitudes are ordered by their FP32 bit patterns with the sign cleared;
  NaN and infinity count as the NaN pattern, above every finite magnitude
  (as in the quantizer's tensor maximum).  BF16 inputs are widened exactly.
"""
import math

import numpy as np

NAN_KEY = np.uint32(0x7FC00000)


def abs_keys(x):
    """|x| as ordered uint32 keys (float32 bits, sign cleared; non-finite -> NaN key)."""
    b = np.asarray(x, dtype=np.float32).reshape(-1).view(np.uint32) & np.uint32(0x7FFFFFFF)
    return np.where(b >= np.uint32(0x7F800000), NAN_KEY, b).astype(np.uint32)


def quantile_rank(q, n):
    """1-based rank k = ceil(q * n) in float64, clamped to [1, n]."""
    if not (0.0 < q <= 1.0):
        raise ValueError("q must lie in (0, 1]")
    k = int(math.ceil(np.float64(q) * np.float64(n)))
    return min(max(k, 1), n)


def abs_quantile(x, q):
    """The q-quantile of |x| (the k-th smallest magnitude) as a float32."""
    keys = abs_keys(x)
    k = quantile_rank(q, keys.size)
    key = np.partition(keys, k - 1)[k - 1]
    return np.array([key], dtype=np.uint32).view(np.float32)[0]
