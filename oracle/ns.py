"""Newton–Schulz orthogonalisation — oracle (test infrastructure only).

Source: Full-Stack FP4 (arXiv 2607.04422).
* §2 "Root optimizer": X_{k+1} = a X_k + b X_k (X_k^T X_k) + c X_k (X_k^T X_k)^2,
  coefficients per step, typically five steps.
* §3.4 "NVFP4 Root Optimizer", the NVFP4 NS iteration: the same step in the
  left-Gram form with every product taken on NVFP4 operands:
      qX = Q_1x16(X),        A  = qX qX^T
      qA = Q_1x16(A),        qA16 = Q_16x1(A),   B = b A + c qA qA16
      qB = Q_1x16(B),        qX16 = Q_16x1(X),   X' = a X + qB qX16
  Every quantization is RTN.  §3.4 also mentions p99 outlier clipping,
  applied here as a clamp of the input before normalisation.

* With ``rht_masks`` (one 16-bit sign mask per step) the iteration takes
  the random Hadamard transform of §3.4 on every quantized operand:
      qX = Q_1x16(X H),  qX16 = Q_16x1(H^T X),
      qA = Q_1x16(A H),  qA16 = Q_16x1(H^T A),  B = b A + c qA qA16,
      qB = Q_1x16(B H),  X' = a X + qB qX16,
  H = H_16^r of that step (see ``rht``); H H^T = I, so each product still
  approximates the untransformed one.

Readings (the pages leave these open):
* The adaptive 4/6 scaling of §3.4 is not applied (the method computed
  here is NVFP4 RTN with the block maximum mapped to 6); without
  ``rht_masks`` neither is the Hadamard transform.
* Orientation: if m > n the iteration runs on G^T and the result is
  transposed back, so the Gram matrix A is the smaller m x m side.
* X_0 = clamp(G, -clip, clip) / (||clamp(G)||_F + eps), eps = 1e-7, the
  clamp leaving NaN as NaN; clip = +inf disables it.
* Without the transform qX and qX16 share one s_g (from max|X|); with it
  X H and H^T X are different tensors and each has its own s_g.  A and B
  always get their own.
* b A and a X use the unquantized A and X; A itself is never re-rounded.
* Because A is symmetric, Q_16x1(A) equals Q_1x16(A)^T, so the second
  product is qA qA^T; the oracle still forms Q_16x1(A) from A itself.
* All unquantized values are float64; products of quantized operands are
  float64 matrix products of exactly dequantized values.
"""
import numpy as np

from .nvfp4 import (quantize_rows, quantize_cols, dequantize_rows,
                    dequantize_cols, tensor_amax)
from .rht import rht_rows, rht_cols

EPS = 1e-7


def clip_and_normalize(G, clip=np.inf, eps=EPS):
    """X_0 = clamp(G) / (||clamp(G)||_F + eps) in float64 (NaN stays NaN)."""
    X = np.asarray(G, dtype=np.float64)
    if np.isfinite(clip):
        X = np.where(X > clip, clip, np.where(X < -clip, -clip, X))
    norm = np.sqrt(np.sum(X * X))
    return X / (norm + eps)


def gemm_nt(P, Q):
    """C = P Q^T in float64 (a library matrix product)."""
    return np.asarray(P, np.float64) @ np.asarray(Q, np.float64).T


def _orient(G):
    G = np.asarray(G)
    if G.ndim != 2:
        raise ValueError("G must be 2-D")
    return (G.T, True) if G.shape[0] > G.shape[1] else (G, False)


def ns_exact(G, coeffs, clip=np.inf, eps=EPS):
    """Newton–Schulz on unquantized float64 operands (left-Gram form).

    X' = a X + (b A + c A A) X with A = X X^T, i.e. the Root recurrence of §2
    written for the smaller Gram side.
    """
    Gt, transposed = _orient(G)
    X = clip_and_normalize(Gt, clip, eps)
    for a, b, c in coeffs:
        A = gemm_nt(X, X)
        B = b * A + c * (A @ A)
        X = a * X + B @ X
    return X.T if transposed else X


def ns_nvfp4_step(X, a, b, c, rht_mask=None, adaptive46=False, trace=None):
    """One NVFP4 Newton–Schulz step (the three-line iteration of §3.4) from
    the iterate X (m x n, m <= n, any float dtype, widened exactly to
    float64), returning X' as float64:

        qX = Q_1x16(X [H]),   qX16 = Q_16x1([H^T] X),   A = qX qX^T
        qA = Q_1x16(A [H]),   qA16 = Q_16x1([H^T] A),   B = b A + c qA qA16
        qB = Q_1x16(B [H]),                             X' = a X + qB qX16

    ``rht_mask``: None, or the 16-bit sign mask of this step's random
    Hadamard transform H.  ``adaptive46``: every quantization picks M = 4 or
    6 per block (oracle/nvfp4.py).  ``trace``, if a list, receives a dict
    with the quantized operands and the float64 intermediates.
    """
    X = np.asarray(X, dtype=np.float64)
    if rht_mask is None:
        amax_x = tensor_amax(X)
        qX = quantize_rows(X, amax=amax_x, adaptive46=adaptive46)       # Q_1x16(X)
        qX16 = quantize_cols(X, amax=amax_x, adaptive46=adaptive46)     # Q_16x1(X), stored as X^T rows
    else:
        qX = quantize_rows(rht_rows(X, rht_mask), adaptive46=adaptive46)      # Q_1x16(X H)
        qX16 = quantize_cols(rht_cols(X, rht_mask), adaptive46=adaptive46)    # Q_16x1(H^T X)
    dX = dequantize_rows(qX)
    A = gemm_nt(dX, dX)                          # qX qX^T
    if rht_mask is None:
        qA = quantize_rows(A, adaptive46=adaptive46)                    # Q_1x16(A)
        qA16 = quantize_cols(A, adaptive46=adaptive46)                  # Q_16x1(A)
    else:
        qA = quantize_rows(rht_rows(A, rht_mask), adaptive46=adaptive46)      # Q_1x16(A H)
        qA16 = quantize_cols(rht_cols(A, rht_mask), adaptive46=adaptive46)    # Q_16x1(H^T A)
    B = b * A + c * (dequantize_rows(qA) @ dequantize_cols(qA16))
    qB = quantize_rows(B if rht_mask is None else rht_rows(B, rht_mask),
                       adaptive46=adaptive46)                           # Q_1x16(B [H])
    Xn = a * X + dequantize_rows(qB) @ dequantize_cols(qX16)
    if trace is not None:
        trace.append(dict(X=X, qX=qX, qX16=qX16, A=A, qA=qA, qA16=qA16,
                          B=B, qB=qB, X_next=Xn, coeffs=(a, b, c), rht_mask=rht_mask))
    return Xn


def ns_nvfp4(G, coeffs, clip=np.inf, eps=EPS, trace=None, rht_masks=None, adaptive46=False):
    """Newton–Schulz with NVFP4 operands for every product (§3.4 iteration):
    orientation, clip and normalisation, then ``ns_nvfp4_step`` once per
    coefficient triple.

    ``rht_masks``: None, or one 16-bit sign mask per step for the random
    Hadamard transform of that step.  ``adaptive46``: every quantization
    picks M = 4 or 6 per block (oracle/nvfp4.py).  ``trace``, if a list,
    receives one dict per step with the quantized operands and the float64
    intermediates (X before the step, A, B, X after).
    """
    Gt, transposed = _orient(G)
    X = clip_and_normalize(Gt, clip, eps)
    if rht_masks is not None and len(rht_masks) != len(coeffs):
        raise ValueError("one Hadamard mask per step")
    for it, (a, b, c) in enumerate(coeffs):
        X = ns_nvfp4_step(X, a, b, c, rht_mask=None if rht_masks is None else rht_masks[it],
                          adaptive46=adaptive46, trace=trace)
    return X.T if transposed else X


def ns_iteration_flops(m, n):
    """Algorithmic flops of one step on an m x n (m <= n) iterate.

    The two Gram products are symmetric, so only their upper triangle with
    the diagonal counts: m(m+1)n + m(m+1)m; the third product is 2 m^2 n.
    """
    m, n = min(m, n), max(m, n)
    return m * (m + 1) * n + m * (m + 1) * m + 2 * m * m * n
