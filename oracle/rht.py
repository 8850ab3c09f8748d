"""Random 16 x 16 Hadamard transform — oracle (test infrastructure only).

Source: Full-Stack FP4 (arXiv 2607.04422), §3.4 "NVFP4 Root Optimizer": in
the NVFP4 NS iteration every quantized operand is first multiplied along
the contraction axis by H = H_16^r, a fresh 16 x 16 random Hadamard
transform (X H and H^T X, A H and H^T A, B H); §3.1 and §3.3 describe the
same primitive as a randomised Hadamard matrix with a butterfly
implementation.

Readings (the pages name the transform but do not define it further):
* H_16 is the Sylvester Hadamard matrix of order 16,
  H_16[i][j] = (-1)^popcount(i & j); the random transform is
  H^r = diag(s) H_16 / 4 with a sign vector s in {+1, -1}^16, orthogonal.
  The caller supplies s as a 16-bit mask: bit j set means s_j = -1.
* "X H" acts on every 16-element block along the rows: columns
  16b .. 16b+15 of each row x become x H^r.  "H^T X" acts on every block of
  16 rows of each column; stored like every 16x1 operand as the rows of its
  transpose, that is (X^T H^r) again.
* The three products of one iteration share one H^r (the pages write one
  symbol); each iteration takes a fresh one (one mask per step).
* ``rht_rows`` is the FP64 product (what the NS oracle uses).
  ``rht_rows_f32`` is the FP32 evaluation the GPU quantizer performs, fixed
  here so that quantized codes can be compared bit for bit: signs applied,
  then the radix-2 butterfly with half-widths 1, 2, 4, 8, each pair
  (a, b) -> (a + b, a - b) rounded to nearest even in FP32, then a
  multiplication by 1/4.  It differs from the FP64 product by FP32
  rounding only.
"""
import numpy as np

BLOCK = 16


def hadamard16():
    """Sylvester Hadamard matrix of order 16 (entries +-1, int64)."""
    i = np.arange(BLOCK)
    pc = np.vectorize(lambda v: bin(v).count("1"))(i[:, None] & i[None, :])
    return np.where(pc % 2 == 0, 1, -1).astype(np.int64)


def sign_vector(mask):
    """s_j = -1 where bit j of the 16-bit mask is set, else +1."""
    bits = (int(mask) >> np.arange(BLOCK)) & 1
    return np.where(bits == 1, -1.0, 1.0)


def rht_matrix(mask):
    """H^r = diag(s) H_16 / 4 in float64 (exact: entries +-1/4)."""
    return sign_vector(mask)[:, None] * hadamard16().astype(np.float64) / 4.0


def rht_rows(t, mask):
    """Every 16-block along the rows of t times H^r, in float64."""
    t = np.asarray(t, dtype=np.float64)
    r, c = t.shape
    if c % BLOCK:
        raise ValueError("columns must be a multiple of 16")
    return (t.reshape(r, c // BLOCK, BLOCK) @ rht_matrix(mask)).reshape(r, c)


def rht_cols(t, mask):
    """H^r^T applied to every 16-block down the columns of t, in float64."""
    return rht_rows(np.asarray(t).T, mask).T


def rht_rows_f32(t, mask):
    """The FP32 butterfly evaluation of ``rht_rows`` (see the module notes)."""
    t = np.asarray(t, dtype=np.float32)
    r, c = t.shape
    if c % BLOCK:
        raise ValueError("columns must be a multiple of 16")
    v = t.reshape(r, c // BLOCK, BLOCK).copy()
    s = sign_vector(mask).astype(np.float32)
    v = v * s                                   # exact sign flips
    h = 1
    while h < BLOCK:
        out = v.copy()
        for i in range(BLOCK):
            if i & h:
                continue
            a, b = v[..., i], v[..., i + h]
            out[..., i] = a + b                 # float32 arithmetic
            out[..., i + h] = a - b
        v = out
        h *= 2
    return (v * np.float32(0.25)).reshape(r, c).astype(np.float32)
