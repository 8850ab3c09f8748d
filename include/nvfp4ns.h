/*
 * nvfp4ns.h — C ABI of the NVFP4 Newton–Schulz library for MI355X (gfx950).
 *
 * The operations follow "Full-Stack FP4: Stable LLM Pretraining with
 * Quantized Projections, Optimizers, and Attention" (arXiv 2607.04422):
 *   - the NVFP4 format of §2 "Preliminaries", paragraph "NVFP4 format":
 *     E2M1 element codes, one FP8 E4M3 scale s per 16-element block, one
 *     FP32 scale s_g per tensor, value = x_E2M1 * s * s_g;
 *   - the Root optimizer's Newton–Schulz iteration of §2 ("Root optimizer")
 *     in the NVFP4 form of §3.4 ("NVFP4 Root Optimizer", the three-line
 *     NVFP4 NS iteration), every quantization round-to-nearest.
 *
 * Conventions shared by every entry point
 *   - Pointers named x, codes, scales, G, out, ws, global_scale and the
 *     per-matrix arrays' elements are DEVICE pointers; coeffs, m, n, clip
 *     and the pointer arrays themselves are HOST memory.
 *   - Matrices are dense row-major with no padding.
 *   - Device arrays must be 16-byte aligned, and single device floats or
 *     words (global_scale, sg_p, sg_q, amax_out, ns_abs_quantile's out)
 *     4-byte aligned; hipMalloc and torch allocations are.  What a call
 *     writes (outputs and workspace) must not overlap what it reads or
 *     another of its outputs, except that nvfp4_gemm's addend may be out
 *     itself.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call
 *     only enqueues work on it and returns; nothing synchronises.  The
 *     caller owns all memory; the library allocates no device memory and
 *     keeps no data between calls (ns_orthogonalize_grouped and _ex keep
 *     only their streams; ns_orthogonalize_grouped_on keeps nothing).
 *   - Arguments are validated before anything is enqueued; a negative
 *     status means nothing was launched.  NS_ERR_HIP means a launch failed.
 *   - Data-dependent cases are defined, never errors: a NaN or infinity in
 *     a tensor makes its s_g NaN, all its scale bytes 0x7F and all its
 *     magnitude codes 0, and NaN propagates to every result; an all-zero
 *     tensor gives s_g = 0, zero scales and codes carrying only sign bits.
 *
 * NVFP4 storage (readings of the format paragraph, which prints the decode
 * rule only): s_g = RN_f32(amax / 2688); s = RNE_E4M3FN(amax_block /
 * (6 s_g)) of the exact quotient, saturating at 448 (0 if it rounds to 0);
 * code = sign | RNE_E2M1(|x| / (s s_g)) of the exact quotient, ties to the
 * even code, saturating at 6, magnitude 0 when s or s_g is 0.  Codes are
 * packed two per byte, element 2i in the low nibble; scales are E4M3FN
 * bytes, row-major [rows][cols/16].
 */
#ifndef NVFP4NS_H
#define NVFP4NS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NS_OK = 0,
  NS_ERR_ARG = -1,        /* null pointer, bad enum, k <= 0, clip NaN or <= 0, a
                             misaligned pointer, overlapping arrays */
  NS_ERR_SHAPE = -2,      /* a dimension <= 0 or not a multiple of 16, or a matrix of
                             2^31 or more elements in ns_orthogonalize / nvfp4_gemm */
  NS_ERR_WORKSPACE = -3,  /* ws is NULL or ws_bytes is below the required size */
  NS_ERR_HIP = -4         /* a kernel launch failed */
} ns_status;

typedef enum { NS_F32 = 0, NS_BF16 = 1 } ns_dtype;

/* NVFP4_ROWS: Q_1x16, blocks of 16 consecutive elements along each row.
 * NVFP4_COLS: Q_16x1, blocks of 16 down each column, stored as the Q_1x16
 * layout of the transpose (cols rows of rows/2 code bytes and rows/16
 * scale bytes). */
typedef enum { NVFP4_ROWS = 0, NVFP4_COLS = 1 } nvfp4_axis;

/* Workspace of nvfp4_quantize, nvfp4_quantize_rht and nvfp4_quantize_46, in
 * bytes (the partial tensor maxima: 2 KiB, independent of the shape). */
size_t nvfp4_quantize_workspace_bytes(int64_t rows, int64_t cols);

/*
 * nvfp4_quantize — Q_1x16 or Q_16x1 of a rows x cols matrix
 * (§2 "NVFP4 format"; the quantizers Q_1x16 / Q_16x1 of §3.4).
 *   x            [rows][cols] FP32 or BF16 (xt), read only.
 *   codes        out, rows*cols/2 bytes.
 *   scales       out, rows*cols/16 bytes.
 *   global_scale out, one float (s_g).
 *   ws           scratch of nvfp4_quantize_workspace_bytes(); contents on
 *                entry are ignored.
 * rows and cols must be positive multiples of 16.
 */
ns_status nvfp4_quantize(const void* x, ns_dtype xt, int64_t rows, int64_t cols,
                         nvfp4_axis axis, uint8_t* codes, uint8_t* scales,
                         float* global_scale, void* ws, size_t ws_bytes,
                         void* stream);

/*
 * nvfp4_quantize_noalloc — nvfp4_quantize without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  Its scratch, the
 * nvfp4_quantize_workspace_bytes() (2 KiB) of partial tensor maxima, lives in
 * a static device array of 2 KiB that each GPU the library runs on holds
 * until the process ends; the call allocates nothing.  Every call on one GPU
 * shares that array: calls that overlap on one GPU (concurrent streams)
 * race and must be ordered by the caller.  The array is cleared by a kernel
 * of each call.  Arguments, layouts, results and errors as nvfp4_quantize;
 * NS_ERR_WORKSPACE if a shape ever needed more scratch than the array holds
 * (none does: the scratch does not grow with the tensor); NS_ERR_HIP if the
 * array's device address cannot be obtained.
 */
ns_status nvfp4_quantize_noalloc(const void* x, ns_dtype xt, int64_t rows, int64_t cols,
                                 nvfp4_axis axis, uint8_t* codes, uint8_t* scales,
                                 float* global_scale, void* stream);

/*
 * nvfp4_quantize_rht — the quantizers of the §3.4 NS iteration with the
 * random Hadamard transform: Q_1x16(x H) (NVFP4_ROWS) or Q_16x1(H^T x)
 * (NVFP4_COLS, stored as the Q_1x16 layout of the transpose), where
 * H = H_16^r acts on every 16-block along the blocked axis.
 *   mask  H_16^r = diag(s) H_16 / 4 with H_16 the Sylvester Hadamard matrix,
 *         s_j = -1 where bit j of mask is set, else +1.
 *   The transformed values are computed in FP32 by the radix-2 butterfly:
 *   signs applied, then half-widths 1, 2, 4, 8, each pair (a, b) becoming
 *   (a + b, a - b) rounded to nearest even, then times 1/4.  The tensor
 *   scale s_g is that of the transformed tensor.
 * Other arguments, layout and errors as nvfp4_quantize.  nvfp4_dequantize
 * of the result returns the transformed tensor's approximation (the
 * transform is not undone).
 */
ns_status nvfp4_quantize_rht(const void* x, ns_dtype xt, int64_t rows, int64_t cols,
                             nvfp4_axis axis, uint16_t mask, uint8_t* codes, uint8_t* scales,
                             float* global_scale, void* ws, size_t ws_bytes, void* stream);

/*
 * nvfp4_quantize_46 — nvfp4_quantize with adaptive 4/6 block scaling, the
 * quantization the Root iteration uses (Full-Stack FP4 §3.4: RTN with
 * adaptive 4/6 scaling; §5: adaptive M = 4 / M = 6 block scaling of Four
 * Over Six).  Each block is encoded twice, with its maximum mapped to 6
 * (s = RNE_E4M3FN(amax_b / (6 s_g)), as nvfp4_quantize) and to 4
 * (s = RNE_E4M3FN(amax_b / (4 s_g)), saturating at 448), and keeps the
 * encoding whose squared error sum (x - q s s_g)^2 -- each operation rounded
 * in double, elements in order -- is smaller; M = 6 on ties.  s_g, the
 * layouts, the decode rule and the errors are those of nvfp4_quantize.
 */
ns_status nvfp4_quantize_46(const void* x, ns_dtype xt, int64_t rows, int64_t cols,
                            nvfp4_axis axis, uint8_t* codes, uint8_t* scales,
                            float* global_scale, void* ws, size_t ws_bytes, void* stream);

/*
 * nvfp4_dequantize — x_hat = x_E2M1 * s * s_g (§2 "NVFP4 format").
 * Inputs as written by nvfp4_quantize for the same rows, cols and axis;
 * out is [rows][cols] in the ORIGINAL orientation (an NVFP4_COLS tensor is
 * transposed back), FP32 or BF16 (ot), each value rounded once (RNE) from
 * the exact product.
 */
ns_status nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales,
                           const float* global_scale, int64_t rows, int64_t cols,
                           nvfp4_axis axis, void* out, ns_dtype ot, void* stream);

/*
 * nvfp4_gemm — one NVFP4 product of the §3.4 iteration, C = P * Q^T with
 * both operands in the Q_1x16 layout along the contraction axis K:
 *   P: codes_p [M][K/2], scales_p [M][K/16], s_g at sg_p (device float)
 *   Q: codes_q [N][K/2], scales_q [N][K/16], s_g at sg_q
 * and the epilogue
 *   out[i][j] = beta * addend[i][j] + alpha * s_gP * s_gQ * sum_k P_ik Q_jk
 * with products of dequantized values exact and FP32 accumulation.
 *   symmetric != 0: P and Q must be the same tensor (M == N); only the
 *     upper triangle is computed and mirrored, so out is exactly symmetric
 *     (the Gram products A = qX qX^T and qA qA^T).
 *   addend may be NULL when beta == 0, and may equal out.
 *   amax_out (device uint32, may be NULL): atomically maxed with the bit
 *     pattern of |out| (non-finite values count as NaN); the caller zeroes it.
 *   ws: device scratch of nvfp4_gemm_workspace_bytes(); it lets the tiles
 *     left over after an equal number per CU be split along K across
 *     workgroups (FP32 partials summed in a fixed order, so results do not
 *     depend on timing).  ws = NULL, ws_bytes = 0 runs every tile whole.
 *     Calls sharing one ws must not overlap.  ws must be ordinary device
 *     memory of the GPU that runs the call (hipMalloc, a torch tensor):
 *     within one launch the K-parts of a tile hand their partials to the
 *     part that sums them through ws, with stores and loads coherent at
 *     device scope and a device-scope counter, which relies on ws being
 *     device-local memory.
 * M, N, K must be positive multiples of 16.
 */
size_t nvfp4_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int symmetric);
ns_status nvfp4_gemm(const uint8_t* codes_p, const uint8_t* scales_p, const float* sg_p,
                     const uint8_t* codes_q, const uint8_t* scales_q, const float* sg_q,
                     int64_t M, int64_t N, int64_t K, int symmetric,
                     float alpha, float beta, const float* addend,
                     float* out, uint32_t* amax_out, void* ws, size_t ws_bytes,
                     void* stream);

/* Workspace of ns_orthogonalize for one m x n matrix, in bytes. */
size_t ns_workspace_bytes(int64_t m, int64_t n);

/*
 * ns_workspace_map — where ns_orthogonalize (and its _rht / _ex variants)
 * keeps the iteration's operands inside its workspace, as byte offsets from
 * ws.  An inspection aid (tests, debugging); the kernels need nothing from
 * the caller beyond ns_workspace_bytes().  The iterate is xm x xn with
 * xm = min(m, n), xn = max(m, n) (G^T when m > n).
 *   x                  FP32 X [xm][xn]
 *   a, b               FP32 A and B [xm][xm]; only the elements with
 *                      row <= col are written (A and B are symmetric)
 *   qx_codes/_scales   Q_1x16(X [H]): [xm][xn/2] codes, [xm][xn/16] scales
 *   qt_codes/_scales   Q_16x1([H^T] X) stored as rows of X^T: [xn][xm/2], [xn][xm/16]
 *   qa_codes/_scales   Q_1x16(A [H]): [xm][xm/2], [xm][xm/16]
 *   qb_codes/_scales   Q_1x16(B [H]): likewise
 *   global_scales      4 floats: s_g of qX, qA, qB, and of qX16 under the
 *                      transform (without it qX16 uses s_g of qX)
 * After a call of k steps these hold the last step's values: its input
 * iterate X_{k-1} in x when the call is untransposed with FP32 output (the
 * last product writes `out` directly), else X_k; the last step's A, B and
 * every quantized operand of that step.
 * Returns NS_ERR_SHAPE for shapes ns_orthogonalize rejects, NS_ERR_ARG for
 * map == NULL.
 */
typedef struct {
  int64_t xm, xn;
  size_t x, a, b;
  size_t qx_codes, qx_scales, qt_codes, qt_scales;
  size_t qa_codes, qa_scales, qb_codes, qb_scales;
  size_t global_scales;
  size_t total;             /* == ns_workspace_bytes(m, n) */
} ns_workspace_map;
ns_status ns_workspace_layout(int64_t m, int64_t n, ns_workspace_map* map);

/*
 * ns_orthogonalize — k NVFP4 Newton–Schulz steps (§2 "Root optimizer",
 * §3.4 NVFP4 NS iteration) on one matrix:
 *   X_0 = clamp(G, -clip, clip) / (||clamp(G)||_F + 1e-7)     (on G^T if m > n)
 *   for i < k:  A = qX qX^T;  B = b_i A + c_i qA qA^T;  X = a_i X + qB qX16
 *   out = X (transposed back if m > n)
 *   G      [m][n] FP32 or BF16 (gt), read only.
 *   coeffs HOST array of k triples (a_i, b_i, c_i).
 *   clip   > 0; +inf disables clipping.  NaN passes through the clamp.
 *   out    [m][n] FP32 or BF16 (ot); must not overlap G or ws.
 *   ws     device scratch of ns_workspace_bytes(m, n).
 */
ns_status ns_orthogonalize(const void* G, ns_dtype gt, int64_t m, int64_t n,
                           const float* coeffs, int k, float clip,
                           void* out, ns_dtype ot, void* ws, size_t ws_bytes,
                           void* stream);

/*
 * ns_orthogonalize_rht — ns_orthogonalize with the random Hadamard transform
 * of the §3.4 iteration on every quantized operand:
 *   qX = Q_1x16(X H), qX16 = Q_16x1(H^T X), A = qX qX^T
 *   qA = Q_1x16(A H), qA16 = Q_16x1(H^T A), B = b A + c qA qA16
 *   qB = Q_1x16(B H), X' = a X + qB qX16
 * with H = H_16^r of step i built from masks[i] as in nvfp4_quantize_rht
 * (H H^T = I, so each product still approximates the untransformed one).
 *   masks  HOST array of k 16-bit sign masks, one per step (not NULL).
 * X H and H^T X each take their own s_g.  Other arguments, workspace
 * (ns_workspace_bytes) and errors as ns_orthogonalize.
 */
ns_status ns_orthogonalize_rht(const void* G, ns_dtype gt, int64_t m, int64_t n,
                               const float* coeffs, int k, float clip, const uint16_t* masks,
                               void* out, ns_dtype ot, void* ws, size_t ws_bytes, void* stream);

/*
 * ns_abs_quantile — the q-quantile of |x| over `count` elements, the clip
 * threshold of the NVFP4 Root path (§3.4 "p99 outlier clipping"; App. F
 * Table 8 "Root quantile ratio 0.99"), read as an order statistic: the k-th
 * smallest magnitude, k = ceil(q * count) computed in double and clamped to
 * [1, count].  Magnitudes are ordered by their FP32 bit patterns with the
 * sign cleared (BF16 widened exactly); NaN and infinity count as NaN, above
 * every finite value, so a result that reaches them is NaN.
 *   x      device, `count` FP32 or BF16 (xt) values, read only.
 *   q      in (0, 1].
 *   out    device, one float (written when the enqueued work runs).
 *   ws     device scratch of ns_abs_quantile_workspace_bytes() (256 KiB).
 * count must be a positive multiple of 16 below 2^31.
 */
size_t ns_abs_quantile_workspace_bytes(void);
ns_status ns_abs_quantile(const void* x, ns_dtype xt, int64_t count, double q, float* out,
                          void* ws, size_t ws_bytes, void* stream);

/* Options of ns_orthogonalize_ex. */
typedef struct {
  float clip;               /* as in ns_orthogonalize; ignored when clip_quantile > 0 */
  double clip_quantile;     /* 0: use clip.  In (0, 1]: clip = the clip_quantile-quantile
                               of |G| (as ns_abs_quantile), found on the device */
  const uint16_t* rht_masks;/* NULL, or a HOST array of k masks (as ns_orthogonalize_rht) */
  int adaptive46;           /* nonzero: every quantization of the iteration uses adaptive
                               4/6 block scaling (as nvfp4_quantize_46) */
} ns_options;

/*
 * ns_orthogonalize_ex — ns_orthogonalize with the clip threshold taken on
 * the device as a quantile of |G|, the random Hadamard transform and/or
 * adaptive 4/6 block scaling, as set in `opt` (HOST pointer, not NULL).
 * NS_ERR_ARG for a clip_quantile outside {0} U (0, 1].  Workspace
 * ns_workspace_bytes(m, n); other arguments and errors as ns_orthogonalize.
 */
ns_status ns_orthogonalize_ex(const void* G, ns_dtype gt, int64_t m, int64_t n,
                              const float* coeffs, int k, const ns_options* opt, void* out,
                              ns_dtype ot, void* ws, size_t ws_bytes, void* stream);

/* Workspace of ns_orthogonalize_grouped for `count` matrices (host arrays m, n). */
size_t ns_grouped_workspace_bytes(int count, const int64_t* m, const int64_t* n);

/*
 * ns_orthogonalize_grouped — ns_orthogonalize on `count` independent
 * matrices with one coefficient schedule, as one batch of launches.
 *   G, out  HOST arrays of `count` device pointers.
 *   m, n    HOST arrays of shapes.   clip  HOST array of per-matrix clips.
 *   ws      device scratch of ns_grouped_workspace_bytes() (one part per
 *           matrix).
 * Matrices that share an iterate shape (min(m, n) x max(m, n), either
 * orientation) run in batches: each pass of a step is one launch for
 * several of them, each matrix on its single call's kernels and tile
 * schedule.  The batches run concurrently on up to four library-owned
 * streams of the current device (default priority, created on the first
 * grouped call and kept until the process ends), forked from `stream`
 * through an event and
 * joined back into it: the call is ordered on `stream` like any other and
 * can be captured into a graph.  Each result equals its single call's bit
 * for bit.  Calls that overlap on one device share the streams.
 */
ns_status ns_orthogonalize_grouped(int count, const void* const* G, const int64_t* m,
                                   const int64_t* n, ns_dtype gt, const float* coeffs,
                                   int k, const float* clip, void* const* out,
                                   ns_dtype ot, void* ws, size_t ws_bytes, void* stream);

/*
 * ns_orthogonalize_grouped_ex — ns_orthogonalize_grouped with the options of
 * ns_orthogonalize_ex shared by every matrix: with opt->clip_quantile > 0
 * each matrix is clipped at that quantile of its own |G| (clip may then be
 * NULL), else at clip[i]; opt->rht_masks (k masks) and opt->adaptive46
 * apply to every matrix.
 * Workspace ns_grouped_workspace_bytes(); concurrency and ordering as for
 * ns_orthogonalize_grouped.
 */
ns_status ns_orthogonalize_grouped_ex(int count, const void* const* G, const int64_t* m,
                                      const int64_t* n, ns_dtype gt, const float* coeffs, int k,
                                      const float* clip, const ns_options* opt, void* const* out,
                                      ns_dtype ot, void* ws, size_t ws_bytes, void* stream);

/*
 * ns_orthogonalize_grouped_on — ns_orthogonalize_grouped_ex on streams the
 * caller owns: the matrices run on streams[0 .. nstreams-1] (hipStream_t
 * values, 1 <= nstreams <= 16, none NULL), forked from `stream` through an
 * event and joined back into it, so the call is ordered on `stream` (work
 * already queued on the given streams runs before their share) and can be
 * captured into a graph.  The library keeps nothing between calls.  opt may
 * be NULL: clip[i] per matrix, no transform, no 4/6.  Results equal
 * ns_orthogonalize_grouped_ex's bit for bit.  NS_ERR_ARG for a bad stream
 * list; other arguments and errors as ns_orthogonalize_grouped_ex.
 */
ns_status ns_orthogonalize_grouped_on(int count, const void* const* G, const int64_t* m,
                                      const int64_t* n, ns_dtype gt, const float* coeffs, int k,
                                      const float* clip, const ns_options* opt, void* const* out,
                                      ns_dtype ot, void* ws, size_t ws_bytes,
                                      void* const* streams, int nstreams, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* NVFP4NS_H */
