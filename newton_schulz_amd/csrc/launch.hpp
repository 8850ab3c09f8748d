// Host-side launchers shared between the translation units of the library.
// Every launcher only enqueues on `s` and returns hipGetLastError().
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

enum class Dt : int { F32 = 0, BF16 = 1 };

// Per-block options of the tiled quantizer kernels.  With `on` every 16-block
// is multiplied by H^r = diag(s) H_16 / 4 before it is used, s_j = -1 where
// bit j of `mask` is set.  With `adaptive46` every block keeps the better of
// its M = 6 and M = 4 encodings (encode_block16_46 in nvfp4_device.hpp).
struct RhtArg {
  uint32_t on, mask, adaptive46;
};

// Words of one amax slot (kAmaxParts partials spaced one 128-byte line
// apart; see nvfp4_device.hpp).  Zeroed by the caller before a producer
// folds into it.
constexpr int kAmaxSlotWords = 16 * 32;

// ---- quantizer (quant.hip) -------------------------------------------------
// max |x| over n elements into *slot (atomic max on the bit pattern; the
// caller zeroes *slot first).  Non-finite values count as NaN.
hipError_t launch_amax(const void* x, Dt xt, int64_t n, uint32_t* slot, hipStream_t s);

// Q_1x16 of a rows x cols matrix, streaming one 16-block per thread.
// s_g comes from *amax_slot; it is also stored to *sg_out (may be null).
// *zero_slot (may be null) is set to 0 by the kernel.
hipError_t launch_quant_rows(const void* x, Dt xt, int64_t rows, int64_t cols,
                             const uint32_t* amax_slot, float* sg_out,
                             uint8_t* codes, uint8_t* scales, uint32_t* zero_slot,
                             hipStream_t s);

// Q_1x16 of a symmetric m x m FP32 matrix of which only the tiles on or
// above the diagonal (64 x 64) are read: the column blocks of tile (I, J)
// are the row blocks of tile (J, I).
// With batch > 1 the launch quantizes `batch` matrices, each with every
// pointer moved by b * bstride bytes from matrix 0's (the same holds for
// launch_quant_tiles).
// With rht_on every block (row blocks, and the column blocks that stand for
// the row blocks of the lower tiles) is first multiplied by H^r of rht_mask.
hipError_t launch_quant_sym_tiles(const float* x, int64_t m, const uint32_t* amax_slot,
                                  float* sg_out, uint8_t* codes, uint8_t* scales,
                                  uint32_t* zero_slot, bool adaptive46, hipStream_t s,
                                  int batch = 1, int64_t bstride = 0, uint32_t rht_on = 0,
                                  uint32_t rht_mask = 0);

// Q_1x16 and/or Q_16x1 of a rows x cols matrix through 64x64 LDS tiles, one
// read of x for both layouts.  Either output pair may be null.  The column
// layout takes its s_g from amax_c / sg_out_c when given (else the row
// ones); with rht.on every block is transformed first, with rht.adaptive46
// every block takes the better of its 4/6 encodings.
hipError_t launch_quant_tiles(const void* x, Dt xt, int64_t rows, int64_t cols,
                              const uint32_t* amax_slot, float* sg_out,
                              uint8_t* row_codes, uint8_t* row_scales,
                              uint8_t* col_codes, uint8_t* col_scales,
                              uint32_t* zero_slot, hipStream_t s,
                              const uint32_t* amax_c = nullptr, float* sg_out_c = nullptr,
                              RhtArg rht = RhtArg{0u, 0u, 0u}, int batch = 1,
                              int64_t bstride = 0);
// The first NS quantization fused with the normalisation: X = clamp(G) * inv
// (G is rows x cols, the X layout), written to X and quantized in both
// layouts in the same pass.  amax_slot must already hold max |X| (from
// launch_norm_finalize); the other arguments as launch_quant_tiles.
hipError_t launch_normalize_quant_tiles(const void* G, Dt gt, int64_t rows, int64_t cols, float clip,
                                        const float* clip_dev, const double* inv, float* X,
                                        const uint32_t* amax_slot, float* sg_out,
                                        uint8_t* row_codes, uint8_t* row_scales,
                                        uint8_t* col_codes, uint8_t* col_scales,
                                        uint32_t* zero_slot, bool adaptive46, hipStream_t s);
// Maxima of |x H^r| over the row blocks into slot_r and of |H^r^T x| over the
// column blocks into slot_c (either may be null); the caller zeroes them.
hipError_t launch_amax_tiles(const void* x, Dt xt, int64_t rows, int64_t cols, uint32_t* slot_r,
                             uint32_t* slot_c, RhtArg rht, hipStream_t s);
// Maximum of |A H^r| over the row blocks of a symmetric m x m FP32 matrix of
// which only the tiles on or above the diagonal are read, into slot (the
// caller zeroes it).
hipError_t launch_amax_sym_tiles(const float* x, int64_t m, uint32_t* slot, RhtArg rht,
                                 hipStream_t s);

// Exact dequantisation of a Q_1x16 tensor; rows x cols output.
hipError_t launch_dequant_rows(const uint8_t* codes, const uint8_t* scales, const float* sg,
                               int64_t rows, int64_t cols, void* out, Dt ot, hipStream_t s);
// Dequantisation of a Q_16x1 tensor stored as the Q_1x16 layout of its
// transpose (crows x ccols = cols x rows of the result); the output is the
// original rows x cols orientation.
hipError_t launch_dequant_cols(const uint8_t* codes, const uint8_t* scales, const float* sg,
                               int64_t rows, int64_t cols, void* out, Dt ot, hipStream_t s);

// ---- GEMM (gemm.hip) ------------------------------------------------------
struct GemmProblem {
  const uint8_t* codes_p; const uint8_t* scales_p; const float* sg_p;
  const uint8_t* codes_q; const uint8_t* scales_q; const float* sg_q;
  int64_t M, N, K;
  int symmetric;
  float alpha, beta;
  const float* addend;
  float* out;
  uint32_t* amax_out;
  int amax_parts;   // amax_out is an amax slot of partials (1) or one word (0)
  int upper_only;   // symmetric: tiles wholly above the diagonal skip their
                   // mirror (only row <= col and the diagonal tiles are stored)
  // `batch` problems of one shape in one launch: problem b's pointers (every
  // one above, and the GEMM workspace) are problem 0's plus b * batch_stride
  // bytes.  Each runs its single-problem schedule, so its result equals the
  // single launch's bit for bit.  Needs a fast-path plan.
  int batch = 1;
  int64_t batch_stride = 0;
  // batched: with out_each (a host array of `batch` pointers, at most
  // kMaxBatchOut) problem b writes its result to out_each[b] instead
  float* const* out_each = nullptr;
  // transformed maxima (128 x 128 tiles with 256-wide stages, tiles
  // unsplit or summed in the product kernel): with rht_on the
  // epilogue folds max |out H^r| over the row blocks into amax_out and
  // max |H^r^T out| over the column blocks into amax_out_c -- for a
  // symmetric product stored upper-only, the column blocks of a tile above
  // the diagonal stand for the row blocks of its mirror and go to amax_out
  // too -- instead of max |out|.  clear_a / clear_b (may be null): amax
  // slots that workgroup 0 zeroes first.
  int rht_on = 0;
  uint32_t rht_mask = 0;
  uint32_t* amax_out_c = nullptr;
  uint32_t* clear_a = nullptr;
  uint32_t* clear_b = nullptr;
};
constexpr int kMaxBatchOut = 32;

// Launch plan of one product: the fast path needs K % 128 == 0 and picks a
// tile shape from the tile count; tiles left over after an equal number per
// CU may be split along K, which needs a workspace of ws_bytes: a counter
// region of kGemmCounterBytes (one word per split tile) followed by the FP32
// partials.  With `fixup` the K-part that finishes last sums the partials
// inside the product kernel; otherwise a second kernel does.
constexpr size_t kGemmCounterBytes = 1024;
struct GemmPlan {
  bool fast;
  int cfg;                // fast-path config: 128 x 128 tiles with 256-wide row-line
                          // stages (0) or 128-wide ones (2), 64 x 128 tiles (3)
  int splits;             // K-parts of each leftover tile (1: none split)
  bool fixup;             // split tiles summed by their last K-part (no second kernel)
  int64_t TM, TN, tiles;
  int64_t units;          // workgroups of the product kernel
  int64_t split_tiles;    // tiles split into K-parts (0 when splits == 1)
  size_t partial_bytes, ws_bytes;
};
GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, bool symmetric, bool allow_split);
// Whether a product of this plan can fold transformed maxima (rht_on).
inline bool plan_rht_maxima(const GemmPlan& p) {
  return p.fast && p.cfg == 0 && (p.splits == 1 || p.fixup);
}
// ws: the plan's workspace.  The counters must be zero when the product
// starts; every launch leaves them zero.  zero_counters clears them first
// (a small kernel) for callers that cannot guarantee that.
hipError_t launch_gemm(const GemmProblem& g, const GemmPlan& p, void* ws, bool zero_counters,
                       hipStream_t s);

// ---- quantile of |x| (select.hip) ------------------------------------------
// State of the radix selection: bits of the answer fixed so far and the rank
// still sought among the keys that share them.
struct SelectState {
  uint32_t prefix, rank;
};
// Workspace of launch_abs_quantile, in bytes (independent of n).
size_t abs_quantile_workspace_bytes();
// *out = the rank-th smallest |x| (1-based, 1 <= rank <= n) over n elements,
// magnitudes ordered by FP32 bits, non-finite values last (as NaN).
hipError_t launch_abs_quantile(const void* x, Dt xt, int64_t n, uint32_t rank, float* out,
                               void* ws, hipStream_t s);

// ---- Newton–Schulz prologue / epilogue (ns.hip) ---------------------------
// Partial sums of clamp(G)^2 into part[0..kNormParts) and partial maxima of
// |clamp(G)| (as bit patterns, non-finite as NaN) into part_amax.  The clip
// is the device value *clip_dev when that is given, else `clip`.
constexpr int kNormParts = 1024;
hipError_t launch_norm_partials(const void* G, Dt gt, int64_t n, float clip, const float* clip_dev,
                                double* part, uint32_t* part_amax, hipStream_t s);
// inv[0] = 1 / (sqrt(sum part) + eps); zeroes the listed slots and the
// n_words words at `words` (may be null), then stores max |X_0| =
// RN_f32(max |clamp(G)| * inv) -- rounding is monotone, so this is the
// maximum of the normalised elements -- into the slot zero0.
hipError_t launch_norm_finalize(const double* part, const uint32_t* part_amax, double* inv,
                                uint32_t* zero0, uint32_t* zero1, uint32_t* zero2, uint32_t* words,
                                int n_words, hipStream_t s);
// X[m][n] = clamp(G) * inv (G is m x n, or n x m read transposed), amax into slot.
hipError_t launch_normalize(const void* G, Dt gt, int64_t m, int64_t n, bool transposed,
                            float clip, const float* clip_dev, const double* inv, float* X,
                            uint32_t* amax_slot, hipStream_t s);
// out = X (m x n), or X^T written as n x m when transposed; f32 or bf16.
hipError_t launch_write_out(const float* X, int64_t m, int64_t n, bool transposed, void* out,
                            Dt ot, hipStream_t s);

}  // namespace nvfp4
