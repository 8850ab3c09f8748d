// C ABI of the NVFP4 Newton–Schulz library (declared in include/nvfp4ns.h):
// argument validation, workspace planning and the launch sequence of the
// NVFP4 NS iteration of Full-Stack FP4 (arXiv 2607.04422), §3.4.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstddef>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <algorithm>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <utility>
#include <vector>

#include "../../include/nvfp4ns.h"
#include "launch.hpp"

using nvfp4::Dt;

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

inline bool dims_ok(int64_t a) { return a > 0 && a % 16 == 0; }
// tile-local offsets in the GEMM epilogue are 32-bit
constexpr int64_t kMaxElems = (int64_t)1 << 31;
inline bool dtype_ok(int d) { return d == NS_F32 || d == NS_BF16; }
inline size_t dtype_size(ns_dtype d) { return d == NS_F32 ? 4 : 2; }
inline hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// Device arrays must be 16-byte aligned (the kernels move 16-byte vectors);
// single floats and words 4-byte aligned.
inline bool al(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// A byte range of device memory; null or empty ranges overlap nothing.
struct Span {
  const void* p;
  size_t n;
};
// Whether the written range `o` shares a byte with any of `others`.
bool hits(Span o, std::initializer_list<Span> others) {
  if (!o.p || o.n == 0) return false;
  for (const Span& t : others)
    if (t.p && t.n && overlaps(o.p, o.n, t.p, t.n)) return true;
  return false;
}

// ---- concurrent problems of a grouped call --------------------------------
// The problems of a grouped call are independent (each has its own part of
// the workspace), so they run on kGroupStreams internal streams: the caller's
// stream forks into them through an event and joins them back, so the call
// stays ordered on the caller's stream and can be captured into a graph.
// Small problems then fill the GPU together, and one problem's tail kernels
// overlap another's.  The streams (default priority) are created once per
// device and kept until the process ends.
constexpr int kGroupStreams = 4;
constexpr int kMaxDevices = 64;

hipError_t group_streams(hipStream_t (&out)[kGroupStreams]) {
  static std::mutex mu;
  static hipStream_t streams[kMaxDevices][kGroupStreams];
  static bool made[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!made[dev]) {
    for (int i = 0; i < kGroupStreams; ++i) {
      e = hipStreamCreateWithFlags(&streams[dev][i], hipStreamNonBlocking);
      if (e != hipSuccess) return e;
    }
    made[dev] = true;
  }
  for (int i = 0; i < kGroupStreams; ++i) out[i] = streams[dev][i];
  return hipSuccess;
}

// ---- scratch of the allocation-free quantizer ------------------------------
// nvfp4_quantize_noalloc keeps the quantizer's scratch (the partial words of
// the tensor maximum, nvfp4_quantize_workspace_bytes()) in this array
// instead of a caller workspace.  Each device holds its own copy until the
// process ends; host code reaches it only through the address that
// hipGetSymbolAddress returns on that device (the array's name is a
// host-side stand-in).
constexpr size_t kNoAllocScratchBytes = 2048;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

// The device address of `scratch` on the current device, looked up once per
// device.  Null (and e set) if the lookup fails.
void* scratch_address(hipError_t& e) {
  static std::mutex mu;
  static void* addr[kMaxDevices];
  int dev = 0;
  e = hipGetDevice(&dev);
  if (e != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    e = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return nullptr;
    addr[dev] = p;
  }
  e = hipSuccess;
  return addr[dev];
}

// A failed launch returns NS_ERR_HIP; with NVFP4NS_DEBUG set in the
// environment the HIP error and the failing call are also printed.
inline ns_status hip_failed(hipError_t e, const char* what, int line) {
  if (std::getenv("NVFP4NS_DEBUG"))
    std::fprintf(stderr, "nvfp4ns: %s (%d) from %s, api.hip:%d\n", hipGetErrorString(e), (int)e, what,
                 line);
  return NS_ERR_HIP;
}

#define NS_TRY(call)                                          \
  do {                                                        \
    const hipError_t ns_e_ = (call);                          \
    if (ns_e_ != hipSuccess) return hip_failed(ns_e_, #call, __LINE__); \
  } while (0)

// Zero device words with a kernel launch (no memset node, so the sequence
// can be captured into a graph).
__global__ void zero_words_kernel(uint32_t* p, int n) {
  for (int i = (int)threadIdx.x; i < n; i += (int)blockDim.x) p[i] = 0u;
}

constexpr int kSlotWords = nvfp4::kAmaxSlotWords;

// ---- workspace of one Newton–Schulz problem (iterate is xm x xn, xm <= xn)
struct NsLayout {
  size_t X, A, B, qx_c, qx_s, qt_c, qt_s, qa_c, qa_s, qb_c, qb_s, sg, slot, part, part_amax, inv,
      clip, sel;
  size_t gemm_part, total;
  nvfp4::GemmPlan p1, p2, p3;
};

NsLayout ns_layout(int64_t m, int64_t n) {
  const size_t xm = (size_t)(m < n ? m : n), xn = (size_t)(m < n ? n : m);
  NsLayout L;
  L.p1 = nvfp4::plan_gemm((int64_t)xm, (int64_t)xm, (int64_t)xn, true, true);
  L.p2 = nvfp4::plan_gemm((int64_t)xm, (int64_t)xm, (int64_t)xm, true, true);
  L.p3 = nvfp4::plan_gemm((int64_t)xm, (int64_t)xn, (int64_t)xm, false, true);
  size_t part_bytes = 0;   // the products run one after another on one GEMM workspace
  for (const nvfp4::GemmPlan* p : {&L.p1, &L.p2, &L.p3})
    part_bytes = p->ws_bytes > part_bytes ? p->ws_bytes : part_bytes;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align_up(o + bytes); return at; };
  L.X = take(xm * xn * 4);
  L.A = take(xm * xm * 4);
  L.B = take(xm * xm * 4);
  L.qx_c = take(xm * xn / 2);
  L.qx_s = take(xm * xn / 16);
  L.qt_c = take(xm * xn / 2);
  L.qt_s = take(xm * xn / 16);
  L.qa_c = take(xm * xm / 2);
  L.qa_s = take(xm * xm / 16);
  L.qb_c = take(xm * xm / 2);
  L.qb_s = take(xm * xm / 16);
  L.sg = take(4 * sizeof(float));
  L.slot = take(4 * kSlotWords * sizeof(uint32_t));
  L.part = take(nvfp4::kNormParts * sizeof(double));
  L.part_amax = take(nvfp4::kNormParts * sizeof(uint32_t));
  L.inv = take(sizeof(double));
  L.clip = take(sizeof(float));
  L.sel = take(nvfp4::abs_quantile_workspace_bytes());
  L.gemm_part = take(part_bytes);
  L.total = o;
  return L;
}

// The iteration of §3.4.  With `masks` (k host masks) every quantized
// operand is first multiplied along K by that step's random Hadamard
// transform H^r: qX = Q_1x16(X H), qX16 = Q_16x1(H^T X) (own s_g),
// qA = Q_1x16(A H) (= Q_16x1(H^T A)^T since A is symmetric), qB = Q_1x16(B H);
// the maxima of the transformed tensors are folded into the epilogue of the
// product that writes each tensor (the first step's X, and every tensor of
// shapes whose products cannot, take a tiled maximum pass instead).
// 1-based rank of the q-quantile among n values: ceil(q n) in double,
// clamped to [1, n].
uint32_t quantile_rank(double q, int64_t n) {
  double k = std::ceil(q * (double)n);
  if (k < 1.0) k = 1.0;
  if (k > (double)n) k = (double)n;
  return (uint32_t)k;
}

ns_status ns_run(const void* G, ns_dtype gt, int64_t m, int64_t n, const float* coeffs, int k,
                 float clip, double clip_q, const uint16_t* masks, bool a46, void* out,
                 ns_dtype ot, uint8_t* ws, hipStream_t s) {
  const uint32_t o46 = a46 ? 1u : 0u;   // adaptive 4/6 on every quantization
  const NsLayout L = ns_layout(m, n);
  const bool tr = m > n;
  const int64_t xm = tr ? n : m, xn = tr ? m : n;
  float* X = reinterpret_cast<float*>(ws + L.X);
  float* A = reinterpret_cast<float*>(ws + L.A);
  float* B = reinterpret_cast<float*>(ws + L.B);
  float* sg = reinterpret_cast<float*>(ws + L.sg);
  uint32_t* slot = reinterpret_cast<uint32_t*>(ws + L.slot);
  double* part = reinterpret_cast<double*>(ws + L.part);
  uint32_t* part_amax = reinterpret_cast<uint32_t*>(ws + L.part_amax);
  double* inv = reinterpret_cast<double*>(ws + L.inv);
  uint32_t *slotX = slot, *slotA = slot + kSlotWords, *slotB = slot + 2 * kSlotWords,
           *slotXc = slot + 3 * kSlotWords;
  float *sgX = sg, *sgA = sg + 1, *sgB = sg + 2, *sgXc = sg + 3;

  // GEMM workspace; its split-tile counters are zeroed once per call (by
  // the norm pass below) and every product leaves them zero
  uint8_t* gws = ws + L.gemm_part;
  const bool any_split = L.total > L.gemm_part;

  // with clip_q > 0 the clip is the q-quantile of |G|, found on the device
  float* clipd = nullptr;
  if (clip_q > 0.0) {
    clipd = reinterpret_cast<float*>(ws + L.clip);
    NS_TRY(nvfp4::launch_abs_quantile(G, (Dt)gt, m * n, quantile_rank(clip_q, m * n), clipd,
                                      ws + L.sel, s));
  }
  NS_TRY(nvfp4::launch_norm_partials(G, (Dt)gt, m * n, clip, clipd, part, part_amax, s));
  NS_TRY(nvfp4::launch_norm_finalize(part, part_amax, inv, slotX, slotA, slotB,
                                     any_split ? reinterpret_cast<uint32_t*>(gws) : nullptr,
                                     (int)(nvfp4::kGemmCounterBytes / sizeof(uint32_t)), s));
  // untransformed and untransposed: the first quantization pass also
  // normalises G into X (max |X| is already in slotX)
  const bool fused = !masks && !tr;
  // transformed: the products fold the transformed maxima (all three plans
  // on 128 x 128 row-line tiles, unsplit or summed in the product kernel)
  const bool fused_rht = masks && nvfp4::plan_rht_maxima(L.p1) && nvfp4::plan_rht_maxima(L.p2) &&
                         nvfp4::plan_rht_maxima(L.p3);
  if (!fused) NS_TRY(nvfp4::launch_normalize(G, (Dt)gt, xm, xn, tr, clip, clipd, inv, X, slotX, s));

  for (int it = 0; it < k; ++it) {
    const float a = coeffs[3 * it], b = coeffs[3 * it + 1], c = coeffs[3 * it + 2];
    if (masks) {
      const nvfp4::RhtArg h{1u, (uint32_t)masks[it], o46};
      // fused: each product's epilogue folds the transformed maxima of its
      // output (the next quantizer's s_g) into that quantizer's slot, and
      // the passes clear the slots the next producer folds into, as in the
      // plain step; otherwise a maximum pass per quantized tensor
      const bool fx = fused_rht;
      if (!fx || it == 0) {
        zero_words_kernel<<<1, 256, 0, s>>>(slot, 4 * kSlotWords);
        NS_TRY(hipGetLastError());
        NS_TRY(nvfp4::launch_amax_tiles(X, Dt::F32, xm, xn, slotX, slotXc, h, s));
      }
      // the next step's X H and H^T X maxima come from this step's update
      // product (none after the last step)
      const bool next_max = fx && it + 1 < k;
      // qX = Q_1x16(X H), qX16 = Q_16x1(H^T X), each with its own s_g
      NS_TRY(nvfp4::launch_quant_tiles(X, Dt::F32, xm, xn, slotX, sgX, ws + L.qx_c, ws + L.qx_s,
                                       ws + L.qt_c, ws + L.qt_s, fx ? slotA : nullptr, s, slotXc,
                                       sgXc, h));
      // A = qX qX^T, upper triangle only (as without the transform)
      nvfp4::GemmProblem g1{ws + L.qx_c, ws + L.qx_s, sgX, ws + L.qx_c, ws + L.qx_s, sgX,
                            xm, xm, xn, 1, 1.0f, 0.0f, nullptr, A, fx ? slotA : nullptr, 1, 1};
      if (fx) {
        g1.rht_on = 1;
        g1.rht_mask = h.mask;
        g1.clear_a = next_max ? slotX : nullptr;    // read by this step's quantizer only
        g1.clear_b = next_max ? slotXc : nullptr;
      }
      NS_TRY(nvfp4::launch_gemm(g1, L.p1, gws, false, s));
      // qA = Q_1x16(A H), from the tiles on and above the diagonal: the row
      // blocks of a lower tile are the column blocks of its mirror
      if (!fx) NS_TRY(nvfp4::launch_amax_sym_tiles(A, xm, slotA, h, s));
      NS_TRY(nvfp4::launch_quant_sym_tiles(A, xm, slotA, sgA, ws + L.qa_c, ws + L.qa_s,
                                           fx ? slotB : nullptr, a46, s, 1, 0, 1u, h.mask));
      nvfp4::GemmProblem g2{ws + L.qa_c, ws + L.qa_s, sgA, ws + L.qa_c, ws + L.qa_s, sgA,
                            xm, xm, xm, 1, c, b, A, B, fx ? slotB : nullptr, 1, 1};
      if (fx) {
        g2.rht_on = 1;
        g2.rht_mask = h.mask;
      }
      NS_TRY(nvfp4::launch_gemm(g2, L.p2, gws, false, s));
      // qB = Q_1x16(B H), likewise
      if (!fx) NS_TRY(nvfp4::launch_amax_sym_tiles(B, xm, slotB, h, s));
      NS_TRY(nvfp4::launch_quant_sym_tiles(B, xm, slotB, sgB, ws + L.qb_c, ws + L.qb_s, nullptr,
                                           a46, s, 1, 0, 1u, h.mask));
      const bool direct = it == k - 1 && !tr && ot == NS_F32;
      nvfp4::GemmProblem g3{ws + L.qb_c, ws + L.qb_s, sgB, ws + L.qt_c, ws + L.qt_s, sgXc,
                            xm, xn, xm, 0, 1.0f, a, X, direct ? static_cast<float*>(out) : X,
                            nullptr, 0};
      if (next_max) {
        // X' H (rows) and H'^T X' (columns) under the next step's transform
        g3.rht_on = 1;
        g3.rht_mask = (uint32_t)masks[it + 1];
        g3.amax_out = slotX;
        g3.amax_out_c = slotXc;
        g3.amax_parts = 1;
      }
      NS_TRY(nvfp4::launch_gemm(g3, L.p3, gws, false, s));
      if (direct) return NS_OK;
      continue;
    }
    // qX = Q_1x16(X) and qX16 = Q_16x1(X) (stored as rows of X^T), one s_g
    if (fused && it == 0)
      NS_TRY(nvfp4::launch_normalize_quant_tiles(G, (Dt)gt, xm, xn, clip, clipd, inv, X, slotX, sgX,
                                                 ws + L.qx_c, ws + L.qx_s, ws + L.qt_c,
                                                 ws + L.qt_s, slotA, a46, s));
    else
      NS_TRY(nvfp4::launch_quant_tiles(X, Dt::F32, xm, xn, slotX, sgX, ws + L.qx_c, ws + L.qx_s,
                                       ws + L.qt_c, ws + L.qt_s, slotA, s, nullptr, nullptr,
                                       nvfp4::RhtArg{0u, 0u, o46}));
    // A = qX qX^T (symmetric, K = xn); only its upper triangle is stored
    // (and the diagonal tiles whole), which is all that its quantizer and
    // the addend of the next product read
    nvfp4::GemmProblem g1{ws + L.qx_c, ws + L.qx_s, sgX, ws + L.qx_c, ws + L.qx_s, sgX,
                          xm, xm, xn, 1, 1.0f, 0.0f, nullptr, A, slotA, 1, 1};
    NS_TRY(nvfp4::launch_gemm(g1, L.p1, gws, false, s));
    // qA = Q_1x16(A) from the tiles on and above the diagonal (A is exactly
    // symmetric: the rows of a lower tile are the columns of an upper one,
    // and Q_16x1(A) = qA^T)
    NS_TRY(nvfp4::launch_quant_sym_tiles(A, xm, slotA, sgA, ws + L.qa_c, ws + L.qa_s, slotB, a46,
                                         s));
    // B = b A + c qA qA^T (symmetric, K = xm), upper triangle as for A
    nvfp4::GemmProblem g2{ws + L.qa_c, ws + L.qa_s, sgA, ws + L.qa_c, ws + L.qa_s, sgA,
                          xm, xm, xm, 1, c, b, A, B, slotB, 1, 1};
    NS_TRY(nvfp4::launch_gemm(g2, L.p2, gws, false, s));
    // qB = Q_1x16(B), likewise
    NS_TRY(nvfp4::launch_quant_sym_tiles(B, xm, slotB, sgB, ws + L.qb_c, ws + L.qb_s, slotX, a46,
                                         s));
    // X' = a X + qB qX16 (K = xm), in place; the last step of an FP32,
    // untransposed call writes straight into `out` (no copy pass)
    const bool direct = it == k - 1 && !tr && ot == NS_F32;
    float* dst = direct ? static_cast<float*>(out) : X;
    nvfp4::GemmProblem g3{ws + L.qb_c, ws + L.qb_s, sgB, ws + L.qt_c, ws + L.qt_s, sgX,
                          xm, xn, xm, 0, 1.0f, a, X, dst, direct ? nullptr : slotX, 1};
    NS_TRY(nvfp4::launch_gemm(g3, L.p3, gws, false, s));
    if (direct) return NS_OK;
  }
  NS_TRY(nvfp4::launch_write_out(X, xm, xn, tr, out, (Dt)ot, s));
  return NS_OK;
}

// ns_run for `count` matrices whose iterates share one shape xm x xn
// (matrix j is G[j], m[j] x n[j], transposed when m > n),
// with workspace regions of ns_layout size at ws + j * stride.  The passes
// done once per call (clip quantile, norm, first quantization, write-out)
// run per matrix; every pass of a step runs once for all of them, one
// launch per phase with grid row y = matrix.  Each matrix runs the kernels
// and tile schedules of its own ns_run in the same order, so every result
// equals ns_run's bit for bit.  All three products need fast-path plans,
// and with the transform (`masks`) plans that fold the transformed maxima
// (batchable).  The transformed step's first maximum pass runs per matrix.
ns_status ns_run_batch(int count, const void* const* G, ns_dtype gt, const int64_t* m,
                       const int64_t* n, const float* coeffs, int k, const float* clip,
                       double clip_q, const uint16_t* masks, bool a46, void* const* out,
                       ns_dtype ot, uint8_t* ws, size_t stride, hipStream_t s) {
  const uint32_t o46 = a46 ? 1u : 0u;
  const NsLayout L = ns_layout(m[0], n[0]);
  const int64_t xm = m[0] < n[0] ? m[0] : n[0], xn = m[0] < n[0] ? n[0] : m[0];
  const int64_t bs = (int64_t)stride;
  auto at = [&](int j, size_t off) { return ws + (size_t)j * stride + off; };
  const bool any_split = L.total > L.gemm_part;

  // once per matrix: clip, norm, and the first quantization of X
  for (int j = 0; j < count; ++j) {
    const bool tr = m[j] > n[j];
    float* X = reinterpret_cast<float*>(at(j, L.X));
    uint32_t* slot = reinterpret_cast<uint32_t*>(at(j, L.slot));
    float* sg = reinterpret_cast<float*>(at(j, L.sg));
    double* part = reinterpret_cast<double*>(at(j, L.part));
    uint32_t* part_amax = reinterpret_cast<uint32_t*>(at(j, L.part_amax));
    double* inv = reinterpret_cast<double*>(at(j, L.inv));
    uint8_t* gws = at(j, L.gemm_part);
    float* clipd = nullptr;
    if (clip_q > 0.0) {
      clipd = reinterpret_cast<float*>(at(j, L.clip));
      NS_TRY(nvfp4::launch_abs_quantile(G[j], (Dt)gt, m[j] * n[j],
                                        quantile_rank(clip_q, m[j] * n[j]), clipd, at(j, L.sel), s));
    }
    NS_TRY(nvfp4::launch_norm_partials(G[j], (Dt)gt, m[j] * n[j], clip[j], clipd, part, part_amax,
                                       s));
    NS_TRY(nvfp4::launch_norm_finalize(part, part_amax, inv, slot, slot + kSlotWords,
                                       slot + 2 * kSlotWords,
                                       any_split ? reinterpret_cast<uint32_t*>(gws) : nullptr,
                                       (int)(nvfp4::kGemmCounterBytes / sizeof(uint32_t)), s));
    if (masks) {
      // as ns_run's transformed call: X0, then the maxima of X0 H and H^T X0
      NS_TRY(nvfp4::launch_normalize(G[j], (Dt)gt, xm, xn, tr, clip[j], clipd, inv, X, slot, s));
      zero_words_kernel<<<1, 256, 0, s>>>(slot, 4 * kSlotWords);
      NS_TRY(hipGetLastError());
      NS_TRY(nvfp4::launch_amax_tiles(X, Dt::F32, xm, xn, slot, slot + 3 * kSlotWords,
                                      nvfp4::RhtArg{1u, (uint32_t)masks[0], o46}, s));
    } else if (tr) {
      NS_TRY(nvfp4::launch_normalize(G[j], (Dt)gt, xm, xn, true, clip[j], clipd, inv, X, slot, s));
      NS_TRY(nvfp4::launch_quant_tiles(X, Dt::F32, xm, xn, slot, sg, at(j, L.qx_c), at(j, L.qx_s),
                                       at(j, L.qt_c), at(j, L.qt_s), slot + kSlotWords, s, nullptr,
                                       nullptr, nvfp4::RhtArg{0u, 0u, o46}));
    } else {
      NS_TRY(nvfp4::launch_normalize_quant_tiles(G[j], (Dt)gt, xm, xn, clip[j], clipd, inv, X, slot,
                                                 sg, at(j, L.qx_c), at(j, L.qx_s), at(j, L.qt_c),
                                                 at(j, L.qt_s), slot + kSlotWords, a46, s));
    }
  }

  // the steps, each phase one launch for every matrix (matrix 0's pointers)
  float* X = reinterpret_cast<float*>(at(0, L.X));
  float* A = reinterpret_cast<float*>(at(0, L.A));
  float* B = reinterpret_cast<float*>(at(0, L.B));
  float* sg = reinterpret_cast<float*>(at(0, L.sg));
  uint32_t* slot = reinterpret_cast<uint32_t*>(at(0, L.slot));
  uint32_t *slotX = slot, *slotA = slot + kSlotWords, *slotB = slot + 2 * kSlotWords,
           *slotXc = slot + 3 * kSlotWords;
  float *sgX = sg, *sgA = sg + 1, *sgB = sg + 2, *sgXc = sg + 3;
  uint8_t* gws = at(0, L.gemm_part);
  // per matrix: where its last update product writes (its output, or X)
  std::vector<float*> direct((size_t)count);
  for (int j = 0; j < count; ++j)
    direct[(size_t)j] = (m[j] <= n[j] && ot == NS_F32) ? static_cast<float*>(out[j])
                                                       : reinterpret_cast<float*>(at(j, L.X));
  for (int it = 0; it < k; ++it) {
    const float a = coeffs[3 * it], b = coeffs[3 * it + 1], c = coeffs[3 * it + 2];
    if (masks) {
      // ns_run's transformed step, each phase one launch for every matrix
      const nvfp4::RhtArg h{1u, (uint32_t)masks[it], o46};
      const bool next_max = it + 1 < k;
      NS_TRY(nvfp4::launch_quant_tiles(X, Dt::F32, xm, xn, slotX, sgX, at(0, L.qx_c), at(0, L.qx_s),
                                       at(0, L.qt_c), at(0, L.qt_s), slotA, s, slotXc, sgXc, h,
                                       count, bs));
      nvfp4::GemmProblem g1{at(0, L.qx_c), at(0, L.qx_s), sgX, at(0, L.qx_c), at(0, L.qx_s), sgX,
                            xm, xm, xn, 1, 1.0f, 0.0f, nullptr, A, slotA, 1, 1, count, bs};
      g1.rht_on = 1;
      g1.rht_mask = h.mask;
      g1.clear_a = next_max ? slotX : nullptr;
      g1.clear_b = next_max ? slotXc : nullptr;
      NS_TRY(nvfp4::launch_gemm(g1, L.p1, gws, false, s));
      NS_TRY(nvfp4::launch_quant_sym_tiles(A, xm, slotA, sgA, at(0, L.qa_c), at(0, L.qa_s), slotB,
                                           a46, s, count, bs, 1u, h.mask));
      nvfp4::GemmProblem g2{at(0, L.qa_c), at(0, L.qa_s), sgA, at(0, L.qa_c), at(0, L.qa_s), sgA,
                            xm, xm, xm, 1, c, b, A, B, slotB, 1, 1, count, bs};
      g2.rht_on = 1;
      g2.rht_mask = h.mask;
      NS_TRY(nvfp4::launch_gemm(g2, L.p2, gws, false, s));
      NS_TRY(nvfp4::launch_quant_sym_tiles(B, xm, slotB, sgB, at(0, L.qb_c), at(0, L.qb_s), nullptr,
                                           a46, s, count, bs, 1u, h.mask));
      nvfp4::GemmProblem g3{at(0, L.qb_c), at(0, L.qb_s), sgB, at(0, L.qt_c), at(0, L.qt_s), sgXc,
                            xm, xn, xm, 0, 1.0f, a, X, X, nullptr, 1, 0, count, bs};
      if (next_max) {
        g3.rht_on = 1;
        g3.rht_mask = (uint32_t)masks[it + 1];
        g3.amax_out = slotX;
        g3.amax_out_c = slotXc;
      }
      if (it == k - 1) g3.out_each = direct.data();
      NS_TRY(nvfp4::launch_gemm(g3, L.p3, gws, false, s));
      continue;
    }
    if (it > 0)
      NS_TRY(nvfp4::launch_quant_tiles(X, Dt::F32, xm, xn, slotX, sgX, at(0, L.qx_c), at(0, L.qx_s),
                                       at(0, L.qt_c), at(0, L.qt_s), slotA, s, nullptr, nullptr,
                                       nvfp4::RhtArg{0u, 0u, o46}, count, bs));
    nvfp4::GemmProblem g1{at(0, L.qx_c), at(0, L.qx_s), sgX, at(0, L.qx_c), at(0, L.qx_s), sgX,
                          xm, xm, xn, 1, 1.0f, 0.0f, nullptr, A, slotA, 1, 1, count, bs};
    NS_TRY(nvfp4::launch_gemm(g1, L.p1, gws, false, s));
    NS_TRY(nvfp4::launch_quant_sym_tiles(A, xm, slotA, sgA, at(0, L.qa_c), at(0, L.qa_s), slotB,
                                         a46, s, count, bs));
    nvfp4::GemmProblem g2{at(0, L.qa_c), at(0, L.qa_s), sgA, at(0, L.qa_c), at(0, L.qa_s), sgA,
                          xm, xm, xm, 1, c, b, A, B, slotB, 1, 1, count, bs};
    NS_TRY(nvfp4::launch_gemm(g2, L.p2, gws, false, s));
    NS_TRY(nvfp4::launch_quant_sym_tiles(B, xm, slotB, sgB, at(0, L.qb_c), at(0, L.qb_s), slotX,
                                         a46, s, count, bs));
    nvfp4::GemmProblem g3{at(0, L.qb_c), at(0, L.qb_s), sgB, at(0, L.qt_c), at(0, L.qt_s), sgX,
                          xm, xn, xm, 0, 1.0f, a, X, X, slotX, 1, 0, count, bs};
    // the last step of an FP32, untransposed matrix writes straight into
    // its output, as its single call does (the others keep X in place)
    if (it == k - 1) g3.out_each = direct.data();
    NS_TRY(nvfp4::launch_gemm(g3, L.p3, gws, false, s));
  }
  for (int j = 0; j < count; ++j)   // k >= 1 (validated): the others hold X_k in X
    if (direct[(size_t)j] != out[j])
      NS_TRY(nvfp4::launch_write_out(reinterpret_cast<float*>(at(j, L.X)), xm, xn, m[j] > n[j],
                                     out[j], (Dt)ot, s));
  return NS_OK;
}

// A batch needs every product on the fast path (K a multiple of 128), and
// with the transform (rht) products that fold the transformed maxima.
bool batchable(int64_t m, int64_t n, bool rht) {
  const NsLayout L = ns_layout(m, n);
  if (rht)
    return nvfp4::plan_rht_maxima(L.p1) && nvfp4::plan_rht_maxima(L.p2) &&
           nvfp4::plan_rht_maxima(L.p3);
  return L.p1.fast && L.p2.fast && L.p3.fast;
}

ns_status validate_ns(const void* G, int gt, int64_t m, int64_t n, const float* coeffs, int k,
                      float clip, const void* out, int ot) {
  if (!G || !out || !coeffs || k <= 0 || !dtype_ok(gt) || !dtype_ok(ot)) return NS_ERR_ARG;
  if (std::isnan(clip) || !(clip > 0.0f)) return NS_ERR_ARG;
  if (!dims_ok(m) || !dims_ok(n)) return NS_ERR_SHAPE;
  if (m * n >= kMaxElems) return NS_ERR_SHAPE;
  for (int i = 0; i < 3 * k; ++i)
    if (!std::isfinite(coeffs[i])) return NS_ERR_ARG;
  if (!al(G, 16) || !al(out, 16)) return NS_ERR_ARG;
  if (overlaps(G, (size_t)(m * n) * dtype_size((ns_dtype)gt), out,
               (size_t)(m * n) * dtype_size((ns_dtype)ot)))
    return NS_ERR_ARG;
  return NS_OK;
}

// The workspace of one NS problem: 16-byte aligned, clear of G and out.
ns_status check_ns_ws(const void* G, int gt, int64_t m, int64_t n, const void* out, int ot,
                      const void* ws, size_t ws_bytes) {
  if (!al(ws, 16)) return NS_ERR_ARG;
  const size_t e = (size_t)(m * n);
  if (hits(Span{ws, ws_bytes}, {Span{G, e * dtype_size((ns_dtype)gt)},
                                Span{out, e * dtype_size((ns_dtype)ot)}}))
    return NS_ERR_ARG;
  return NS_OK;
}

// Arguments shared by the three quantizer entry points.
ns_status validate_quant(const void* x, int xt, int64_t rows, int64_t cols, int axis,
                         const void* codes, const void* scales, const void* global_scale,
                         const void* ws, size_t ws_bytes) {
  if (!x || !codes || !scales || !global_scale || !dtype_ok(xt) ||
      (axis != NVFP4_ROWS && axis != NVFP4_COLS))
    return NS_ERR_ARG;
  if (!dims_ok(rows) || !dims_ok(cols)) return NS_ERR_SHAPE;
  if (!ws || ws_bytes < align_up(kSlotWords * sizeof(uint32_t))) return NS_ERR_WORKSPACE;
  if (!al(x, 16) || !al(codes, 16) || !al(scales, 16) || !al(ws, 16) || !al(global_scale, 4))
    return NS_ERR_ARG;
  const size_t e = (size_t)(rows * cols);
  const Span X{x, e * dtype_size((ns_dtype)xt)}, C{codes, e / 2}, S{scales, e / 16},
      Gs{global_scale, sizeof(float)}, W{ws, ws_bytes};
  if (hits(C, {X, S, Gs, W}) || hits(S, {X, Gs, W}) || hits(Gs, {X, W}) || hits(W, {X}))
    return NS_ERR_ARG;
  return NS_OK;
}

}  // namespace

extern "C" {

size_t nvfp4_quantize_workspace_bytes(int64_t, int64_t) { return align_up(kSlotWords * sizeof(uint32_t)); }

ns_status nvfp4_quantize(const void* x, ns_dtype xt, int64_t rows, int64_t cols, nvfp4_axis axis,
                         uint8_t* codes, uint8_t* scales, float* global_scale, void* ws,
                         size_t ws_bytes, void* stream) {
  const ns_status st =
      validate_quant(x, xt, rows, cols, axis, codes, scales, global_scale, ws, ws_bytes);
  if (st != NS_OK) return st;
  hipStream_t s = as_stream(stream);
  uint32_t* slot = static_cast<uint32_t*>(ws);
  zero_words_kernel<<<1, 256, 0, s>>>(slot, kSlotWords);
  NS_TRY(hipGetLastError());
  NS_TRY(nvfp4::launch_amax(x, (Dt)xt, rows * cols, slot, s));
  if (axis == NVFP4_ROWS)
    NS_TRY(nvfp4::launch_quant_rows(x, (Dt)xt, rows, cols, slot, global_scale, codes, scales,
                                    nullptr, s));
  else
    NS_TRY(nvfp4::launch_quant_tiles(x, (Dt)xt, rows, cols, slot, global_scale, nullptr, nullptr,
                                     codes, scales, nullptr, s));
  return NS_OK;
}

ns_status nvfp4_quantize_noalloc(const void* x, ns_dtype xt, int64_t rows, int64_t cols,
                                 nvfp4_axis axis, uint8_t* codes, uint8_t* scales,
                                 float* global_scale, void* stream) {
  // the scratch this call needs must fit the static array (it does for every
  // shape: the quantizer's scratch does not grow with the tensor)
  if (nvfp4_quantize_workspace_bytes(rows, cols) > kNoAllocScratchBytes) {
    if (std::getenv("NVFP4NS_DEBUG"))
      std::fprintf(stderr, "nvfp4ns: nvfp4_quantize_noalloc needs more than its %zu-byte scratch\n",
                   kNoAllocScratchBytes);
    return NS_ERR_WORKSPACE;
  }
  hipError_t e = hipSuccess;
  void* ws = scratch_address(e);
  if (!ws) return hip_failed(e, "hipGetSymbolAddress(scratch)", __LINE__);
  return nvfp4_quantize(x, xt, rows, cols, axis, codes, scales, global_scale, ws,
                        kNoAllocScratchBytes, stream);
}

ns_status nvfp4_quantize_rht(const void* x, ns_dtype xt, int64_t rows, int64_t cols,
                             nvfp4_axis axis, uint16_t mask, uint8_t* codes, uint8_t* scales,
                             float* global_scale, void* ws, size_t ws_bytes, void* stream) {
  const ns_status st =
      validate_quant(x, xt, rows, cols, axis, codes, scales, global_scale, ws, ws_bytes);
  if (st != NS_OK) return st;
  hipStream_t s = as_stream(stream);
  uint32_t* slot = static_cast<uint32_t*>(ws);
  const nvfp4::RhtArg h{1u, (uint32_t)mask, 0u};
  zero_words_kernel<<<1, 256, 0, s>>>(slot, kSlotWords);
  NS_TRY(hipGetLastError());
  if (axis == NVFP4_ROWS) {
    NS_TRY(nvfp4::launch_amax_tiles(x, (Dt)xt, rows, cols, slot, nullptr, h, s));
    NS_TRY(nvfp4::launch_quant_tiles(x, (Dt)xt, rows, cols, slot, global_scale, codes, scales,
                                     nullptr, nullptr, nullptr, s, nullptr, nullptr, h));
  } else {
    NS_TRY(nvfp4::launch_amax_tiles(x, (Dt)xt, rows, cols, nullptr, slot, h, s));
    NS_TRY(nvfp4::launch_quant_tiles(x, (Dt)xt, rows, cols, slot, global_scale, nullptr, nullptr,
                                     codes, scales, nullptr, s, nullptr, nullptr, h));
  }
  return NS_OK;
}

ns_status nvfp4_quantize_46(const void* x, ns_dtype xt, int64_t rows, int64_t cols, nvfp4_axis axis,
                            uint8_t* codes, uint8_t* scales, float* global_scale, void* ws,
                            size_t ws_bytes, void* stream) {
  const ns_status st =
      validate_quant(x, xt, rows, cols, axis, codes, scales, global_scale, ws, ws_bytes);
  if (st != NS_OK) return st;
  hipStream_t s = as_stream(stream);
  uint32_t* slot = static_cast<uint32_t*>(ws);
  const nvfp4::RhtArg o{0u, 0u, 1u};
  zero_words_kernel<<<1, 256, 0, s>>>(slot, kSlotWords);
  NS_TRY(hipGetLastError());
  NS_TRY(nvfp4::launch_amax(x, (Dt)xt, rows * cols, slot, s));
  if (axis == NVFP4_ROWS)
    NS_TRY(nvfp4::launch_quant_tiles(x, (Dt)xt, rows, cols, slot, global_scale, codes, scales,
                                     nullptr, nullptr, nullptr, s, nullptr, nullptr, o));
  else
    NS_TRY(nvfp4::launch_quant_tiles(x, (Dt)xt, rows, cols, slot, global_scale, nullptr, nullptr,
                                     codes, scales, nullptr, s, nullptr, nullptr, o));
  return NS_OK;
}

ns_status nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, const float* global_scale,
                           int64_t rows, int64_t cols, nvfp4_axis axis, void* out, ns_dtype ot,
                           void* stream) {
  if (!codes || !scales || !global_scale || !out || !dtype_ok(ot) ||
      (axis != NVFP4_ROWS && axis != NVFP4_COLS))
    return NS_ERR_ARG;
  if (!dims_ok(rows) || !dims_ok(cols)) return NS_ERR_SHAPE;
  if (!al(codes, 16) || !al(scales, 16) || !al(out, 16) || !al(global_scale, 4)) return NS_ERR_ARG;
  const size_t e = (size_t)(rows * cols);
  if (hits(Span{out, e * dtype_size(ot)},
           {Span{codes, e / 2}, Span{scales, e / 16}, Span{global_scale, sizeof(float)}}))
    return NS_ERR_ARG;
  hipStream_t s = as_stream(stream);
  if (axis == NVFP4_ROWS)
    NS_TRY(nvfp4::launch_dequant_rows(codes, scales, global_scale, rows, cols, out, (Dt)ot, s));
  else
    NS_TRY(nvfp4::launch_dequant_cols(codes, scales, global_scale, rows, cols, out, (Dt)ot, s));
  return NS_OK;
}

size_t nvfp4_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int symmetric) {
  if (!dims_ok(M) || !dims_ok(N) || !dims_ok(K)) return 0;
  return nvfp4::plan_gemm(M, N, K, symmetric != 0, true).ws_bytes;
}

ns_status nvfp4_gemm(const uint8_t* codes_p, const uint8_t* scales_p, const float* sg_p,
                     const uint8_t* codes_q, const uint8_t* scales_q, const float* sg_q,
                     int64_t M, int64_t N, int64_t K, int symmetric, float alpha, float beta,
                     const float* addend, float* out, uint32_t* amax_out, void* ws,
                     size_t ws_bytes, void* stream) {
  if (!codes_p || !scales_p || !sg_p || !codes_q || !scales_q || !sg_q || !out) return NS_ERR_ARG;
  if (beta != 0.0f && !addend) return NS_ERR_ARG;
  if (!std::isfinite(alpha) || !std::isfinite(beta)) return NS_ERR_ARG;
  if (!dims_ok(M) || !dims_ok(N) || !dims_ok(K)) return NS_ERR_SHAPE;
  if (M * N >= kMaxElems || M * K >= kMaxElems || N * K >= kMaxElems) return NS_ERR_SHAPE;
  if (symmetric && (M != N || codes_p != codes_q || scales_p != scales_q || sg_p != sg_q))
    return NS_ERR_ARG;
  // with a workspace of nvfp4_gemm_workspace_bytes() the split-K schedule is
  // used; without one (ws == NULL, ws_bytes == 0) the product runs unsplit
  const bool split_ok = ws != nullptr;
  nvfp4::GemmPlan plan = nvfp4::plan_gemm(M, N, K, symmetric != 0, split_ok);
  if (split_ok && ws_bytes < plan.ws_bytes) return NS_ERR_WORKSPACE;
  if (!al(codes_p, 16) || !al(scales_p, 16) || !al(codes_q, 16) || !al(scales_q, 16) ||
      !al(out, 16) || !al(sg_p, 4) || !al(sg_q, 4) || !al(addend, 16) || !al(ws, 16) ||
      !al(amax_out, 4))
    return NS_ERR_ARG;
  const size_t mk = (size_t)(M * K), nk = (size_t)(N * K), mn = (size_t)(M * N) * sizeof(float);
  const Span P{codes_p, mk / 2}, PS{scales_p, mk / 16}, Q{codes_q, nk / 2}, QS{scales_q, nk / 16},
      SP{sg_p, sizeof(float)}, SQ{sg_q, sizeof(float)}, O{out, mn},
      Ad{beta != 0.0f && addend != out ? addend : nullptr, mn}, Am{amax_out, sizeof(uint32_t)},
      W{ws, split_ok ? ws_bytes : 0};
  if (hits(O, {P, PS, Q, QS, SP, SQ, Ad, Am, W}) || hits(Am, {P, PS, Q, QS, SP, SQ, Ad, W}) ||
      hits(W, {P, PS, Q, QS, SP, SQ, Ad}))
    return NS_ERR_ARG;
  nvfp4::GemmProblem g{codes_p, scales_p, sg_p, codes_q, scales_q, sg_q, M, N, K,
                       symmetric ? 1 : 0, alpha, beta, beta != 0.0f ? addend : nullptr, out,
                       amax_out, 0};
  NS_TRY(nvfp4::launch_gemm(g, plan, ws, true, as_stream(stream)));
  return NS_OK;
}

size_t ns_workspace_bytes(int64_t m, int64_t n) {
  if (!dims_ok(m) || !dims_ok(n)) return 0;
  return ns_layout(m, n).total;
}

ns_status ns_workspace_layout(int64_t m, int64_t n, ns_workspace_map* map) {
  if (!map) return NS_ERR_ARG;
  if (!dims_ok(m) || !dims_ok(n) || m * n >= kMaxElems) return NS_ERR_SHAPE;
  const NsLayout L = ns_layout(m, n);
  map->xm = m < n ? m : n;
  map->xn = m < n ? n : m;
  map->x = L.X;
  map->a = L.A;
  map->b = L.B;
  map->qx_codes = L.qx_c;
  map->qx_scales = L.qx_s;
  map->qt_codes = L.qt_c;
  map->qt_scales = L.qt_s;
  map->qa_codes = L.qa_c;
  map->qa_scales = L.qa_s;
  map->qb_codes = L.qb_c;
  map->qb_scales = L.qb_s;
  map->global_scales = L.sg;
  map->total = L.total;
  return NS_OK;
}

ns_status ns_orthogonalize(const void* G, ns_dtype gt, int64_t m, int64_t n, const float* coeffs,
                           int k, float clip, void* out, ns_dtype ot, void* ws, size_t ws_bytes,
                           void* stream) {
  ns_status st = validate_ns(G, gt, m, n, coeffs, k, clip, out, ot);
  if (st != NS_OK) return st;
  if (!ws || ws_bytes < ns_workspace_bytes(m, n)) return NS_ERR_WORKSPACE;
  st = check_ns_ws(G, gt, m, n, out, ot, ws, ws_bytes);
  if (st != NS_OK) return st;
  return ns_run(G, gt, m, n, coeffs, k, clip, 0.0, nullptr, false, out, ot, static_cast<uint8_t*>(ws),
                as_stream(stream));
}

ns_status ns_orthogonalize_rht(const void* G, ns_dtype gt, int64_t m, int64_t n,
                               const float* coeffs, int k, float clip, const uint16_t* masks,
                               void* out, ns_dtype ot, void* ws, size_t ws_bytes, void* stream) {
  if (!masks) return NS_ERR_ARG;
  ns_status st = validate_ns(G, gt, m, n, coeffs, k, clip, out, ot);
  if (st != NS_OK) return st;
  if (!ws || ws_bytes < ns_workspace_bytes(m, n)) return NS_ERR_WORKSPACE;
  st = check_ns_ws(G, gt, m, n, out, ot, ws, ws_bytes);
  if (st != NS_OK) return st;
  return ns_run(G, gt, m, n, coeffs, k, clip, 0.0, masks, false, out, ot, static_cast<uint8_t*>(ws),
                as_stream(stream));
}

ns_status ns_orthogonalize_ex(const void* G, ns_dtype gt, int64_t m, int64_t n,
                              const float* coeffs, int k, const ns_options* opt, void* out,
                              ns_dtype ot, void* ws, size_t ws_bytes, void* stream) {
  if (!opt) return NS_ERR_ARG;
  const double q = opt->clip_quantile;
  if (std::isnan(q) || q < 0.0 || q > 1.0) return NS_ERR_ARG;
  // with a quantile the clip value is not used; validate as if clipping were off
  const float clip = q > 0.0 ? INFINITY : opt->clip;
  ns_status st = validate_ns(G, gt, m, n, coeffs, k, clip, out, ot);
  if (st != NS_OK) return st;
  if (!ws || ws_bytes < ns_workspace_bytes(m, n)) return NS_ERR_WORKSPACE;
  st = check_ns_ws(G, gt, m, n, out, ot, ws, ws_bytes);
  if (st != NS_OK) return st;
  return ns_run(G, gt, m, n, coeffs, k, clip, q, opt->rht_masks, opt->adaptive46 != 0, out, ot,
                static_cast<uint8_t*>(ws), as_stream(stream));
}

size_t ns_abs_quantile_workspace_bytes(void) { return align_up(nvfp4::abs_quantile_workspace_bytes()); }

ns_status ns_abs_quantile(const void* x, ns_dtype xt, int64_t count, double q, float* out, void* ws,
                          size_t ws_bytes, void* stream) {
  if (!x || !out || !dtype_ok(xt) || std::isnan(q) || !(q > 0.0) || q > 1.0) return NS_ERR_ARG;
  if (!dims_ok(count) || count >= kMaxElems) return NS_ERR_SHAPE;
  if (!ws || ws_bytes < ns_abs_quantile_workspace_bytes()) return NS_ERR_WORKSPACE;
  if (!al(x, 16) || !al(ws, 16) || !al(out, 4)) return NS_ERR_ARG;
  const Span X{x, (size_t)count * dtype_size(xt)}, W{ws, ws_bytes};
  if (hits(Span{out, sizeof(float)}, {X, W}) || hits(W, {X})) return NS_ERR_ARG;
  NS_TRY(nvfp4::launch_abs_quantile(x, (Dt)xt, count, quantile_rank(q, count), out, ws,
                                    as_stream(stream)));
  return NS_OK;
}

}  // extern "C" (reopened below)

namespace {

// Runs run(i, stream) for work items 0 .. count-1 on the group streams,
// forked from and joined back into `caller`: largest item first (cost[i]),
// each to the stream with the least work so far.  Every stream used is
// joined back, also after an error.
// Streams a grouped call may be given by its caller, at most.
constexpr int kMaxCallerStreams = 16;

template <class F>
ns_status run_grouped_on(int count, const std::vector<double>& cost, hipStream_t caller,
                         const hipStream_t* ss, int nss, F&& run) {
  const int used = count < nss ? count : nss;
  hipEvent_t ev[kMaxCallerStreams + 1] = {};  // ev[0] forks, ev[1 + j] joins stream j
  for (int j = 0; j <= used; ++j) {
    const hipError_t e = hipEventCreateWithFlags(&ev[j], hipEventDisableTiming);
    if (e != hipSuccess) {
      for (int t = 0; t < j; ++t) (void)hipEventDestroy(ev[t]);
      return hip_failed(e, "hipEventCreateWithFlags", __LINE__);
    }
  }
  std::vector<int> order((size_t)count);
  for (int i = 0; i < count; ++i) order[(size_t)i] = i;
  std::stable_sort(order.begin(), order.end(),
                   [&](int x, int y) { return cost[(size_t)x] > cost[(size_t)y]; });
  ns_status st = NS_OK;
  hipError_t e = hipEventRecord(ev[0], caller);
  for (int j = 0; j < used && e == hipSuccess; ++j) e = hipStreamWaitEvent(ss[j], ev[0], 0);
  if (e == hipSuccess) {
    double load[kMaxCallerStreams] = {};
    for (int i : order) {
      int j = 0;
      for (int t = 1; t < used; ++t) j = load[t] < load[j] ? t : j;
      st = run(i, ss[j]);
      if (st != NS_OK) break;
      load[j] += cost[(size_t)i];
    }
    for (int j = 0; j < used; ++j) {
      hipError_t ej = hipEventRecord(ev[1 + j], ss[j]);
      if (ej == hipSuccess) ej = hipStreamWaitEvent(caller, ev[1 + j], 0);
      if (e == hipSuccess) e = ej;
    }
  }
  for (int j = 0; j <= used; ++j) (void)hipEventDestroy(ev[j]);
  if (st != NS_OK) return st;
  if (e != hipSuccess) return hip_failed(e, "group fork/join", __LINE__);
  return NS_OK;
}

// On the library's own streams of the current device.
template <class F>
ns_status run_grouped(int count, const std::vector<double>& cost, hipStream_t caller, F&& run) {
  hipStream_t ss[kGroupStreams];
  NS_TRY(group_streams(ss));
  return run_grouped_on(count, cost, caller, ss, kGroupStreams, run);
}

// The problems of a grouped call run concurrently: no output may touch
// another problem's input or output, and the workspace touches none of them.
ns_status check_group(int count, const void* const* G, const int64_t* m, const int64_t* n,
                      ns_dtype gt, void* const* out, ns_dtype ot, const void* ws, size_t ws_bytes) {
  if (!al(ws, 16)) return NS_ERR_ARG;
  const Span W{ws, ws_bytes};
  for (int i = 0; i < count; ++i) {
    const size_t e = (size_t)(m[i] * n[i]);
    const Span Gi{G[i], e * dtype_size(gt)}, Oi{out[i], e * dtype_size(ot)};
    if (hits(W, {Gi, Oi})) return NS_ERR_ARG;
    for (int j = 0; j < count; ++j) {
      if (j == i) continue;
      const size_t f = (size_t)(m[j] * n[j]);
      if (hits(Oi, {Span{G[j], f * dtype_size(gt)}, Span{out[j], f * dtype_size(ot)}}))
        return NS_ERR_ARG;
    }
  }
  return NS_OK;
}

// The work items of a grouped call.  Matrices that share an iterate shape
// (min(m, n) x max(m, n)) form a class, in order of first appearance,
// members in call order; each class's workspace parts are contiguous, one
// stride apart (the part size depends on the iterate shape only), and the
// total is the sum of the parts, as ns_grouped_workspace_bytes counts it.
// A class of matrices too small to fill the GPU alone (Gram products of
// fewer than two 128 x 128 tiles per CU) is one work item, one batch: that
// is where batching pays, by evening out the tile schedule.  A larger class
// is cut into as many runs of consecutive members as there are streams, so
// that it spreads over all of them in items of equal cost.  Matrices that
// cannot be batched (a transform, products off the fast path) are one work
// item each.  Measured on one MI355X, five quintic steps, interleaved runs
// against one matrix per item: the four 3072-wide blocks 28.6-28.7 -> 26.1-26.2
// ms, the pages' blocks at d = 4096 62.4-62.6 -> 59.4-59.5 ms, at d = 6144
// 159.8-160.2 -> 159.7-160.1 ms; large classes as single matrices instead:
// 61.0-61.3 and 158.9-159.5 ms; large classes in runs of at most the group's
// cost over the stream count (coarser items, worse balance) 1-2 ms slower at
// d = 6144.
constexpr int64_t kFillTiles = 2 * 256;
struct GroupPlan {
  std::vector<std::vector<int>> items;   // member indices per run
  std::vector<size_t> off;               // per matrix: byte offset of its part
  std::vector<size_t> stride;            // per run: bytes between members' parts
  std::vector<double> cost;              // per run: sum of m n min(m, n)
};

GroupPlan plan_group(int count, const int64_t* m, const int64_t* n, int nstreams, bool rht) {
  std::vector<std::pair<int64_t, int64_t>> keys;
  std::vector<std::vector<int>> classes;
  auto cost_of = [&](int i) {
    const double a = (double)m[i], b = (double)n[i];
    return a * b * (a < b ? a : b);
  };
  for (int i = 0; i < count; ++i) {
    const std::pair<int64_t, int64_t> key{m[i] < n[i] ? m[i] : n[i], m[i] < n[i] ? n[i] : m[i]};
    size_t c = 0;
    while (c < keys.size() && keys[c] != key) ++c;
    if (c == keys.size()) {
      keys.push_back(key);
      classes.emplace_back();
    }
    classes[c].push_back(i);
  }
  GroupPlan P;
  P.off.assign((size_t)count, 0);
  size_t o = 0;
  for (const std::vector<int>& cls : classes) {
    const size_t part = ns_workspace_bytes(m[cls[0]], n[cls[0]]);
    const double each = cost_of(cls[0]);
    const bool small = ns_layout(m[cls[0]], n[cls[0]]).p1.tiles < kFillTiles;
    const size_t ns_ = (size_t)(nstreams > 0 ? nstreams : 1);
    size_t run = small ? cls.size() : (cls.size() + ns_ - 1) / ns_;
    if (!batchable(m[cls[0]], n[cls[0]], rht) || run < 1) run = 1;   // one matrix per item
    if (run > (size_t)nvfp4::kMaxBatchOut) run = nvfp4::kMaxBatchOut;
    for (size_t a = 0; a < cls.size(); a += run) {
      const size_t b = a + run < cls.size() ? a + run : cls.size();
      P.items.emplace_back(cls.begin() + (std::ptrdiff_t)a, cls.begin() + (std::ptrdiff_t)b);
      P.stride.push_back(part);
      P.cost.push_back(each * (double)(b - a));
      for (size_t t = a; t < b; ++t) {
        P.off[(size_t)cls[t]] = o;
        o += part;
      }
    }
  }
  return P;
}

// Run c of a grouped call on stream s: one batch when it has several
// members (see ns_run_batch), else its members one by one.
template <class One>
ns_status run_class(const GroupPlan& P, int c, const void* const* G, ns_dtype gt,
                    const int64_t* m, const int64_t* n, const float* coeffs, int k,
                    const float* clip, double clip_q, const uint16_t* masks, bool a46,
                    void* const* out, ns_dtype ot, uint8_t* base, hipStream_t s, One&& one) {
  const std::vector<int>& mem = P.items[(size_t)c];
  const int first = mem[0];
  if (mem.size() < 2 || !batchable(m[first], n[first], masks != nullptr)) {
    for (int i : mem) {
      const ns_status st = one(i, s);
      if (st != NS_OK) return st;
    }
    return NS_OK;
  }
  const size_t cnt = mem.size();
  std::vector<const void*> g(cnt);
  std::vector<void*> o(cnt);
  std::vector<int64_t> mm(cnt), nn(cnt);
  std::vector<float> cl(cnt);
  for (size_t j = 0; j < cnt; ++j) {
    const int i = mem[j];
    g[j] = G[i];
    o[j] = out[i];
    mm[j] = m[i];
    nn[j] = n[i];
    cl[j] = clip_q > 0.0 ? INFINITY : clip[i];
  }
  return ns_run_batch((int)cnt, g.data(), gt, mm.data(), nn.data(), coeffs, k, cl.data(), clip_q,
                      masks, a46, o.data(), ot, base + P.off[(size_t)first], P.stride[(size_t)c], s);
}

}  // namespace

extern "C" {

size_t ns_grouped_workspace_bytes(int count, const int64_t* m, const int64_t* n) {
  if (count <= 0 || !m || !n) return 0;
  size_t total = 0;
  for (int i = 0; i < count; ++i) {
    const size_t b = ns_workspace_bytes(m[i], n[i]);
    if (b == 0) return 0;
    total += b;
  }
  return total;
}

}  // extern "C"

namespace {
ns_status grouped_ex_impl(int count, const void* const* G, const int64_t* m, const int64_t* n,
                          ns_dtype gt, const float* coeffs, int k, const float* clip,
                          const ns_options* opt, void* const* out, ns_dtype ot, void* ws,
                          size_t ws_bytes, void* const* streams, int nstreams, void* stream);
}  // namespace

extern "C" {

ns_status ns_orthogonalize_grouped_ex(int count, const void* const* G, const int64_t* m,
                                      const int64_t* n, ns_dtype gt, const float* coeffs, int k,
                                      const float* clip, const ns_options* opt, void* const* out,
                                      ns_dtype ot, void* ws, size_t ws_bytes, void* stream) {
  return grouped_ex_impl(count, G, m, n, gt, coeffs, k, clip, opt, out, ot, ws, ws_bytes, nullptr,
                         0, stream);
}

ns_status ns_orthogonalize_grouped_on(int count, const void* const* G, const int64_t* m,
                                      const int64_t* n, ns_dtype gt, const float* coeffs, int k,
                                      const float* clip, const ns_options* opt, void* const* out,
                                      ns_dtype ot, void* ws, size_t ws_bytes,
                                      void* const* streams, int nstreams, void* stream) {
  if (!streams || nstreams < 1 || nstreams > kMaxCallerStreams) return NS_ERR_ARG;
  for (int j = 0; j < nstreams; ++j)
    if (!streams[j]) return NS_ERR_ARG;
  const ns_options plain{INFINITY, 0.0, nullptr, 0};   // clip[i] per matrix, nothing else
  return grouped_ex_impl(count, G, m, n, gt, coeffs, k, clip, opt ? opt : &plain, out, ot, ws,
                         ws_bytes, streams, nstreams, stream);
}

}  // extern "C"

namespace {

// The grouped call with options; streams = NULL runs on the library's own
// streams, else on the caller's nstreams streams.
ns_status grouped_ex_impl(int count, const void* const* G, const int64_t* m, const int64_t* n,
                          ns_dtype gt, const float* coeffs, int k, const float* clip,
                          const ns_options* opt, void* const* out, ns_dtype ot, void* ws,
                          size_t ws_bytes, void* const* streams, int nstreams, void* stream) {
  if (count <= 0 || !G || !m || !n || !out || !opt) return NS_ERR_ARG;
  const double q = opt->clip_quantile;
  if (std::isnan(q) || q < 0.0 || q > 1.0) return NS_ERR_ARG;
  if (q == 0.0 && !clip) return NS_ERR_ARG;
  for (int i = 0; i < count; ++i) {
    const float ci = q > 0.0 ? INFINITY : clip[i];
    ns_status st = validate_ns(G[i], gt, m[i], n[i], coeffs, k, ci, out[i], ot);
    if (st != NS_OK) return st;
  }
  const size_t need = ns_grouped_workspace_bytes(count, m, n);
  if (!ws || ws_bytes < need) return NS_ERR_WORKSPACE;
  {
    const ns_status st = check_group(count, G, m, n, gt, out, ot, ws, ws_bytes);
    if (st != NS_OK) return st;
  }
  uint8_t* base = static_cast<uint8_t*>(ws);
  const GroupPlan P = plan_group(count, m, n, streams ? nstreams : kGroupStreams,
                                 opt->rht_masks != nullptr);
  const bool a46 = opt->adaptive46 != 0;
  auto one = [&](int i, hipStream_t s) {
    const float ci = q > 0.0 ? INFINITY : clip[i];
    return ns_run(G[i], gt, m[i], n[i], coeffs, k, ci, q, opt->rht_masks, a46, out[i], ot,
                  base + P.off[(size_t)i], s);
  };
  auto cls = [&](int c, hipStream_t s) {
    return run_class(P, c, G, gt, m, n, coeffs, k, clip, q, opt->rht_masks, a46, out, ot, base, s,
                     one);
  };
  const int items = (int)P.items.size();
  if (!streams) return run_grouped(items, P.cost, as_stream(stream), cls);
  hipStream_t ss[kMaxCallerStreams];
  for (int j = 0; j < nstreams; ++j) ss[j] = as_stream(streams[j]);
  return run_grouped_on(items, P.cost, as_stream(stream), ss, nstreams, cls);
}

}  // namespace

extern "C" {

ns_status ns_orthogonalize_grouped(int count, const void* const* G, const int64_t* m,
                                   const int64_t* n, ns_dtype gt, const float* coeffs, int k,
                                   const float* clip, void* const* out, ns_dtype ot, void* ws,
                                   size_t ws_bytes, void* stream) {
  if (count <= 0 || !G || !m || !n || !clip || !out) return NS_ERR_ARG;
  for (int i = 0; i < count; ++i) {
    ns_status st = validate_ns(G[i], gt, m[i], n[i], coeffs, k, clip[i], out[i], ot);
    if (st != NS_OK) return st;
  }
  const size_t need = ns_grouped_workspace_bytes(count, m, n);
  if (!ws || ws_bytes < need) return NS_ERR_WORKSPACE;
  {
    const ns_status st = check_group(count, G, m, n, gt, out, ot, ws, ws_bytes);
    if (st != NS_OK) return st;
  }
  uint8_t* base = static_cast<uint8_t*>(ws);
  const GroupPlan P = plan_group(count, m, n, kGroupStreams, false);
  auto one = [&](int i, hipStream_t s) {
    return ns_run(G[i], gt, m[i], n[i], coeffs, k, clip[i], 0.0, nullptr, false, out[i], ot,
                  base + P.off[(size_t)i], s);
  };
  return run_grouped((int)P.items.size(), P.cost, as_stream(stream), [&](int c, hipStream_t s) {
    return run_class(P, c, G, gt, m, n, coeffs, k, clip, 0.0, nullptr, false, out, ot, base, s,
                     one);
  });
}

}  // extern "C"
