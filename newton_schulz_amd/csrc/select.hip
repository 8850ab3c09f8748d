// Exact q-quantile of |x| on gfx950: the clip threshold of the NVFP4 Root
// path (Full-Stack FP4, arXiv 2607.04422: §3.4 p99 outlier clipping; App. F
// Table 8, Root quantile ratio 0.99), taken as the k-th smallest magnitude,
// k = ceil(q N).
//
// Magnitudes are ordered by their FP32 bit patterns with the sign cleared
// (non-finite values as the NaN pattern, above every finite one), so the
// k-th smallest is found by radix selection on 31-bit keys: three passes
// over an FP32 input fix bits 30..20, 19..9 and 8..0 of the answer.  Each
// pass builds per-workgroup LDS histograms of the keys that match the
// prefix found so far and folds them into a global histogram whose bins sit
// one 128-byte line apart (atomics on distinct lines proceed in parallel); a
// one-workgroup kernel then scans the bins, picks the one holding the
// remaining rank and extends the prefix.  BF16 keys (widened exactly) have
// only 15 bits that can be set, so one pass over a histogram of all 2^15
// of them finds the answer directly (hist15_kernel below).
#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {
namespace {

constexpr int kThreads = 256;
constexpr int kHistBlocks = 512;     // workgroups of a histogram pass
constexpr int kBins = 2048;          // 11 key bits per pass at most
constexpr int kBinStride = 32;       // words between global bins
constexpr int kScanThreads = 1024;   // scan: two bins per thread
constexpr int kHist15Blocks = 256;   // one-pass BF16 histogram: one workgroup per CU

struct Pass {
  int shift, bits;
};
constexpr Pass kPassesF32[3] = {{20, 11}, {9, 11}, {0, 9}};

__device__ __forceinline__ uint32_t magnitude_key(uint32_t f32_bits) {
  const uint32_t b = f32_bits & 0x7FFFFFFFu;
  return b >= 0x7F800000u ? kNaNBits : b;
}

// Histogram of the keys whose bits above `shift + bits` equal the prefix
// (FP32 input).
__global__ __launch_bounds__(kThreads) void radix_hist_kernel(const void* x, int64_t n,
                                                              const SelectState* st, int shift,
                                                              int bits, uint32_t* ghist) {
  __shared__ uint32_t h[kBins];
  for (int i = threadIdx.x; i < kBins; i += kThreads) h[i] = 0u;
  __syncthreads();
  const int top = shift + bits;
  const uint32_t pmask = top >= 32 ? 0u : (~0u << top);
  const uint32_t prefix = st->prefix;
  const uint32_t bmask = (1u << bits) - 1u;
  auto count = [&](uint32_t f32_bits) {
    const uint32_t key = magnitude_key(f32_bits);
    if ((key & pmask) == prefix) atomicAdd(&h[(key >> shift) & bmask], 1u);
  };
  // 16-byte vectors of 4 values (n is a multiple of 16)
  const int64_t nvec = n / 4;
  const uint4* p = static_cast<const uint4*>(x);
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nvec;
       i += (int64_t)gridDim.x * kThreads) {
    const uint4 w = p[i];
    count(w.x);
    count(w.y);
    count(w.z);
    count(w.w);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kBins; i += kThreads)
    if (h[i]) atomicAdd(ghist + (size_t)i * kBinStride, h[i]);
}

// One workgroup: find the bin holding the remaining rank, extend the
// prefix, subtract the counts below it, clear the bins; after the last pass
// write the threshold.
__global__ __launch_bounds__(kScanThreads) void radix_select_kernel(SelectState* st, uint32_t* ghist,
                                                                    int shift, int bits, float* out) {
  __shared__ uint32_t wsum[kScanThreads / 64];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int nb = 1 << bits;
  const uint32_t c0 = 2 * t < nb ? ghist[(size_t)(2 * t) * kBinStride] : 0u;
  const uint32_t c1 = 2 * t + 1 < nb ? ghist[(size_t)(2 * t + 1) * kBinStride] : 0u;
  // inclusive scan of per-thread sums: within the wave, then across waves
  uint32_t v = c0 + c1;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  if (lane == 63) wsum[w] = v;
  __syncthreads();
  uint32_t before_wave = 0;
  for (int i = 0; i < w; ++i) before_wave += wsum[i];
  const uint32_t incl = before_wave + v;            // bins 0 .. 2t+1
  const uint32_t excl = incl - c0 - c1;             // bins 0 .. 2t-1
  const uint32_t rank = st->rank;                   // 1-based, within the matching keys
  __syncthreads();                                  // every thread has read rank
  if (excl < rank && rank <= incl) {
    const int bin = rank <= excl + c0 ? 2 * t : 2 * t + 1;
    const uint32_t below = bin == 2 * t ? excl : excl + c0;
    const uint32_t prefix = st->prefix | ((uint32_t)bin << shift);
    st->prefix = prefix;
    st->rank = rank - below;
    if (out) *out = __uint_as_float(prefix);
  }
  if (2 * t < nb) ghist[(size_t)(2 * t) * kBinStride] = 0u;
  if (2 * t + 1 < nb) ghist[(size_t)(2 * t + 1) * kBinStride] = 0u;
}

__global__ void select_init_kernel(SelectState* st, uint32_t* ghist, uint32_t rank) {
  for (int i = threadIdx.x; i < kBins; i += blockDim.x) ghist[(size_t)i * kBinStride] = 0u;
  if (threadIdx.x == 0) {
    st->prefix = 0u;
    st->rank = rank;
  }
}

// ---- BF16 keys in one pass ------------------------------------------------
// A BF16 magnitude has 15 bits, so one histogram of 2^15 bins (128 KB of
// LDS, one workgroup of 1024 threads per CU) counts every key exactly and a
// scan of it finds the rank-th smallest: one read of the input instead of
// two, three launches instead of five.  The global histogram is 2^15
// consecutive words (inside the workspace of the multi-pass path).
constexpr int kBins15 = 1 << 15;
constexpr int kThreads15 = 1024;
constexpr int kBinsPerThread15 = kBins15 / kThreads15;   // 32

__device__ __forceinline__ uint32_t bf16_magnitude_key(uint32_t bf16_bits) {
  const uint32_t b = bf16_bits & 0x7FFFu;
  return b >= 0x7F80u ? (kNaNBits >> 16) : b;
}

__global__ __launch_bounds__(kThreads15) void hist15_init_kernel(SelectState* st, uint32_t* ghist,
                                                                 uint32_t rank) {
  uint4* g = reinterpret_cast<uint4*>(ghist);
  for (int i = threadIdx.x; i < kBins15 / 4; i += blockDim.x) g[i] = make_uint4(0u, 0u, 0u, 0u);
  if (threadIdx.x == 0) {
    st->prefix = 0u;
    st->rank = rank;
  }
}

__global__ __launch_bounds__(kThreads15) void hist15_kernel(const void* x, int64_t n,
                                                            uint32_t* ghist) {
  __shared__ uint32_t h[kBins15];
  for (int i = threadIdx.x; i < kBins15; i += kThreads15) h[i] = 0u;
  __syncthreads();
  auto count = [&](uint4 w) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      atomicAdd(&h[bf16_magnitude_key(ws[t])], 1u);
      atomicAdd(&h[bf16_magnitude_key(ws[t] >> 16)], 1u);
    }
  };
  const int64_t nvec = n / 8;
  const uint4* p = static_cast<const uint4*>(x);
  const int64_t stride = (int64_t)gridDim.x * kThreads15;
  int64_t i = (int64_t)blockIdx.x * kThreads15 + threadIdx.x;
  for (; i + 3 * stride < nvec; i += 4 * stride) {
    uint4 w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) w[u] = p[i + u * stride];
#pragma unroll
    for (int u = 0; u < 4; ++u) count(w[u]);
  }
  for (; i < nvec; i += stride) count(p[i]);
  __syncthreads();
  for (int b = threadIdx.x; b < kBins15; b += kThreads15)
    if (h[b]) atomicAdd(ghist + b, h[b]);
}

// One workgroup: thread t owns bins 32t .. 32t + 31; the thread whose range
// holds the rank finds the bin, whose 15 bits are the BF16 answer.
__global__ __launch_bounds__(kThreads15) void select15_kernel(const SelectState* st,
                                                              const uint32_t* ghist, float* out) {
  __shared__ uint32_t wsum[kThreads15 / 64];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  uint32_t c[kBinsPerThread15];
  const uint4* g = reinterpret_cast<const uint4*>(ghist) + t * (kBinsPerThread15 / 4);
#pragma unroll
  for (int j = 0; j < kBinsPerThread15 / 4; ++j) {
    const uint4 q = g[j];
    c[4 * j] = q.x; c[4 * j + 1] = q.y; c[4 * j + 2] = q.z; c[4 * j + 3] = q.w;
  }
  uint32_t mine = 0;
#pragma unroll
  for (int j = 0; j < kBinsPerThread15; ++j) mine += c[j];
  uint32_t v = mine;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  if (lane == 63) wsum[w] = v;
  __syncthreads();
  uint32_t before = 0;
  for (int i = 0; i < w; ++i) before += wsum[i];
  const uint32_t incl = before + v, excl = incl - mine;   // bins before 32t: excl
  const uint32_t rank = st->rank;
  if (excl < rank && rank <= incl) {
    uint32_t acc = excl;
    int bin = t * kBinsPerThread15;
    for (int j = 0; j < kBinsPerThread15; ++j) {
      if (rank <= acc + c[j]) { bin = t * kBinsPerThread15 + j; break; }
      acc += c[j];
    }
    *out = __uint_as_float((uint32_t)bin << 16);
  }
}

}  // namespace

size_t abs_quantile_workspace_bytes() {
  return (size_t)kBins * kBinStride * sizeof(uint32_t) + 256;
}

hipError_t launch_abs_quantile(const void* x, Dt xt, int64_t n, uint32_t rank, float* out,
                               void* ws, hipStream_t s) {
  uint32_t* ghist = static_cast<uint32_t*>(ws);
  SelectState* st = reinterpret_cast<SelectState*>(static_cast<uint8_t*>(ws) +
                                                   (size_t)kBins * kBinStride * sizeof(uint32_t));
  if (xt == Dt::BF16) {
    static_assert((size_t)kBins15 <= (size_t)kBins * kBinStride, "one-pass bins fit the workspace");
    hist15_init_kernel<<<1, kThreads15, 0, s>>>(st, ghist, rank);
    const int64_t nvec = n / 8;
    int64_t grid = (nvec + kThreads15 * 4 - 1) / (kThreads15 * 4);
    grid = grid < 1 ? 1 : (grid > kHist15Blocks ? kHist15Blocks : grid);
    hist15_kernel<<<(unsigned)grid, kThreads15, 0, s>>>(x, n, ghist);
    select15_kernel<<<1, kThreads15, 0, s>>>(st, ghist, out);
    return hipGetLastError();
  }
  select_init_kernel<<<1, 256, 0, s>>>(st, ghist, rank);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nvec = n / 4;
  int64_t grid = (nvec + kThreads * 4 - 1) / (kThreads * 4);
  grid = grid < 1 ? 1 : (grid > kHistBlocks ? kHistBlocks : grid);
  for (int p = 0; p < 3; ++p) {
    const Pass ps = kPassesF32[p];
    radix_hist_kernel<<<(unsigned)grid, kThreads, 0, s>>>(x, n, st, ps.shift, ps.bits, ghist);
    radix_select_kernel<<<1, kScanThreads, 0, s>>>(st, ghist, ps.shift, ps.bits,
                                                   p == 2 ? out : nullptr);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace nvfp4
