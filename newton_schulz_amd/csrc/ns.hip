// Newton–Schulz prologue and epilogue kernels for gfx950: clip + Frobenius
// normalisation with the m <= n orientation, and the final write-out.
//
// X_0 = clamp(G, -clip, clip) / (||clamp(G)||_F + eps): the clip stands for
// the p99 outlier clipping that the Full-Stack FP4 paper applies before its
// NVFP4 NS (§3.4, "NVFP4 Root Optimizer"); the threshold is the caller's.
// The norm is a deterministic two-level FP64 reduction.
#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {
namespace {

constexpr int kThreads = 256;
constexpr int kFlatGrid = 4096;   // workgroups of the flat passes at most

// clamp that lets NaN through
__device__ __forceinline__ float clampf(float x, float c) {
  return x > c ? c : (x < -c ? -c : x);
}

__device__ __forceinline__ double block_sum(double v) {
  __shared__ double red[kThreads / 64];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double r = 0.0;
  if (threadIdx.x == 0)
    for (int w = 0; w < kThreads / 64; ++w) r += red[w];
  return r;
}

__device__ __forceinline__ uint32_t block_max_u32(uint32_t v) {
  __shared__ uint32_t red[kThreads / 64];
  v = wave_max_u32(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t r = 0;
  if (threadIdx.x == 0)
    for (int w = 0; w < kThreads / 64; ++w) r = red[w] > r ? red[w] : r;
  return r;
}

template <Dt T>
__global__ __launch_bounds__(kThreads) void norm_partials_kernel(const void* G, int64_t n, float clip,
                                                                  const float* clip_dev, double* part,
                                                                  uint32_t* part_amax) {
  if (clip_dev) clip = *clip_dev;
  // 16-byte units (4 FP32 or 8 BF16 values), consecutive lanes on
  // consecutive units, four loads in flight; each thread keeps four FP64
  // chains (one per 32-bit word of a unit) and adds them in a fixed order
  constexpr int EPU = T == Dt::F32 ? 4 : 8;
  constexpr int U = 4;
  const int64_t nu = n / EPU, stride = (int64_t)gridDim.x * kThreads;
  double ch[4] = {0.0, 0.0, 0.0, 0.0};
  uint32_t amax = 0;
  auto add = [&](uint4 w) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if constexpr (T == Dt::F32) {
        const float c = clampf(__uint_as_float(ws[t]), clip);
        const double x = (double)c;
        ch[t] = fma(x, x, ch[t]);
        const uint32_t a = abs_bits(c);
        amax = a > amax ? a : amax;
      } else {
        const float c0 = clampf(__uint_as_float(ws[t] << 16), clip);
        const double x0 = (double)c0;
        ch[t] = fma(x0, x0, ch[t]);
        const float c1 = clampf(__uint_as_float(ws[t] & 0xFFFF0000u), clip);
        const double x1 = (double)c1;
        ch[t] = fma(x1, x1, ch[t]);
        const uint32_t a0 = abs_bits(c0), a1 = abs_bits(c1);
        amax = a0 > amax ? a0 : amax;
        amax = a1 > amax ? a1 : amax;
      }
    }
  };
  const uint4* p = static_cast<const uint4*>(G);
  int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; u + (U - 1) * stride < nu; u += U * stride) {
    uint4 w[U];
#pragma unroll
    for (int k = 0; k < U; ++k) w[k] = p[u + k * stride];
#pragma unroll
    for (int k = 0; k < U; ++k) add(w[k]);
  }
  for (; u < nu; u += stride) add(p[u]);
  double s = block_sum((ch[0] + ch[1]) + (ch[2] + ch[3]));
  __syncthreads();
  const uint32_t m = block_max_u32(amax);
  if (threadIdx.x == 0) {
    part[blockIdx.x] = s;
    part_amax[blockIdx.x] = m;
  }
}

__global__ __launch_bounds__(kThreads) void norm_finalize_kernel(const double* part,
                                                                  const uint32_t* part_amax,
                                                                  double* inv, uint32_t* z0,
                                                                  uint32_t* z1, uint32_t* z2,
                                                                  uint32_t* words, int n_words) {
  double acc = 0.0;
  uint32_t am = 0;
  for (int i = threadIdx.x; i < kNormParts; i += kThreads) {
    acc += part[i];
    am = part_amax[i] > am ? part_amax[i] : am;
  }
  double s = block_sum(acc);
  __syncthreads();
  am = block_max_u32(am);
  if (z0) amax_clear(z0);
  if (z1) amax_clear(z1);
  if (z2) amax_clear(z2);
  for (int i = threadIdx.x; i < n_words; i += kThreads) words[i] = 0u;
  if (threadIdx.x == 0) {
    const double iv = 1.0 / (sqrt(s) + 1e-7);
    *inv = iv;
    // max |X_0|: the normalisation of the largest |clamp(G)| (monotone
    // rounding); a non-finite maximum stays NaN.  Thread 0 cleared partial 0
    // of z0 above, in program order before this store.
    if (z0) z0[0] = am >= 0x7F800000u ? kNaNBits : abs_bits((float)((double)__uint_as_float(am) * iv));
  }
}

// 64 x 64 transposing tiles: a workgroup reads a tile of the source, whose
// 64 rows hold 16 four-value units each, with lanes 16k .. 16k+15 on one
// row's units (contiguous), keeps it in LDS as FP32, and writes the
// transposed tile the same way: lanes 16k .. 16k+15 on the 16 units of one
// destination row.  With the 65-float row pitch both LDS phases are free of
// bank conflicts.
constexpr int kTile = 64;
using TileBuf = float[kTile][kTile + 1];

// tile[r][c] = src[(row0 + r) * ld + col0 + c] for rows < nrows, cols < ncols
template <Dt T>
__device__ __forceinline__ void tile_load(const void* src, int64_t ld, int64_t row0, int64_t col0,
                                          int64_t nrows, int64_t ncols, TileBuf& tile) {
  const int u = threadIdx.x & 15;
#pragma unroll
  for (int pass = 0; pass < kTile / 16; ++pass) {
    const int r = pass * 16 + (threadIdx.x >> 4);
    uint4 w = make_uint4(0u, 0u, 0u, 0u);
    if (row0 + r < nrows && col0 + 4 * u < ncols) w = load4<T>(src, ((row0 + r) * ld + col0) / 4 + u);
    tile[r][4 * u] = __uint_as_float(w.x);
    tile[r][4 * u + 1] = __uint_as_float(w.y);
    tile[r][4 * u + 2] = __uint_as_float(w.z);
    tile[r][4 * u + 3] = __uint_as_float(w.w);
  }
}

// X = normalised G^T: G is xn x xm, X is xm x xn.
template <Dt T>
__global__ __launch_bounds__(kThreads) void normalize_tr_kernel(const void* G, int64_t xm, int64_t xn,
                                                                 float clip, const float* clip_dev,
                                                                 const double* invp, float* X,
                                                                 uint32_t* amax_slot) {
  __shared__ TileBuf tile;
  if (clip_dev) clip = *clip_dev;
  const double inv = *invp;
  const int64_t r0 = (int64_t)blockIdx.y * kTile, c0 = (int64_t)blockIdx.x * kTile;   // X tile
  tile_load<T>(G, xm, c0, r0, xn, xm, tile);      // tile[X col][X row]
  __syncthreads();
  const int u = threadIdx.x & 15;
  uint32_t amax = 0;
#pragma unroll
  for (int pass = 0; pass < kTile / 16; ++pass) {
    const int r = pass * 16 + (threadIdx.x >> 4);
    if (r0 + r < xm && c0 + 4 * u < xn) {
      float y[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        y[i] = (float)((double)clampf(tile[4 * u + i][r], clip) * inv);
        const uint32_t a = abs_bits(y[i]);
        amax = a > amax ? a : amax;
      }
      reinterpret_cast<float4*>(X + (r0 + r) * xn + c0)[u] = make_float4(y[0], y[1], y[2], y[3]);
    }
  }
  amax_publish_block(amax, amax_slot);
}

// X = G (same layout): a flat pass over 4-value units, consecutive lanes on
// consecutive units, four loads in flight per thread.
template <Dt T>
__global__ __launch_bounds__(kThreads) void normalize_flat_kernel(const void* G, int64_t nq, float clip,
                                                                   const float* clip_dev, const double* invp,
                                                                   float* X, uint32_t* amax_slot) {
  constexpr int U = 4;
  if (clip_dev) clip = *clip_dev;
  const double inv = *invp;
  uint32_t amax = 0;
  auto emit = [&](int64_t q, uint4 w) {
    const uint32_t v[4] = {w.x, w.y, w.z, w.w};
    float y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      y[i] = (float)((double)clampf(__uint_as_float(v[i]), clip) * inv);
      const uint32_t a = abs_bits(y[i]);
      amax = a > amax ? a : amax;
    }
    reinterpret_cast<float4*>(X)[q] = make_float4(y[0], y[1], y[2], y[3]);
  };
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t q = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; q + (U - 1) * stride < nq; q += U * stride) {
    uint4 w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) w[u] = load4<T>(G, q + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) emit(q + u * stride, w[u]);
  }
  for (; q < nq; q += stride) emit(q, load4<T>(G, q));
  amax_publish_block(amax, amax_slot);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((b >> 16) | 0x40u);
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ uint2 bf16x4(float a, float b, float c, float d) {
  return make_uint2((uint32_t)f32_to_bf16_rne(a) | ((uint32_t)f32_to_bf16_rne(b) << 16),
                    (uint32_t)f32_to_bf16_rne(c) | ((uint32_t)f32_to_bf16_rne(d) << 16));
}

// out = X in the output type (same layout): a flat pass over 4-value units.
template <Dt O>
__global__ __launch_bounds__(kThreads) void write_out_flat_kernel(const float* X, int64_t nq, void* out) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t q = (int64_t)blockIdx.x * kThreads + threadIdx.x; q < nq; q += stride) {
    const float4 w = reinterpret_cast<const float4*>(X)[q];
    if constexpr (O == Dt::F32)
      reinterpret_cast<float4*>(out)[q] = w;
    else
      reinterpret_cast<uint2*>(out)[q] = bf16x4(w.x, w.y, w.z, w.w);
  }
}

// out = X^T (xn x xm) through 64 x 64 tiles of X.
template <Dt O>
__global__ __launch_bounds__(kThreads) void write_out_tr_kernel(const float* X, int64_t xm, int64_t xn,
                                                                 void* out) {
  __shared__ TileBuf tile;
  const int64_t r0 = (int64_t)blockIdx.y * kTile, c0 = (int64_t)blockIdx.x * kTile;   // X tile
  tile_load<Dt::F32>(X, xn, r0, c0, xm, xn, tile);   // tile[X row][X col]
  __syncthreads();
  const int u = threadIdx.x & 15;
#pragma unroll
  for (int pass = 0; pass < kTile / 16; ++pass) {
    const int c = pass * 16 + (threadIdx.x >> 4);      // out row c0 + c, columns r0 + 4u ..
    if (c0 + c < xn && r0 + 4 * u < xm) {
      const float a = tile[4 * u][c], b = tile[4 * u + 1][c], d = tile[4 * u + 2][c], e = tile[4 * u + 3][c];
      const int64_t q = ((c0 + c) * xm + r0) / 4 + u;
      if constexpr (O == Dt::F32)
        reinterpret_cast<float4*>(out)[q] = make_float4(a, b, d, e);
      else
        reinterpret_cast<uint2*>(out)[q] = bf16x4(a, b, d, e);
    }
  }
}

}  // namespace

hipError_t launch_norm_partials(const void* G, Dt gt, int64_t n, float clip, const float* clip_dev,
                                double* part, uint32_t* part_amax, hipStream_t s) {
  if (gt == Dt::F32)
    norm_partials_kernel<Dt::F32><<<kNormParts, kThreads, 0, s>>>(G, n, clip, clip_dev, part, part_amax);
  else
    norm_partials_kernel<Dt::BF16><<<kNormParts, kThreads, 0, s>>>(G, n, clip, clip_dev, part, part_amax);
  return hipGetLastError();
}

hipError_t launch_norm_finalize(const double* part, const uint32_t* part_amax, double* inv,
                                uint32_t* z0, uint32_t* z1, uint32_t* z2, uint32_t* words,
                                int n_words, hipStream_t s) {
  norm_finalize_kernel<<<1, kThreads, 0, s>>>(part, part_amax, inv, z0, z1, z2, words,
                                              words ? n_words : 0);
  return hipGetLastError();
}

hipError_t launch_normalize(const void* G, Dt gt, int64_t xm, int64_t xn, bool transposed,
                            float clip, const float* clip_dev, const double* inv, float* X,
                            uint32_t* amax_slot, hipStream_t s) {
  if (!transposed) {
    const int64_t nq = xm * xn / 4;
    int64_t g = (nq + kThreads - 1) / kThreads;
    g = g > kFlatGrid ? kFlatGrid : g;
    if (gt == Dt::F32)
      normalize_flat_kernel<Dt::F32><<<(unsigned)g, kThreads, 0, s>>>(G, nq, clip, clip_dev, inv, X, amax_slot);
    else
      normalize_flat_kernel<Dt::BF16><<<(unsigned)g, kThreads, 0, s>>>(G, nq, clip, clip_dev, inv, X, amax_slot);
    return hipGetLastError();
  }
  dim3 grid((unsigned)((xn + kTile - 1) / kTile), (unsigned)((xm + kTile - 1) / kTile));
  if (gt == Dt::F32)
    normalize_tr_kernel<Dt::F32><<<grid, kThreads, 0, s>>>(G, xm, xn, clip, clip_dev, inv, X, amax_slot);
  else
    normalize_tr_kernel<Dt::BF16><<<grid, kThreads, 0, s>>>(G, xm, xn, clip, clip_dev, inv, X, amax_slot);
  return hipGetLastError();
}

hipError_t launch_write_out(const float* X, int64_t xm, int64_t xn, bool transposed, void* out,
                            Dt ot, hipStream_t s) {
  if (!transposed) {
    const int64_t nq = xm * xn / 4;
    int64_t g = (nq + kThreads - 1) / kThreads;
    g = g > kFlatGrid ? kFlatGrid : g;
    if (ot == Dt::F32)
      write_out_flat_kernel<Dt::F32><<<(unsigned)g, kThreads, 0, s>>>(X, nq, out);
    else
      write_out_flat_kernel<Dt::BF16><<<(unsigned)g, kThreads, 0, s>>>(X, nq, out);
    return hipGetLastError();
  }
  dim3 grid((unsigned)((xn + kTile - 1) / kTile), (unsigned)((xm + kTile - 1) / kTile));
  if (ot == Dt::F32)
    write_out_tr_kernel<Dt::F32><<<grid, kThreads, 0, s>>>(X, xm, xn, out);
  else
    write_out_tr_kernel<Dt::BF16><<<grid, kThreads, 0, s>>>(X, xm, xn, out);
  return hipGetLastError();
}

}  // namespace nvfp4
