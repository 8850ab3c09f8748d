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

template <Dt T>
__device__ __forceinline__ void load16_raw(const void* base, int64_t idx, uint32_t (&v)[16]) {
  if constexpr (T == Dt::F32) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(base) + idx);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint4 w = p[j];
      v[4 * j] = w.x; v[4 * j + 1] = w.y; v[4 * j + 2] = w.z; v[4 * j + 3] = w.w;
    }
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + idx);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint4 w = p[j];
      uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        v[8 * j + 2 * t] = ws[t] << 16;
        v[8 * j + 2 * t + 1] = ws[t] & 0xFFFF0000u;
      }
    }
  }
}

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

template <Dt T>
__global__ __launch_bounds__(kThreads) void norm_partials_kernel(const void* G, int64_t nblk,
                                                                  float clip, const float* clip_dev,
                                                                  double* part) {
  if (clip_dev) clip = *clip_dev;
  double acc = 0.0;
  for (int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x; b < nblk;
       b += (int64_t)gridDim.x * kThreads) {
    uint32_t v[16];
    load16_raw<T>(G, b * 16, v);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      double x = (double)clampf(__uint_as_float(v[i]), clip);
      acc = fma(x, x, acc);
    }
  }
  double s = block_sum(acc);
  if (threadIdx.x == 0) part[blockIdx.x] = s;
}

__global__ __launch_bounds__(kThreads) void norm_finalize_kernel(const double* part, double* inv,
                                                                  uint32_t* z0, uint32_t* z1,
                                                                  uint32_t* z2) {
  double acc = 0.0;
  for (int i = threadIdx.x; i < kNormParts; i += kThreads) acc += part[i];
  double s = block_sum(acc);
  if (threadIdx.x == 0) *inv = 1.0 / (sqrt(s) + 1e-7);
  if (z0) amax_clear(z0);
  if (z1) amax_clear(z1);
  if (z2) amax_clear(z2);
}

// X tile 64 x 64 per workgroup; thread t owns X row t/4, columns
// 16*(t%4)..+15.  When transposed, G is xn x xm and its tile passes LDS.
template <Dt T, bool TR>
__global__ __launch_bounds__(kThreads) void normalize_kernel(const void* G, int64_t xm, int64_t xn,
                                                              float clip, const float* clip_dev,
                                                              const double* invp, float* X,
                                                              uint32_t* amax_slot) {
  if (clip_dev) clip = *clip_dev;
  __shared__ float tile[64][65];
  const double inv = *invp;
  const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
  const int tr = threadIdx.x >> 2, tc = (threadIdx.x & 3) * 16;
  float x[16];
  if constexpr (TR) {
    // G row (c0 + tr), G columns (r0 + tc ..): X[r0 + tc + i][c0 + tr]
    uint32_t v[16];
    if (c0 + tr < xn && r0 + tc < xm) {
      load16_raw<T>(G, (c0 + tr) * xm + r0 + tc, v);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = 0u;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) tile[tc + i][tr] = __uint_as_float(v[i]);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = tile[tr][tc + i];
  } else {
    uint32_t v[16];
    if (r0 + tr < xm && c0 + tc < xn) {
      load16_raw<T>(G, (r0 + tr) * xn + c0 + tc, v);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = 0u;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = __uint_as_float(v[i]);
  }
  uint32_t amax = 0;
  if (r0 + tr < xm && c0 + tc < xn) {
    float y[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      y[i] = (float)((double)clampf(x[i], clip) * inv);
      uint32_t a = abs_bits(y[i]);
      amax = a > amax ? a : amax;
    }
    float4* o = reinterpret_cast<float4*>(X + (r0 + tr) * xn + c0 + tc);
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = make_float4(y[4 * j], y[4 * j + 1], y[4 * j + 2], y[4 * j + 3]);
  }
  amax_publish_block(amax, amax_slot);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((b >> 16) | 0x40u);
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

// out = X (xm x xn) or X^T (xn x xm); 64 x 64 tiles of X.
template <Dt O, bool TR>
__global__ __launch_bounds__(kThreads) void write_out_kernel(const float* X, int64_t xm, int64_t xn,
                                                              void* out) {
  __shared__ float tile[64][65];
  const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
  const int tr = threadIdx.x >> 2, tc = (threadIdx.x & 3) * 16;
  float y[16];
  int64_t orow, ocol, ocols;
  bool ok;
  if constexpr (TR) {
    const bool in = r0 + tr < xm && c0 + tc < xn;
#pragma unroll
    for (int i = 0; i < 16; ++i) tile[tr][tc + i] = in ? X[(r0 + tr) * xn + c0 + tc + i] : 0.0f;
    __syncthreads();
    // out row = X column c0 + tr, out columns = X rows r0 + tc ..
#pragma unroll
    for (int i = 0; i < 16; ++i) y[i] = tile[tc + i][tr];
    orow = c0 + tr; ocol = r0 + tc; ocols = xm;
    ok = orow < xn && ocol < xm;
  } else {
    ok = r0 + tr < xm && c0 + tc < xn;
    if (ok) {
      const float4* p = reinterpret_cast<const float4*>(X + (r0 + tr) * xn + c0 + tc);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float4 w = p[j];
        y[4 * j] = w.x; y[4 * j + 1] = w.y; y[4 * j + 2] = w.z; y[4 * j + 3] = w.w;
      }
    }
    orow = r0 + tr; ocol = c0 + tc; ocols = xn;
  }
  if (!ok) return;
  if constexpr (O == Dt::F32) {
    float4* o = reinterpret_cast<float4*>(static_cast<float*>(out) + orow * ocols + ocol);
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = make_float4(y[4 * j], y[4 * j + 1], y[4 * j + 2], y[4 * j + 3]);
  } else {
    uint4* o = reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + orow * ocols + ocol);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint32_t w[4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
        w[t] = (uint32_t)f32_to_bf16_rne(y[8 * j + 2 * t]) |
               ((uint32_t)f32_to_bf16_rne(y[8 * j + 2 * t + 1]) << 16);
      o[j] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

}  // namespace

hipError_t launch_norm_partials(const void* G, Dt gt, int64_t n, float clip, const float* clip_dev,
                                double* part, hipStream_t s) {
  const int64_t nblk = n / 16;
  if (gt == Dt::F32)
    norm_partials_kernel<Dt::F32><<<kNormParts, kThreads, 0, s>>>(G, nblk, clip, clip_dev, part);
  else
    norm_partials_kernel<Dt::BF16><<<kNormParts, kThreads, 0, s>>>(G, nblk, clip, clip_dev, part);
  return hipGetLastError();
}

hipError_t launch_norm_finalize(const double* part, double* inv, uint32_t* z0, uint32_t* z1,
                                uint32_t* z2, hipStream_t s) {
  norm_finalize_kernel<<<1, kThreads, 0, s>>>(part, inv, z0, z1, z2);
  return hipGetLastError();
}

hipError_t launch_normalize(const void* G, Dt gt, int64_t xm, int64_t xn, bool transposed,
                            float clip, const float* clip_dev, const double* inv, float* X,
                            uint32_t* amax_slot, hipStream_t s) {
  dim3 grid((unsigned)((xn + 63) / 64), (unsigned)((xm + 63) / 64));
  if (gt == Dt::F32) {
    if (transposed) normalize_kernel<Dt::F32, true><<<grid, kThreads, 0, s>>>(G, xm, xn, clip, clip_dev, inv, X, amax_slot);
    else normalize_kernel<Dt::F32, false><<<grid, kThreads, 0, s>>>(G, xm, xn, clip, clip_dev, inv, X, amax_slot);
  } else {
    if (transposed) normalize_kernel<Dt::BF16, true><<<grid, kThreads, 0, s>>>(G, xm, xn, clip, clip_dev, inv, X, amax_slot);
    else normalize_kernel<Dt::BF16, false><<<grid, kThreads, 0, s>>>(G, xm, xn, clip, clip_dev, inv, X, amax_slot);
  }
  return hipGetLastError();
}

hipError_t launch_write_out(const float* X, int64_t xm, int64_t xn, bool transposed, void* out,
                            Dt ot, hipStream_t s) {
  dim3 grid((unsigned)((xn + 63) / 64), (unsigned)((xm + 63) / 64));
  if (ot == Dt::F32) {
    if (transposed) write_out_kernel<Dt::F32, true><<<grid, kThreads, 0, s>>>(X, xm, xn, out);
    else write_out_kernel<Dt::F32, false><<<grid, kThreads, 0, s>>>(X, xm, xn, out);
  } else {
    if (transposed) write_out_kernel<Dt::BF16, true><<<grid, kThreads, 0, s>>>(X, xm, xn, out);
    else write_out_kernel<Dt::BF16, false><<<grid, kThreads, 0, s>>>(X, xm, xn, out);
  }
  return hipGetLastError();
}

}  // namespace nvfp4
