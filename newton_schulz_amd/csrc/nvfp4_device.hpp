// Device-side NVFP4 arithmetic for gfx950: exact encode of the E4M3 block
// scale and the E2M1 element codes, FP4 -> f16 dequantisation for the MFMA
// operands, and the NaN-propagating amax on float bit patterns.
//
// Format: Full-Stack FP4 (arXiv 2607.04422), §2 "NVFP4 format" — E2M1
// elements, one E4M3 scale per 16-block, one FP32 tensor scale, value =
// x_E2M1 * s * s_g.  RTN (round to nearest, ties to the even code) for
// every quantization, §3.4.
//
// Exactness.  s_g = RN_f32(amax / 2688) is one double division rounded to
// float (53 >= 2*24 + 2, so the double rounding is innocuous).  The block
// scale rounds the double quotient amax_b / (6 s_g) to E4M3 (again
// innocuous: 53 >= 2*4 + 2 + the extra bits of 6 s_g).  Element codes are
// decided without dividing: each E2M1 midpoint times s*s_g is exact in
// double (<= 3 + 4 + 24 bits) and is turned into the float bit pattern that
// an integer compare against |x|'s bits must exceed; ties go to the even
// code.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"

namespace nvfp4 {

// Four consecutive values (elements 4q .. 4q+3) as FP32 bit patterns (BF16
// widened exactly).  Kernels give consecutive lanes consecutive q, so each
// load instruction of a wave reads one contiguous run of memory: a gather of
// 16-byte pieces from many cache lines costs the texture unit one line
// lookup per lane and runs several times slower.
template <Dt T>
__device__ __forceinline__ uint4 load4(const void* base, int64_t q) {
  if constexpr (T == Dt::F32) {
    return reinterpret_cast<const uint4*>(base)[q];
  } else {
    const uint2 w = reinterpret_cast<const uint2*>(base)[q];
    return make_uint4(w.x << 16, w.x & 0xFFFF0000u, w.y << 16, w.y & 0xFFFF0000u);
  }
}

constexpr uint32_t kNaNBits = 0x7FC00000u;

// |v| as an ordered bit pattern; NaN and +-inf both map to the NaN pattern so
// that one non-finite element makes the tensor maximum NaN.
__device__ __forceinline__ uint32_t abs_bits(float v) {
  uint32_t b = __float_as_uint(v) & 0x7FFFFFFFu;
  return b >= 0x7F800000u ? kNaNBits : b;
}

__device__ __forceinline__ uint32_t abs_bits(uint32_t raw) {
  uint32_t b = raw & 0x7FFFFFFFu;
  return b >= 0x7F800000u ? kNaNBits : b;
}

// Tensor maxima are gathered in "amax slots": kAmaxParts partial words, one
// per 128-byte line.  Device-scope atomics on one address serialise (about
// 10 ns each on MI355X), so each workgroup folds one block-wide maximum into
// partial (workgroup index mod kAmaxParts) and readers take the maximum of
// the partials.  Values are |x| bit patterns (ordered like the magnitudes;
// NaN and infinity map to the NaN pattern, above every finite value).
constexpr int kAmaxParts = 16;
constexpr int kAmaxStride = 32;                        // words between partials
constexpr int kAmaxWords = kAmaxParts * kAmaxStride;   // words per slot

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t m) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t w = __shfl_xor(m, o, 64);
    m = w > m ? w : m;
  }
  return m;
}

// Block-wide maximum of m into `slot`: a partial of an amax slot
// (parts = true) or a single word (parts = false).  Every thread of the
// block must call it (it synchronises the block); at most 16 waves.
__device__ __forceinline__ void amax_publish_block(uint32_t m, uint32_t* slot, bool parts = true) {
  __shared__ uint32_t red[16];
  m = wave_max_u32(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    const int waves = (int)(blockDim.x + 63) >> 6;
    for (int w = 0; w < waves; ++w) r = red[w] > r ? red[w] : r;
    const unsigned b = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    if (r != 0u) atomicMax(parts ? slot + (b % kAmaxParts) * kAmaxStride : slot, r);
  }
}

// Wave-wide maximum of m into `slot`, without a block barrier (for kernels
// whose waves finish independently): lane 0 folds it into partial
// (global wave index mod kAmaxParts), or into the single word.
__device__ __forceinline__ void amax_publish_wave(uint32_t m, uint32_t* slot, bool parts = true) {
  m = wave_max_u32(m);
  if ((threadIdx.x & 63) == 0 && m != 0u) {
    const unsigned b = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    const unsigned w = b * ((blockDim.x + 63) >> 6) + (threadIdx.x >> 6);
    atomicMax(parts ? slot + (w % kAmaxParts) * kAmaxStride : slot, m);
  }
}

// Maximum over the partials of an amax slot.
__device__ __forceinline__ uint32_t amax_read(const uint32_t* slot) {
  uint32_t r = 0;
#pragma unroll
  for (int i = 0; i < kAmaxParts; ++i) {
    const uint32_t v = slot[i * kAmaxStride];
    r = v > r ? v : r;
  }
  return r;
}

// Zero an amax slot with the threads of one block.
__device__ __forceinline__ void amax_clear(uint32_t* slot) {
  for (int i = (int)threadIdx.x; i < kAmaxParts; i += (int)blockDim.x) slot[i * kAmaxStride] = 0u;
}

// s_g = RN_f32(amax / (6 * 448)); NaN stays NaN.
__device__ __forceinline__ float global_scale_from_amax(uint32_t amax_bits) {
  if (amax_bits > 0x7F800000u) return __uint_as_float(kNaNBits);
  return (float)((double)__uint_as_float(amax_bits) / 2688.0);
}

// E4M3FN byte (0x00..0x7E) -> value, as double (exact).
__device__ __forceinline__ double e4m3_value(uint32_t byte) {
  uint32_t e = byte >> 3, m = byte & 7u;
  return e == 0 ? (double)m * 0x1p-9 : ldexp((double)(8u + m), (int)e - 10);
}

// RNE to E4M3FN of a non-negative finite double, saturating at 448 (0x7E).
// The double is split into its binade E (clamped to the subnormal binade
// -6) and scaled by a power of two so that one E4M3 ulp is 1; rint() then
// rounds half to even, and a carry out of the mantissa moves the exponent.
__device__ __forceinline__ uint32_t e4m3_rne_sat(double q) {
  if (!(q < 448.0)) return 0x7Eu;
  int E = (int)((__double_as_longlong(q) >> 52) & 0x7FF) - 1023;
  E = E < -6 ? -6 : E;
  int r = (int)rint(ldexp(q, 3 - E));
  return (uint32_t)(((E + 7) << 3) + r - 8);
}

// Bit pattern of the largest float <= d and of the smallest float >= d
// (d > 0 finite).
__device__ __forceinline__ uint32_t floor_f32_bits(double d) {
  float f = (float)d;
  uint32_t b = __float_as_uint(f);
  return ((double)f > d) ? b - 1u : b;
}
__device__ __forceinline__ uint32_t ceil_f32_bits(double d) {
  float f = (float)d;
  uint32_t b = __float_as_uint(f);
  return ((double)f < d) ? b + 1u : b;
}

// Integer thresholds of one block: magnitude code = number of k with
// bits(|x|) > t_k.  Midpoint k lies between codes k and k+1: for even k
// the value must exceed it (tie stays on the even code k), for odd k it
// must reach it (tie moves to the even code k+1).  Seven named fields, not
// an array, so that nothing is indexed at run time.
struct BlockThresholds {
  uint32_t t0, t1, t2, t3, t4, t5, t6;
};

__device__ __forceinline__ uint32_t midpoint_threshold(double mid, double unit, bool odd) {
  const double thr = mid * unit;            // exact
  return odd ? ceil_f32_bits(thr) - 1u : floor_f32_bits(thr);
}

__device__ __forceinline__ BlockThresholds block_thresholds(double unit /* s * s_g */) {
  BlockThresholds T;
  if (!(unit > 0.0)) {                      // zero scale, zero or NaN s_g
    T.t0 = T.t1 = T.t2 = T.t3 = T.t4 = T.t5 = T.t6 = 0xFFFFFFFFu;
    return T;
  }
  // E2M1 midpoints 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5
  T.t0 = midpoint_threshold(0.25, unit, false);
  T.t1 = midpoint_threshold(0.75, unit, true);
  T.t2 = midpoint_threshold(1.25, unit, false);
  T.t3 = midpoint_threshold(1.75, unit, true);
  T.t4 = midpoint_threshold(2.5, unit, false);
  T.t5 = midpoint_threshold(3.5, unit, true);
  T.t6 = midpoint_threshold(5.0, unit, false);
  return T;
}

// 4-bit code of one element (sign bit from the raw float bits): the
// magnitude is the count of thresholds below |x|.
__device__ __forceinline__ uint32_t encode_element(uint32_t raw_bits, const BlockThresholds& T) {
  const uint32_t a = raw_bits & 0x7FFFFFFFu;
  const uint32_t c = (uint32_t)(a > T.t0) + (uint32_t)(a > T.t1) + (uint32_t)(a > T.t2) +
                     (uint32_t)(a > T.t3) + (uint32_t)(a > T.t4) + (uint32_t)(a > T.t5) +
                     (uint32_t)(a > T.t6);
  return c | ((raw_bits >> 28) & 8u);
}

// RNE to E4M3FN of a non-negative finite float, saturating at 448 (0x7E).
// Below 2^-6 the E4M3 grid is uniform with step 2^-9, so the byte is the
// RNE integer of x * 2^9 (a value of 8 is the byte of 2^-6); above, the
// float's mantissa is rounded to 3 bits in place (a carry moves the
// exponent) and the exponent rebased from 127 to 7.
__device__ __forceinline__ uint32_t e4m3_rne_sat_f32(float x) {
  if (!(x < 448.0f)) return 0x7Eu;
  if (x < 0x1p-6f) return (uint32_t)__builtin_rintf(x * 512.0f);
  const uint32_t b = __float_as_uint(x);
  return ((b + 0x7FFFFu + ((b >> 20) & 1u)) >> 20) - ((127u - 7u) << 3);
}

// Scale byte of a block with maximum |x| = amax_b (as float bits) under s_g,
// the block maximum mapped to M (6; 4 for the adaptive 4/6 candidate):
// RNE_E4M3FN(amax_b / (M s_g)) of the exact quotient, saturating at 448.
// Fast path: the float quotient through the hardware reciprocal is within
// 2^-22 relative of the exact one; widened by 2^-19 either way it brackets
// it, and when both ends round to the same byte (rounding is monotone) that
// byte is exact.  Otherwise, or for extreme s_g, the exact double quotient
// decides.
template <int M>
__device__ __forceinline__ uint32_t block_scale_byte_m(uint32_t amax_b_bits, float sg) {
  if (sg != sg) return 0x7Fu;               // NaN tensor
  if (sg == 0.0f) return 0u;
  if (sg > 0x1p-100f && sg < 0x1p100f) {
    const float q = __uint_as_float(amax_b_bits) * __builtin_amdgcn_rcpf((float)M * sg);
    const uint32_t lo = e4m3_rne_sat_f32(q * (1.0f - 0x1p-19f));
    const uint32_t hi = e4m3_rne_sat_f32(q * (1.0f + 0x1p-19f));
    if (lo == hi) return lo;
  }
  const double q = (double)__uint_as_float(amax_b_bits) / ((double)M * (double)sg);
  return e4m3_rne_sat(q);
}
__device__ __forceinline__ uint32_t block_scale_byte(uint32_t amax_b_bits, float sg) {
  return block_scale_byte_m<6>(amax_b_bits, sg);
}

// Exact encode of 16 values by thresholds (the reference rule above).
__device__ __forceinline__ void encode_block16_exact(const uint32_t (&v)[16], float sg, uint32_t scale,
                                                  uint32_t& lo, uint32_t& hi) {
  const double unit = (scale == 0x7Fu) ? 0.0 : e4m3_value(scale) * (double)sg;
  const BlockThresholds T = block_thresholds(unit);
  lo = 0;
  hi = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) lo |= encode_element(v[i], T) << (4 * i);
#pragma unroll
  for (int i = 0; i < 8; ++i) hi |= encode_element(v[8 + i], T) << (4 * i);
}

// Encode 16 values given as raw float bit patterns.  Returns the packed
// codes (element 2i in the low nibble of byte i) and the scale byte.
//
// Fast path: the hardware f32 -> E2M1 conversion (RNE, ties to even,
// saturating at 6, sign kept — measured on gfx950) is applied to x times two
// approximations of 1/(s*s_g), one below and one above by ~2^-19 relative.
// The exact quotient |x|/(s*s_g) lies strictly between the two products, and
// rounding is monotone, so when both give the same code that code is the
// exact RNE of the quotient.  A block where any element's two codes differ
// (a tie or a near-tie), or whose s*s_g is outside [2^-120, 2^120], is
// encoded by the exact threshold rule instead.
__device__ __forceinline__ void encode_codes16(const uint32_t (&v)[16], float sg, uint32_t scale,
                                              uint32_t& lo, uint32_t& hi) {
  const float s = (scale == 0x7Fu) ? 0.0f : __builtin_amdgcn_cvt_f32_fp8((int)scale, 0);
  const float unit = s * sg;
  if (unit > 0x1p-120f && unit < 0x1p120f) {
    const float r = __builtin_amdgcn_rcpf(unit);          // within 1 ulp of 1/unit
    const float rl = r * (1.0f - 0x1p-19f), rh = r * (1.0f + 0x1p-19f);
    uint32_t l0 = 0, l1 = 0, h0 = 0, h1 = 0;
#define NVFP4_PAIR(dl, dh, i, sel)                                                              \
    dl = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(dl, __uint_as_float(v[i]) * rl,              \
                                                  __uint_as_float(v[i + 1]) * rl, 1.0f, sel);  \
    dh = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(dh, __uint_as_float(v[i]) * rh,              \
                                                  __uint_as_float(v[i + 1]) * rh, 1.0f, sel)
    NVFP4_PAIR(l0, h0, 0, 0);
    NVFP4_PAIR(l0, h0, 2, 1);
    NVFP4_PAIR(l0, h0, 4, 2);
    NVFP4_PAIR(l0, h0, 6, 3);
    NVFP4_PAIR(l1, h1, 8, 0);
    NVFP4_PAIR(l1, h1, 10, 1);
    NVFP4_PAIR(l1, h1, 12, 2);
    NVFP4_PAIR(l1, h1, 14, 3);
#undef NVFP4_PAIR
    if (l0 == h0 && l1 == h1) {
      lo = l0;
      hi = l1;
      return;
    }
  }
  encode_block16_exact(v, sg, scale, lo, hi);
}

__device__ __forceinline__ uint32_t block_amax_bits(const uint32_t (&v)[16]) {
  uint32_t amax_b = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t a = v[i] & 0x7FFFFFFFu;
    amax_b = a > amax_b ? a : amax_b;
  }
  return amax_b;
}

__device__ __forceinline__ void encode_block16(const uint32_t (&v)[16], float sg,
                                               uint32_t& lo, uint32_t& hi, uint32_t& scale) {
  scale = block_scale_byte(block_amax_bits(v), sg);
  encode_codes16(v, sg, scale, lo, hi);
}

// Signed E2M1 values of a block's 16 codes (element 2i in the low nibble of
// byte i of lo:hi), exact in FP32: the hardware conversion at unit scale.
__device__ __forceinline__ void decode_codes16(uint32_t lo, uint32_t hi, float (&q)[16]) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 p[8] = {
      __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(lo, 1.0f, 0),
      __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(lo, 1.0f, 1),
      __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(lo, 1.0f, 2),
      __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(lo, 1.0f, 3),
      __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(hi, 1.0f, 0),
      __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(hi, 1.0f, 1),
      __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(hi, 1.0f, 2),
      __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(hi, 1.0f, 3)};
#pragma unroll
  for (int i = 0; i < 16; ++i) q[i] = p[i >> 1][i & 1];
}

// Squared error of a block's encoding: the sum over its 16 elements, in
// element order, of (x - q s s_g)^2, each difference, square and sum rounded
// in double (no fused multiply-add, so that the comparison below is the one
// the plain definition makes).  q s s_g is exact in double.
__device__ __forceinline__ double block_sq_error(const uint32_t (&v)[16], float sg, uint32_t scale,
                                                 uint32_t lo, uint32_t hi) {
#pragma clang fp contract(off)
  const double unit = e4m3_value(scale) * (double)sg;
  float q[16];
  decode_codes16(lo, hi, q);
  double e = 0.0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const double d = (double)__uint_as_float(v[i]) - (double)q[i] * unit;   // exact product
    e = e + d * d;
  }
  return e;
}

// The same sum in FP32, for screening: q s is exact in FP32 (at most six
// significant bits), so each difference x - (q s) s_g is rounded once (fma),
// and each square is added with one rounding.  The result is within
// 18.1 * 2^-24 of the exact sum relatively, plus 2^-121 absolutely for
// results in FP32's subnormal range, unless it overflowed.
__device__ __forceinline__ float block_sq_error_f32(const uint32_t (&v)[16], float sg,
                                                    uint32_t scale, uint32_t lo, uint32_t hi) {
  const float s = __builtin_amdgcn_cvt_f32_fp8((int)scale, 0);
  float q[16];
  decode_codes16(lo, hi, q);
  float e = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float d = __builtin_fmaf(q[i] * s, -sg, __uint_as_float(v[i]));
    e = __builtin_fmaf(d, d, e);
  }
  return e;
}

// Whether the M = 4 encoding (s4, lo4, hi4) has the strictly smaller squared
// error, as block_sq_error decides it.  The FP32 sums decide whenever they
// differ by more than their error bounds (relative 2^-18 is above
// 18.1 * 2^-24 with room for the rounding of the bounds themselves, and
// 2^-120 covers the subnormal range); otherwise the double sums decide.
__device__ __forceinline__ bool four_is_better(const uint32_t (&v)[16], float sg, uint32_t s6,
                                               uint32_t lo6, uint32_t hi6, uint32_t s4,
                                               uint32_t lo4, uint32_t hi4) {
  const float e6 = block_sq_error_f32(v, sg, s6, lo6, hi6);
  const float e4 = block_sq_error_f32(v, sg, s4, lo4, hi4);
  constexpr float kRel = 0x1p-18f, kAbs = 0x1p-120f, kMax = 0x1.fffffep127f;
  if (e4 <= kMax && e6 <= kMax) {
    if (e4 * (1.0f + kRel) + kAbs < e6 * (1.0f - kRel) - kAbs) return true;
    if (e4 * (1.0f - kRel) - kAbs > e6 * (1.0f + kRel) + kAbs) return false;
  }
  return block_sq_error(v, sg, s4, lo4, hi4) < block_sq_error(v, sg, s6, lo6, hi6);
}

// Adaptive 4/6 block scaling (the Root quantizations of Full-Stack FP4,
// §3.4; adaptive M = 4 / M = 6 block scaling of Four Over Six): the block is
// encoded with its maximum mapped to 6 and to 4 and keeps the encoding with
// the smaller squared error; M = 6 on ties (and when s_g is NaN or zero, or
// both candidates share a scale).  s_g is that of plain NVFP4.
__device__ __forceinline__ void encode_block16_46(const uint32_t (&v)[16], float sg,
                                                  uint32_t& lo, uint32_t& hi, uint32_t& scale) {
  const uint32_t amax_b = block_amax_bits(v);
  scale = block_scale_byte_m<6>(amax_b, sg);
  encode_codes16(v, sg, scale, lo, hi);
  if (!(sg > 0.0f) || scale == 0x7Fu) return;
  const uint32_t s4 = block_scale_byte_m<4>(amax_b, sg);
  if (s4 == scale) return;
  uint32_t lo4, hi4;
  encode_codes16(v, sg, s4, lo4, hi4);
  if (four_is_better(v, sg, scale, lo, hi, s4, lo4, hi4)) {
    lo = lo4;
    hi = hi4;
    scale = s4;
  }
}

// Codes of the EPL (4 or 8) elements one lane holds of a block whose scale
// byte is known: the same bracketed fast path as encode_block16, falling
// back to the exact thresholds for this lane's elements.  Returns EPL
// nibbles, element 2i in the low nibble of byte i.
template <int EPL>
__device__ __forceinline__ uint32_t encode_lane(const uint32_t (&v)[EPL], float sg, uint32_t scale) {
  const float s = (scale == 0x7Fu) ? 0.0f : __builtin_amdgcn_cvt_f32_fp8((int)scale, 0);
  const float unit = s * sg;
  if (unit > 0x1p-120f && unit < 0x1p120f) {
    const float r = __builtin_amdgcn_rcpf(unit);
    const float rl = r * (1.0f - 0x1p-19f), rh = r * (1.0f + 0x1p-19f);
    uint32_t l = 0, h = 0;
#pragma unroll
    for (int p = 0; p < EPL / 2; ++p) {
      const float x0 = __uint_as_float(v[2 * p]), x1 = __uint_as_float(v[2 * p + 1]);
      switch (p) {   // the byte selector must be a constant
        case 0: l = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(l, x0 * rl, x1 * rl, 1.0f, 0);
                h = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(h, x0 * rh, x1 * rh, 1.0f, 0); break;
        case 1: l = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(l, x0 * rl, x1 * rl, 1.0f, 1);
                h = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(h, x0 * rh, x1 * rh, 1.0f, 1); break;
        case 2: l = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(l, x0 * rl, x1 * rl, 1.0f, 2);
                h = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(h, x0 * rh, x1 * rh, 1.0f, 2); break;
        default: l = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(l, x0 * rl, x1 * rl, 1.0f, 3);
                 h = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(h, x0 * rh, x1 * rh, 1.0f, 3); break;
      }
    }
    if (l == h) return l;
  }
  const double unitd = (scale == 0x7Fu) ? 0.0 : e4m3_value(scale) * (double)sg;
  const BlockThresholds T = block_thresholds(unitd);
  uint32_t c = 0;
#pragma unroll
  for (int e = 0; e < EPL; ++e) c |= encode_element(v[e], T) << (4 * e);
  return c;
}

// ------------------------------------------------ random Hadamard, 16 ----

// One 16-block (raw float bits, in place) times H^r = diag(s) H_16 / 4, the
// random Hadamard transform of the NVFP4 NS iteration (Full-Stack FP4,
// §3.4): sign j flipped where bit j of `mask` is set, then the radix-2
// butterfly of the Sylvester matrix H_16 with half-widths 1, 2, 4, 8 --
// each pair (a, b) -> (a + b, a - b) rounded to nearest even in FP32 -- and
// a final multiplication by 1/4.  The fixed order makes the transformed
// values, and so the codes, reproducible bit for bit.
__device__ __forceinline__ void rht16(uint32_t (&v)[16], uint32_t mask) {
  float f[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) f[j] = __uint_as_float(v[j] ^ (((mask >> j) & 1u) << 31));
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i & h) continue;
      const float a = f[i], b = f[i + h];
      f[i] = a + b;
      f[i + h] = a - b;
    }
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = __float_as_uint(f[j] * 0.25f);
}

// ---------------------------------------------------------------- decode --

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));

// Scale byte -> f16 pair (s, s).  The hardware FP8 decode is exact and
// gfx950 decodes OCP E4M3FN; every E4M3 value is an f16 number.
__device__ __forceinline__ half2_t scale_pair_f16(uint32_t byte) {
  float s = __builtin_amdgcn_cvt_f32_fp8((int)byte, 0);
  _Float16 h = (_Float16)s;
  half2_t r = {h, h};
  return r;
}

// Bytes 2w and 2w+1 of a dword of E4M3 scale bytes as an f16 pair (the
// hardware FP8 decode with unit scale is exact).
__device__ __forceinline__ half2_t scale_pair2_f16(uint32_t dword, int w) {
  return w == 0 ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(dword, 1.0f, false)
                : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(dword, 1.0f, true);
}
__device__ __forceinline__ half2_t splat_lo(half2_t v) { half2_t r = {v[0], v[0]}; return r; }
__device__ __forceinline__ half2_t splat_hi(half2_t v) { half2_t r = {v[1], v[1]}; return r; }

// Eight E2M1 codes (one dword, element 2i in the low nibble of byte i) times
// the block scale, as eight f16 values.  The conversion instruction yields
// the exact E2M1 value (its scale operand is 1); the packed f16 multiply is
// exact because q*s has at most 6 significant bits and lies in
// [2^-10, 2688], inside the normal f16 range.
__device__ __forceinline__ half8_t dequant8_f16(uint32_t w, half2_t s2) {
  half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
  half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
  half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
  half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
  half8_t r = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
  return r;
}

}  // namespace nvfp4
