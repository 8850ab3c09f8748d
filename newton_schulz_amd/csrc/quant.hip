// NVFP4 quantizer and dequantizer kernels for gfx950.
//
// Q_1x16 / Q_16x1 of Full-Stack FP4 (arXiv 2607.04422), §2 "NVFP4 format"
// and §3.4: a per-tensor maximum (first pass, HBM-bound read), then per
// 16-block an E4M3 scale and sixteen E2M1 codes (second pass).  The exact
// rounding rules live in nvfp4_device.hpp.
#include <climits>
#include <cstdint>
#include <type_traits>

#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

static_assert(kAmaxSlotWords == kAmaxWords, "amax slot size");

namespace {

constexpr int kThreads = 256;
// Workgroups of the grid-stride passes at most: 2048 (eight per CU) suits
// tensors of tens of MB such as the NS iteration's A and B; from 16 Mi
// 16-byte vectors (256 MB) on, 8192 keep more loads in flight (measured on
// 16384^2 BF16: quantize 258 -> 245 us, dequantize 147 -> 142 us; on
// 3072^2 FP32 the larger grid costs 0.5 us).
constexpr int kMaxGrid = 256 * 8;
constexpr int kMaxGridLarge = 256 * 32;
constexpr int64_t kLargeVectors = (int64_t)1 << 24;
// Items per lane per trip of the row encode and decode passes: with
// non-temporal accesses two keep enough in flight (2^28 BF16 values: pair
// 351 us, against 360 with four, 368 with eight and 435 with one).
#ifndef NVFP4_QUANT_UNROLL
#define NVFP4_QUANT_UNROLL 2
#endif
constexpr int kUnroll = NVFP4_QUANT_UNROLL;     // items per lane per trip
// The tensor-maximum pass reads contiguous chunks, one per workgroup (the
// tensor cut into rounds of kThreads 16-byte vectors, workgroup b taking
// rounds [b R / grid, (b + 1) R / grid)), with kAmaxUnroll loads in flight
// per lane: on 2^28 BF16 values 84-108 us against 101-128 us for the
// grid-stride walk (measured, MI355X).  The encode and decode passes keep
// the grid-stride walk with many more workgroups: they carry enough ALU
// work per item that chunks of 512 workgroups ran at half their speed.
#ifndef NVFP4_AMAX_GRID
#define NVFP4_AMAX_GRID 512
#endif
#ifndef NVFP4_AMAX_UNROLL
#define NVFP4_AMAX_UNROLL 8
#endif
constexpr int kAmaxUnroll = NVFP4_AMAX_UNROLL;
constexpr int64_t kCachedTailBytes = (int64_t)96 << 20;

typedef float float2_t __attribute__((ext_vector_type(2)));
// Streaming accesses of the standalone quantizer's passes, with the
// non-temporal hint: a tensor larger than the Infinity Cache (256 MB) is
// read once per pass and its decoded values written once, so nothing is
// gained by keeping those lines.  On 2^28 BF16 values (MI355X) the hint took
// the quantize + dequantize pair from 403 to 359 us: the decode pass with
// non-temporal stores from 143 to 110 us, the encode pass from 250 to 238
// us with non-temporal loads; outputs unchanged.
//
// What the cache does keep is chosen: the maximum pass reads the last
// kCachedTailBytes of the tensor last, with ordinary (allocating) loads, and
// the encode pass, which walks from the end, reads that tail first, so it
// comes from the cache; the encode pass stores its codes with ordinary
// stores, last-written at the tensor's start, where a decode pass run next
// begins.  Tail and codes (151 MB for 2^28 values) must fit the cache
// together.  Measured on 2^28 BF16 values, interleaved runs on one MI355X:
// the pair 347-348 us with every access non-temporal; 330 us with ordinary
// code stores; with those and a cached tail of 64 / 96 / 128 / 192 MB 322 /
// 320 / 335 / 356 us (a 192 MB tail without the code stores 339 us).
typedef unsigned int nt_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  const nt_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_nt(uint4* p, uint4 r) {
  const nt_u32x4 v = {r.x, r.y, r.z, r.w};
  __builtin_nontemporal_store(v, reinterpret_cast<nt_u32x4*>(p));
}


// 16 consecutive elements starting at element `idx` (a multiple of 16) as
// raw float bit patterns (BF16 widened exactly).
template <Dt T>
__device__ __forceinline__ void load16(const void* base, int64_t idx, uint32_t (&v)[16]) {
  if constexpr (T == Dt::F32) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(base) + idx);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint4 w = p[j];
      v[4 * j + 0] = w.x; v[4 * j + 1] = w.y; v[4 * j + 2] = w.z; v[4 * j + 3] = w.w;
    }
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + idx);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint4 w = p[j];
      uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        v[8 * j + 2 * t + 0] = ws[t] << 16;
        v[8 * j + 2 * t + 1] = ws[t] & 0xFFFF0000u;
      }
    }
  }
}

// 64x64 tiles on a one-dimensional grid (a second grid dimension would cap
// the rows at 65535 tiles): workgroup b takes tile row b / tiles_x and tile
// column b % tiles_x, row-major, the order a two-dimensional grid runs in.
__device__ __forceinline__ int64_t tile_row0(uint32_t tiles_x) {
  return (int64_t)(blockIdx.x / tiles_x) * 64;
}
__device__ __forceinline__ int64_t tile_col0(uint32_t tiles_x) {
  return (int64_t)(blockIdx.x % tiles_x) * 64;
}
// Tiles per row and the grid of a rows x cols tensor; false if the tile
// count does not fit a grid.
inline bool tile_grid(int64_t rows, int64_t cols, uint32_t& tiles_x, uint32_t& grid) {
  const int64_t tx = (cols + 63) / 64, tiles = tx * ((rows + 63) / 64);
  if (tiles <= 0 || tiles > INT32_MAX) return false;
  tiles_x = (uint32_t)tx;
  grid = (uint32_t)tiles;
  return true;
}

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint32_t w = __shfl_xor(v, o, 64);
    v = w > v ? w : v;
  }
  return v;
}

// ---------------------------------------------------------------- amax ----

template <Dt T>
__global__ __launch_bounds__(kThreads) void amax_kernel(const void* x, int64_t nvec, uint32_t* slot) {
  // nvec = number of 16-byte vectors; each holds 4 (F32) or 8 (BF16) values
  const uint4* p = static_cast<const uint4*>(x);
  uint32_t m = 0;
  auto fold = [&](uint4 w) {
    uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if constexpr (T == Dt::F32) {
        uint32_t a = abs_bits(ws[t]);
        m = a > m ? a : m;
      } else {
        uint32_t a0 = abs_bits(ws[t] << 16), a1 = abs_bits(ws[t] & 0xFFFF0000u);
        m = a0 > m ? a0 : m;
        m = a1 > m ? a1 : m;
      }
    }
  };
  // this workgroup's chunk of the rounds of [v0, v1), kAmaxUnroll 16-byte
  // loads in flight per lane
  auto walk = [&](int64_t v0, int64_t v1, auto cached) {
    auto ld = [&](int64_t k) {
      if constexpr (decltype(cached)::value) return p[k];
      else return load_nt(p + k);
    };
    const int64_t rounds = (v1 - v0 + kThreads - 1) / kThreads;
    const int64_t r0 = rounds * blockIdx.x / gridDim.x, r1 = rounds * (blockIdx.x + 1) / gridDim.x;
    const int64_t e = v0 + r1 * kThreads < v1 ? v0 + r1 * kThreads : v1;
    int64_t i = v0 + r0 * kThreads + threadIdx.x;
    for (; i + (kAmaxUnroll - 1) * kThreads < e; i += kAmaxUnroll * kThreads) {
      uint4 w[kAmaxUnroll];
#pragma unroll
      for (int u = 0; u < kAmaxUnroll; ++u) w[u] = ld(i + u * kThreads);
#pragma unroll
      for (int u = 0; u < kAmaxUnroll; ++u) fold(w[u]);
    }
    for (; i < e; i += kThreads) fold(ld(i));
  };
  // the body streams; the tail, read last, is left in the Infinity Cache
  // for the encode pass
  const int64_t tail = nvec < kCachedTailBytes / 16 ? nvec : kCachedTailBytes / 16;
  walk(0, nvec - tail, std::false_type{});
  walk(nvec - tail, nvec, std::true_type{});
  amax_publish_block(m, slot);
}

// ------------------------------------------------------- row quantizer ----

// Maximum over the G lanes of an aligned lane group (G = 2 or 4), on the
// DPP crossbar: quad_perm [1,0,3,2] swaps lanes 2k and 2k+1, [2,3,0,1]
// lanes 4k+j and 4k+j+2.  Every lane of a group is active or none is.
template <int G>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t m) {
  uint32_t t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0xB1, 0xF, 0xF, false);
  m = t > m ? t : m;
  if constexpr (G == 4) {
    t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x4E, 0xF, 0xF, false);
    m = t > m ? t : m;
  }
  return m;
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Each lane owns 16 bytes of input (8 BF16 or 4 FP32 values), so every
// load instruction of a wave reads one contiguous kilobyte; the 2 or 4
// lanes of a block combine their maxima across the DPP crossbar.  The grid
// walks the tensor from its end to its start: the amax pass just read it
// front to back, so the last part it read may still be in the Infinity
// Cache.  Lane i takes item items - 1 - (i xor (G - 1)): blocks in reverse
// order, the lanes of a block in their own order.  Since the grid stride
// is a multiple of G, a lane's next item is exactly one stride lower, so
// the loop steps one index instead of recomputing it per access.
template <Dt T>
__global__ __launch_bounds__(kThreads) void quant_rows_kernel(
    const void* x, int64_t nelem, const uint32_t* amax_slot, float* sg_out,
    uint8_t* codes, uint8_t* scales, uint32_t* zero_slot) {
  constexpr int EPL = T == Dt::F32 ? 4 : 8;   // elements per lane
  constexpr int G = 16 / EPL;                 // lanes per block
  constexpr int LOG_G = G == 2 ? 1 : 2;
  using Word = typename std::conditional<EPL == 8, uint32_t, uint16_t>::type;
  const float sg = global_scale_from_amax(amax_read(amax_slot));
  if (blockIdx.x == 0) {
    if (sg_out && threadIdx.x == 0) *sg_out = sg;
    if (zero_slot) amax_clear(zero_slot);
  }
  const int64_t items = nelem / EPL;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  const bool first = (threadIdx.x & (G - 1)) == 0;   // the lane that stores the scale
  const uint4* src = reinterpret_cast<const uint4*>(x);
  Word* dst = reinterpret_cast<Word*>(codes);
  auto encode_item = [&](int64_t item, uint4 w) {
    uint32_t v[EPL];
    uint32_t amax;
    if constexpr (T == Dt::F32) {
      v[0] = w.x; v[1] = w.y; v[2] = w.z; v[3] = w.w;
      amax = 0;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const uint32_t a = v[e] & 0x7FFFFFFFu;
        amax = a > amax ? a : amax;
      }
    } else {
      // the eight BF16 magnitudes compared as 16-bit pairs; a BF16 value's
      // bits shifted up 16 are its FP32 bits, so the order is the same
      u16x2 m = __builtin_bit_cast(u16x2, w.x & 0x7FFF7FFFu);
      m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w.y & 0x7FFF7FFFu));
      m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w.z & 0x7FFF7FFFu));
      m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w.w & 0x7FFF7FFFu));
      amax = (uint32_t)(m[0] > m[1] ? m[0] : m[1]) << 16;
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int t = 0; t < 4; ++t) { v[2 * t] = ws[t] << 16; v[2 * t + 1] = ws[t] & 0xFFFF0000u; }
    }
    amax = group_max_u32<G>(amax);
    const uint32_t sc = block_scale_byte(amax, sg);
    const uint32_t c = encode_lane<EPL>(v, sg, sc);
    dst[item] = (Word)c;
    if (first) scales[item >> LOG_G] = (uint8_t)sc;
  };
  // kUnroll items per lane per trip, all loads issued before any is encoded,
  // so that each lane keeps kUnroll * 16 bytes in flight
  // the tensor's last kCachedTailBytes, which the maximum pass read last,
  // come first in this walk and are read from the Infinity Cache
  const int64_t tail_start = items - kCachedTailBytes / 16;
  auto load_item = [&](int64_t k) { return k >= tail_start ? src[k] : load_nt(src + k); };
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  int64_t item = items - 1 - (i ^ (G - 1));
  for (; i + (kUnroll - 1) * stride < items; i += kUnroll * stride, item -= kUnroll * stride) {
    uint4 w[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) w[u] = load_item(item - u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) encode_item(item - u * stride, w[u]);
  }
  for (; i < items; i += stride, item -= stride) encode_item(item, load_item(item));
}

// ------------------------------------------- tiled quantizer, both axes ----
// One 64x64 tile per workgroup.  Thread t holds row t/4, columns
// 16*(t%4)..+15 of the tile: that is one Q_1x16 block, encoded straight from
// registers.  For Q_16x1 the tile goes through LDS and thread t encodes
// column t/4, rows 16*(t%4)..+15.  With `rht` every block is first replaced
// by its random Hadamard transform (rht16), and the column layout may take
// its own tensor scale (amax_c, sg_out_c) since X H and H^T X differ.

// With NORM the input is G and each loaded value is first normalised,
// y = RN_f32(clamp(g, -clip, clip) * inv) -- the value the NS normalisation
// writes -- and X = y is stored beside the codes.
// With `sym` the input is a symmetric square matrix of which only the tiles
// on or above the diagonal are read (the GEMM left the rest unwritten):
// tile (I, J), I < J, encodes its rows into the row layout at (I, J) and its
// columns into the row layout at (J, I), which holds the same blocks since
// tile (J, I) is the transpose of tile (I, J); col_codes and col_scales are
// then the row buffers themselves, and a diagonal tile encodes its rows only.

struct NormArg {
  float clip;
  const float* clip_dev;   // device clip, used when not null
  const double* inv;       // 1 / (||clamp(G)||_F + eps)
  float* X;
};

// clamp that lets NaN through
__device__ __forceinline__ float clamp_nan(float x, float c) {
  return x > c ? c : (x < -c ? -c : x);
}

template <class P>
__device__ __forceinline__ P* shift_bytes(P* p, int64_t off) {
  return p ? reinterpret_cast<P*>(reinterpret_cast<uintptr_t>(p) + off) : p;
}

// With bstride != 0 the launch covers one tensor per grid row y, each at
// the same byte offsets as tensor 0 plus y * bstride (every pointer moves).
template <Dt T, bool ROWS, bool COLS, bool NORM = false>
__global__ __launch_bounds__(kThreads) void quant_tile_kernel(
    const void* x, int64_t rows, int64_t cols, uint32_t tiles_x, const uint32_t* amax_slot,
    float* sg_out, uint8_t* row_codes, uint8_t* row_scales, uint8_t* col_codes,
    uint8_t* col_scales, uint32_t* zero_slot, const uint32_t* amax_c, float* sg_out_c,
    RhtArg rht, NormArg nrm, uint32_t sym, int64_t bstride) {
  static_assert(!NORM || COLS, "the normalised X is written from the LDS tile");
  __shared__ uint32_t tile[64][65];
  if (bstride) {
    const int64_t off = (int64_t)blockIdx.y * bstride;
    x = shift_bytes(x, off);
    amax_slot = shift_bytes(amax_slot, off);
    sg_out = shift_bytes(sg_out, off);
    row_codes = shift_bytes(row_codes, off);
    row_scales = shift_bytes(row_scales, off);
    col_codes = shift_bytes(col_codes, off);
    col_scales = shift_bytes(col_scales, off);
    zero_slot = shift_bytes(zero_slot, off);
    amax_c = shift_bytes(amax_c, off);
    sg_out_c = shift_bytes(sg_out_c, off);
  }
  const float sg = global_scale_from_amax(amax_read(amax_slot));
  const float sgc = amax_c ? global_scale_from_amax(amax_read(amax_c)) : sg;
  if (blockIdx.x == 0) {
    if (threadIdx.x == 0) {
      if (sg_out) *sg_out = sg;
      if (sg_out_c) *sg_out_c = sgc;
    }
    if (zero_slot) amax_clear(zero_slot);
  }
  const int64_t r0 = tile_row0(tiles_x), c0 = tile_col0(tiles_x);
  if (sym && r0 > c0) return;   // below the diagonal: done by tile (J, I)
  const int tr = threadIdx.x >> 2, tc = (threadIdx.x & 3) * 16;
  const bool in = (r0 + tr < rows) && (c0 + tc < cols);
  uint32_t v[16];
  if (in) {
    load16<T>(x, (r0 + tr) * cols + c0 + tc, v);
    if constexpr (NORM) {
      const float clip = nrm.clip_dev ? *nrm.clip_dev : nrm.clip;
      const double inv = *nrm.inv;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        v[i] = __float_as_uint((float)((double)clamp_nan(__uint_as_float(v[i]), clip) * inv));
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = 0u;
  }
  if constexpr (COLS) {
#pragma unroll
    for (int i = 0; i < 16; ++i) tile[tr][tc + i] = v[i];
  }
  if constexpr (ROWS) {
    if (in) {
      if (rht.on) rht16(v, rht.mask);
      uint32_t lo, hi, sc;
      if (rht.adaptive46) encode_block16_46(v, sg, lo, hi, sc);
      else encode_block16(v, sg, lo, hi, sc);
      const int64_t e = (r0 + tr) * cols + c0 + tc;
      reinterpret_cast<uint2*>(row_codes)[e / 16] = make_uint2(lo, hi);
      row_scales[e / 16] = (uint8_t)sc;
    }
  }
  if constexpr (COLS) {
    __syncthreads();
    if constexpr (NORM) {
      // X from the LDS tile: 16 lanes per 256-byte row, so each store
      // instruction writes whole lines
      const int u = threadIdx.x & 15;
#pragma unroll
      for (int pass = 0; pass < 4; ++pass) {
        const int r = pass * 16 + (threadIdx.x >> 4);
        if (r0 + r < rows && c0 + 4 * u < cols)
          reinterpret_cast<float4*>(nrm.X + (r0 + r) * cols + c0)[u] =
              make_float4(__uint_as_float(tile[r][4 * u]), __uint_as_float(tile[r][4 * u + 1]),
                          __uint_as_float(tile[r][4 * u + 2]), __uint_as_float(tile[r][4 * u + 3]));
      }
    }
    const int j = threadIdx.x >> 2, b = threadIdx.x & 3;
    if (c0 + j < cols && r0 + 16 * b < rows && !(sym && r0 == c0)) {
      uint32_t w[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) w[i] = tile[16 * b + i][j];
      if (rht.on) rht16(w, rht.mask);
      uint32_t lo, hi, sc;
      if (rht.adaptive46) encode_block16_46(w, sgc, lo, hi, sc);
      else encode_block16(w, sgc, lo, hi, sc);
      const int64_t e = (c0 + j) * rows + r0 + 16 * b;   // element of the transpose
      reinterpret_cast<uint2*>(col_codes)[e / 16] = make_uint2(lo, hi);
      col_scales[e / 16] = (uint8_t)sc;
    }
  }
}

// Tensor maxima of the transformed row blocks (x H^r, into slot_r) and/or
// column blocks (H^r^T x, into slot_c), same tiling as quant_tile_kernel.
// With `sym` the input is a symmetric square matrix of which only the tiles
// on or above the diagonal are read, as in quant_tile_kernel: the column
// blocks of tile (I, J) are the row blocks of tile (J, I), so both go to
// slot_r (slot_c == slot_r), and a diagonal tile counts its rows only.
template <Dt T>
__global__ __launch_bounds__(kThreads) void amax_tiles_kernel(
    const void* x, int64_t rows, int64_t cols, uint32_t tiles_x, uint32_t* slot_r,
    uint32_t* slot_c, RhtArg rht, uint32_t sym) {
  __shared__ uint32_t tile[64][65];
  const int64_t r0 = tile_row0(tiles_x), c0 = tile_col0(tiles_x);
  if (sym && r0 > c0) return;   // below the diagonal: done by tile (J, I)
  if (sym && r0 == c0) slot_c = nullptr;
  const int tr = threadIdx.x >> 2, tc = (threadIdx.x & 3) * 16;
  const bool in = (r0 + tr < rows) && (c0 + tc < cols);
  uint32_t v[16];
  if (in) {
    load16<T>(x, (r0 + tr) * cols + c0 + tc, v);
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = 0u;
  }
  if (slot_c) {
#pragma unroll
    for (int i = 0; i < 16; ++i) tile[tr][tc + i] = v[i];
  }
  if (slot_r) {
    if (rht.on) rht16(v, rht.mask);
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t a = abs_bits(v[i]);
      m = a > m ? a : m;
    }
    amax_publish_block(m, slot_r);
  }
  if (slot_c) {
    __syncthreads();
    const int j = threadIdx.x >> 2, b = threadIdx.x & 3;
    uint32_t m = 0;
    if (c0 + j < cols && r0 + 16 * b < rows) {
      uint32_t w[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) w[i] = tile[16 * b + i][j];
      if (rht.on) rht16(w, rht.mask);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t a = abs_bits(w[i]);
        m = a > m ? a : m;
      }
    }
    amax_publish_block(m, slot_c);
  }
}

// ------------------------------------------------------------ dequant ----

// Round the exact products u * sg (u = q*s has <= 6 significant bits) once
// to bf16, two at a time.  hi = RN_f32(u*sg) then RN_bf16(hi) equals the
// single rounding unless hi landed exactly on a bf16 midpoint (low half
// 0x8000) or is tiny (the f32 product may have lost bits to underflow);
// those rare lanes take the exact double path.  Zero products take it too
// (their exponent field is below the bound), which is exact and, measured,
// no loss: the decode pass is bound by its store stream, and on 2^28 values
// both a check that lets zeros through and one branch per eight values
// instead of per value made it slower (122-125 us against 107; with 1024
// workgroups instead of 8192, 110 us).
__device__ __forceinline__ uint16_t product_to_bf16_exact(float u, float sg) {
  const double d = (double)u * (double)sg;   // exact
  const double a = fabs(d);
  if (!(a == a)) return 0x7FC0u;
  if (a == 0.0) return (uint16_t)((__float_as_uint(u * sg)) >> 16);
  if (a >= 0x1p128) return (uint16_t)(d < 0 ? 0xFF80u : 0x7F80u);
  int E = (int)((__double_as_longlong(a) >> 52) & 0x7FF) - 1023;
  E = E < -126 ? -126 : E;
  const double r = ldexp(rint(ldexp(a, 7 - E)), E - 7);   // RNE at the bf16 ulp
  if (r >= 0x1p128) return (uint16_t)(d < 0 ? 0xFF80u : 0x7F80u);
  const uint32_t fb = __float_as_uint((float)r);           // r is a bf16 number
  return (uint16_t)((fb >> 16) | (d < 0 ? 0x8000u : 0u));
}

__device__ __forceinline__ uint32_t products_to_bf16x2(float u0, float u1, float sg) {
  const float h0 = u0 * sg, h1 = u1 * sg;
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t r = {(__bf16)h0, (__bf16)h1};             // hardware RNE
  uint32_t out = __builtin_bit_cast(uint32_t, r);
  const uint32_t b0 = __float_as_uint(h0), b1 = __float_as_uint(h1);
  const bool bad0 = (b0 & 0xFFFFu) == 0x8000u || (b0 & 0x7F800000u) < 0x0D800000u;
  const bool bad1 = (b1 & 0xFFFFu) == 0x8000u || (b1 & 0x7F800000u) < 0x0D800000u;
  if (bad0) out = (out & 0xFFFF0000u) | product_to_bf16_exact(u0, sg);
  if (bad1) out = (out & 0x0000FFFFu) | ((uint32_t)product_to_bf16_exact(u1, sg) << 16);
  return out;
}

// Values of the 16 codes of one block (exact f32 q*s; the tensor scale is
// applied by the caller).  The conversion instruction with scale 1 yields
// the exact E2M1 value of the two nibbles of the selected byte.
__device__ __forceinline__ void decode_word(uint32_t w, float s, float* u) {
  float2_t q0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  float2_t q1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  float2_t q2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  float2_t q3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  u[0] = q0[0] * s; u[1] = q0[1] * s; u[2] = q1[0] * s; u[3] = q1[1] * s;
  u[4] = q2[0] * s; u[5] = q2[1] * s; u[6] = q3[0] * s; u[7] = q3[1] * s;
}

__device__ __forceinline__ void decode_block(uint2 c, uint32_t scale_byte, float (&u)[16]) {
  const float s = __builtin_amdgcn_cvt_f32_fp8((int)scale_byte, 0);
  decode_word(c.x, s, u);
  decode_word(c.y, s, u + 8);
}

template <Dt O>
__device__ __forceinline__ void store16(void* out, int64_t idx, const float (&u)[16], float sg) {
  if constexpr (O == Dt::F32) {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(out) + idx);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      p[j] = make_float4(u[4 * j] * sg, u[4 * j + 1] * sg, u[4 * j + 2] * sg, u[4 * j + 3] * sg);
  } else {
    uint4* p = reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + idx);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint32_t w[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) w[t] = products_to_bf16x2(u[8 * j + 2 * t], u[8 * j + 2 * t + 1], sg);
      p[j] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// Each lane writes 16 bytes (8 BF16 or 4 FP32 values) of one block, so every
// store instruction of a wave covers one contiguous kilobyte.
template <Dt O>
__global__ __launch_bounds__(kThreads) void dequant_rows_kernel(
    const uint8_t* codes, const uint8_t* scales, const float* sgp, int64_t nelem, void* out) {
  constexpr int EPL = O == Dt::F32 ? 4 : 8;
  constexpr int G = 16 / EPL;
  const float sg = *sgp;
  const int64_t items = nelem / EPL;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  using Word = typename std::conditional<O == Dt::F32, uint16_t, uint32_t>::type;
  auto emit = [&](int64_t item, uint32_t w, uint32_t sbyte) {
    const float s = __builtin_amdgcn_cvt_f32_fp8((int)sbyte, 0);
    if constexpr (O == Dt::BF16) {
      float u[8];
      decode_word(w, s, u);
      uint4 r;
      r.x = products_to_bf16x2(u[0], u[1], sg);
      r.y = products_to_bf16x2(u[2], u[3], sg);
      r.z = products_to_bf16x2(u[4], u[5], sg);
      r.w = products_to_bf16x2(u[6], u[7], sg);
      store_nt(reinterpret_cast<uint4*>(out) + item, r);
    } else {
      const float2_t q0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
      const float2_t q1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
      reinterpret_cast<float4*>(out)[item] =
          make_float4(q0[0] * s * sg, q0[1] * s * sg, q1[0] * s * sg, q1[1] * s * sg);
    }
  };
  // kUnroll items per lane per trip, loads first (see quant_rows_kernel)
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + (kUnroll - 1) * stride < items; i += kUnroll * stride) {
    uint32_t w[kUnroll], sb[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      w[u] = reinterpret_cast<const Word*>(codes)[i + u * stride];
      sb[u] = scales[(i + u * stride) / G];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) emit(i + u * stride, w[u], sb[u]);
  }
  for (; i < items; i += stride) emit(i, reinterpret_cast<const Word*>(codes)[i], scales[i / G]);
}

// Q_16x1 tensor stored as the rows of its transpose: codes [cols][rows/2].
// Workgroup tile: 64 original rows x 64 original columns.
template <Dt O>
__global__ __launch_bounds__(kThreads) void dequant_cols_kernel(
    const uint8_t* codes, const uint8_t* scales, const float* sgp, int64_t rows, int64_t cols,
    uint32_t tiles_x, void* out) {
  __shared__ float tile[64][65];
  const float sg = *sgp;
  const int64_t r0 = tile_row0(tiles_x), c0 = tile_col0(tiles_x);
  {
    const int j = threadIdx.x >> 2, b = threadIdx.x & 3;   // column j, row block b
    float u[16];
    if (c0 + j < cols && r0 + 16 * b < rows) {
      const int64_t e = (c0 + j) * rows + r0 + 16 * b;
      decode_block(reinterpret_cast<const uint2*>(codes)[e / 16], scales[e / 16], u);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) u[i] = 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) tile[16 * b + i][j] = u[i];
  }
  __syncthreads();
  const int tr = threadIdx.x >> 2, tc = (threadIdx.x & 3) * 16;
  if (r0 + tr < rows && c0 + tc < cols) {
    float u[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) u[i] = tile[tr][tc + i];
    store16<O>(out, (r0 + tr) * cols + c0 + tc, u, sg);
  }
}

// `work` is counted in 16-byte vectors.
inline int grid_for(int64_t work, int per_block) {
  int64_t g = (work + per_block - 1) / per_block;
  if (g < 1) g = 1;
  const int64_t cap = work >= kLargeVectors ? kMaxGridLarge : kMaxGrid;
  return (int)(g > cap ? cap : g);
}

}  // namespace

hipError_t launch_amax(const void* x, Dt xt, int64_t n, uint32_t* slot, hipStream_t s) {
  const int64_t nvec = xt == Dt::F32 ? n / 4 : n / 8;
  const int64_t rounds = (nvec + kThreads - 1) / kThreads;
  const int grid = (int)(rounds < NVFP4_AMAX_GRID ? rounds : NVFP4_AMAX_GRID);
  if (xt == Dt::F32)
    amax_kernel<Dt::F32><<<grid, kThreads, 0, s>>>(x, nvec, slot);
  else
    amax_kernel<Dt::BF16><<<grid, kThreads, 0, s>>>(x, nvec, slot);
  return hipGetLastError();
}

hipError_t launch_quant_rows(const void* x, Dt xt, int64_t rows, int64_t cols,
                             const uint32_t* amax_slot, float* sg_out, uint8_t* codes,
                             uint8_t* scales, uint32_t* zero_slot, hipStream_t s) {
  const int64_t nelem = rows * cols;
  if (xt == Dt::F32)
    quant_rows_kernel<Dt::F32><<<grid_for(nelem / 4, kThreads * 4), kThreads, 0, s>>>(
        x, nelem, amax_slot, sg_out, codes, scales, zero_slot);
  else
    quant_rows_kernel<Dt::BF16><<<grid_for(nelem / 8, kThreads * 4), kThreads, 0, s>>>(
        x, nelem, amax_slot, sg_out, codes, scales, zero_slot);
  return hipGetLastError();
}

hipError_t launch_quant_tiles(const void* x, Dt xt, int64_t rows, int64_t cols,
                              const uint32_t* amax_slot, float* sg_out, uint8_t* row_codes,
                              uint8_t* row_scales, uint8_t* col_codes, uint8_t* col_scales,
                              uint32_t* zero_slot, hipStream_t s, const uint32_t* amax_c,
                              float* sg_out_c, RhtArg rht, int batch, int64_t bstride) {
  uint32_t tiles_x, grid;
  if (!tile_grid(rows, cols, tiles_x, grid)) return hipErrorInvalidValue;
  if (batch < 1 || (batch > 1 && bstride <= 0)) return hipErrorInvalidValue;
  const bool R = row_codes != nullptr, C = col_codes != nullptr;
  const dim3 g2(grid, (unsigned)batch);
  const int64_t bs = batch > 1 ? bstride : 0;
#define NVFP4_QT(T, RR, CC)                                                                   \
  quant_tile_kernel<T, RR, CC><<<g2, kThreads, 0, s>>>(x, rows, cols, tiles_x, amax_slot,     \
                                                       sg_out, row_codes, row_scales,         \
                                                       col_codes, col_scales, zero_slot,      \
                                                       amax_c, sg_out_c, rht, NormArg{}, 0u, bs)
  if (xt == Dt::F32) {
    if (R && C) NVFP4_QT(Dt::F32, true, true);
    else if (R) NVFP4_QT(Dt::F32, true, false);
    else NVFP4_QT(Dt::F32, false, true);
  } else {
    if (R && C) NVFP4_QT(Dt::BF16, true, true);
    else if (R) NVFP4_QT(Dt::BF16, true, false);
    else NVFP4_QT(Dt::BF16, false, true);
  }
#undef NVFP4_QT
  return hipGetLastError();
}

hipError_t launch_quant_sym_tiles(const float* x, int64_t m, const uint32_t* amax_slot,
                                  float* sg_out, uint8_t* codes, uint8_t* scales,
                                  uint32_t* zero_slot, bool adaptive46, hipStream_t s, int batch,
                                  int64_t bstride, uint32_t rht_on, uint32_t rht_mask) {
  uint32_t tiles_x, grid;
  if (!tile_grid(m, m, tiles_x, grid)) return hipErrorInvalidValue;
  if (batch < 1 || (batch > 1 && bstride <= 0)) return hipErrorInvalidValue;
  quant_tile_kernel<Dt::F32, true, true><<<dim3(grid, (unsigned)batch), kThreads, 0, s>>>(
      x, m, m, tiles_x, amax_slot, sg_out, codes, scales, codes, scales, zero_slot, nullptr,
      nullptr, RhtArg{rht_on, rht_mask, adaptive46 ? 1u : 0u}, NormArg{}, 1u,
      batch > 1 ? bstride : 0);
  return hipGetLastError();
}

hipError_t launch_normalize_quant_tiles(const void* G, Dt gt, int64_t rows, int64_t cols, float clip,
                                        const float* clip_dev, const double* inv, float* X,
                                        const uint32_t* amax_slot, float* sg_out,
                                        uint8_t* row_codes, uint8_t* row_scales,
                                        uint8_t* col_codes, uint8_t* col_scales,
                                        uint32_t* zero_slot, bool adaptive46, hipStream_t s) {
  uint32_t tiles_x, grid;
  if (!tile_grid(rows, cols, tiles_x, grid)) return hipErrorInvalidValue;
  const RhtArg o{0u, 0u, adaptive46 ? 1u : 0u};
  const NormArg nrm{clip, clip_dev, inv, X};
  if (gt == Dt::F32)
    quant_tile_kernel<Dt::F32, true, true, true><<<grid, kThreads, 0, s>>>(
        G, rows, cols, tiles_x, amax_slot, sg_out, row_codes, row_scales, col_codes, col_scales,
        zero_slot, nullptr, nullptr, o, nrm, 0u, 0);
  else
    quant_tile_kernel<Dt::BF16, true, true, true><<<grid, kThreads, 0, s>>>(
        G, rows, cols, tiles_x, amax_slot, sg_out, row_codes, row_scales, col_codes, col_scales,
        zero_slot, nullptr, nullptr, o, nrm, 0u, 0);
  return hipGetLastError();
}

hipError_t launch_amax_tiles(const void* x, Dt xt, int64_t rows, int64_t cols, uint32_t* slot_r,
                             uint32_t* slot_c, RhtArg rht, hipStream_t s) {
  uint32_t tiles_x, grid;
  if (!tile_grid(rows, cols, tiles_x, grid)) return hipErrorInvalidValue;
  if (xt == Dt::F32)
    amax_tiles_kernel<Dt::F32><<<grid, kThreads, 0, s>>>(x, rows, cols, tiles_x, slot_r, slot_c, rht, 0u);
  else
    amax_tiles_kernel<Dt::BF16><<<grid, kThreads, 0, s>>>(x, rows, cols, tiles_x, slot_r, slot_c, rht, 0u);
  return hipGetLastError();
}

hipError_t launch_amax_sym_tiles(const float* x, int64_t m, uint32_t* slot, RhtArg rht,
                                 hipStream_t s) {
  uint32_t tiles_x, grid;
  if (!tile_grid(m, m, tiles_x, grid)) return hipErrorInvalidValue;
  amax_tiles_kernel<Dt::F32><<<grid, kThreads, 0, s>>>(x, m, m, tiles_x, slot, slot, rht, 1u);
  return hipGetLastError();
}

hipError_t launch_dequant_rows(const uint8_t* codes, const uint8_t* scales, const float* sg,
                               int64_t rows, int64_t cols, void* out, Dt ot, hipStream_t s) {
  const int64_t nelem = rows * cols;
  if (ot == Dt::F32)
    dequant_rows_kernel<Dt::F32><<<grid_for(nelem / 4, kThreads * 4), kThreads, 0, s>>>(
        codes, scales, sg, nelem, out);
  else
    dequant_rows_kernel<Dt::BF16><<<grid_for(nelem / 8, kThreads * 4), kThreads, 0, s>>>(
        codes, scales, sg, nelem, out);
  return hipGetLastError();
}

hipError_t launch_dequant_cols(const uint8_t* codes, const uint8_t* scales, const float* sg,
                               int64_t rows, int64_t cols, void* out, Dt ot, hipStream_t s) {
  uint32_t tiles_x, grid;
  if (!tile_grid(rows, cols, tiles_x, grid)) return hipErrorInvalidValue;
  if (ot == Dt::F32)
    dequant_cols_kernel<Dt::F32><<<grid, kThreads, 0, s>>>(codes, scales, sg, rows, cols, tiles_x, out);
  else
    dequant_cols_kernel<Dt::BF16><<<grid, kThreads, 0, s>>>(codes, scales, sg, rows, cols, tiles_x, out);
  return hipGetLastError();
}

}  // namespace nvfp4
