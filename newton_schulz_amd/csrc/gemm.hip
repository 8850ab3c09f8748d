// NVFP4 x NVFP4 -> FP32 GEMM with fused Newton–Schulz epilogues, gfx950.
//
// The three products of the NVFP4 NS iteration (Full-Stack FP4, arXiv
// 2607.04422, §3.4): A = qX qX^T, B = b A + c qA qA^T, X' = a X + qB qX16.
// Every one is C = P Q^T with both operands stored as packed E2M1 codes plus
// E4M3 scales blocked by 16 along the contraction axis K.
//
// Data path: packed codes and scale bytes (0.5625 B per element) are staged
// in LDS; each lane then turns one 32-bit word of 8 codes and its block
// scale into 8 f16 values (exact: q*s has <= 6 significant bits inside the
// normal f16 range) and feeds v_mfma_f32_32x32x16_f16, FP32 accumulation.
// The tensor scales s_g of both operands multiply the accumulator once in
// the epilogue.
//
// K order inside an MFMA: a product sums over K, so any permutation of K
// applied to both operands leaves it unchanged.  Lane l (row l%32, half
// h = l/32) takes bytes [32h, 32h+32) of each row's 64-byte K chunk and
// MFMA step s uses its 4-byte word s: both operands use the same map.
#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128;      // workgroup tile
constexpr int BK = 128;                // K elements per LDS stage
constexpr int kThreads = 256;          // 4 waves in a 2 x 2 grid of 64 x 64
constexpr int kCodeRow = BK / 2;       // 64 bytes of codes per row per stage
constexpr int kCodeStride = kCodeRow + 16;   // padded LDS row (bank spread)
constexpr int kScaleStride = 12;       // 8 scale bytes per row, padded
constexpr int kCodeTile = BM * kCodeStride;
constexpr int kScaleTile = BM * kScaleStride;
constexpr int kStage = 2 * kCodeTile + 2 * kScaleTile;

struct TileLoad {
  uint2 pc[4], qc[4];   // 8-byte code chunks
  uint32_t ps, qs;      // 4 scale bytes
};

__device__ __forceinline__ void load_tile(const GemmProblem& g, int64_t m0, int64_t n0, int64_t k0,
                                          TileLoad& t) {
  const int tid = threadIdx.x;
  const int64_t kb = g.K / 2;     // code bytes per row
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = tid + kThreads * i;
    const int row = idx >> 3, chunk = idx & 7;
    const int64_t kk = k0 + chunk * 16;
    const bool kin = kk < g.K;
    t.pc[i] = (kin && m0 + row < g.M)
                  ? *reinterpret_cast<const uint2*>(g.codes_p + (m0 + row) * kb + kk / 2)
                  : make_uint2(0u, 0u);
    t.qc[i] = (kin && n0 + row < g.N)
                  ? *reinterpret_cast<const uint2*>(g.codes_q + (n0 + row) * kb + kk / 2)
                  : make_uint2(0u, 0u);
  }
  {
    const int row = tid >> 1, part = tid & 1;
    const int64_t sb = g.K / 16;  // scale bytes per row
    const int64_t blk = k0 / 16 + part * 4;
    uint32_t ps = 0, qs = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (blk + j < sb) {
        if (m0 + row < g.M) ps |= (uint32_t)g.scales_p[(m0 + row) * sb + blk + j] << (8 * j);
        if (n0 + row < g.N) qs |= (uint32_t)g.scales_q[(n0 + row) * sb + blk + j] << (8 * j);
      }
    }
    t.ps = ps;
    t.qs = qs;
  }
}

__device__ __forceinline__ void store_tile(uint8_t* stage, const TileLoad& t) {
  const int tid = threadIdx.x;
  uint8_t* sp = stage;
  uint8_t* sq = stage + kCodeTile;
  uint8_t* sps = stage + 2 * kCodeTile;
  uint8_t* sqs = sps + kScaleTile;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = tid + kThreads * i;
    const int row = idx >> 3, chunk = idx & 7;
    *reinterpret_cast<uint2*>(sp + row * kCodeStride + chunk * 8) = t.pc[i];
    *reinterpret_cast<uint2*>(sq + row * kCodeStride + chunk * 8) = t.qc[i];
  }
  const int row = tid >> 1, part = tid & 1;
  *reinterpret_cast<uint32_t*>(sps + row * kScaleStride + part * 4) = t.ps;
  *reinterpret_cast<uint32_t*>(sqs + row * kScaleStride + part * 4) = t.qs;
}

// Fragment of one 32-row subtile for a whole stage: 8 code words (one per
// MFMA step) and the 4 block scales they use.
struct Frag {
  uint32_t w[8];
  half2_t s[4];
};

__device__ __forceinline__ void read_frag(const uint8_t* codes, const uint8_t* scales, int row,
                                          int h, Frag& f) {
  const uint4 a = *reinterpret_cast<const uint4*>(codes + row * kCodeStride + 32 * h);
  const uint4 b = *reinterpret_cast<const uint4*>(codes + row * kCodeStride + 32 * h + 16);
  f.w[0] = a.x; f.w[1] = a.y; f.w[2] = a.z; f.w[3] = a.w;
  f.w[4] = b.x; f.w[5] = b.y; f.w[6] = b.z; f.w[7] = b.w;
  const uint32_t sc = *reinterpret_cast<const uint32_t*>(scales + row * kScaleStride + 4 * h);
#pragma unroll
  for (int j = 0; j < 4; ++j) f.s[j] = scale_pair_f16((sc >> (8 * j)) & 0xFFu);
}

__device__ __forceinline__ void wave_amax_atomic(uint32_t m, uint32_t* slot) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint32_t w = __shfl_xor(m, o, 64);
    m = w > m ? w : m;
  }
  if ((threadIdx.x & 63) == 0) atomicMax(slot, m);
}

template <bool SYM>
__global__ __launch_bounds__(kThreads, 2) void gemm_kernel(GemmProblem g) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStage];

  // ---- tile of this workgroup
  int64_t ti, tj;
  if constexpr (SYM) {
    const int64_t nt = (g.M + BM - 1) / BM;
    int64_t rem = blockIdx.x, r = 0;
    while (rem >= nt - r) { rem -= nt - r; ++r; }
    ti = r;
    tj = r + rem;
  } else {
    ti = blockIdx.y;
    tj = blockIdx.x;
  }
  const int64_t m0 = ti * BM, n0 = tj * BN;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, r32 = lane & 31;

  floatx16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int64_t nk = (g.K + BK - 1) / BK;
  TileLoad tl;
  load_tile(g, m0, n0, 0, tl);
  store_tile(smem, tl);
  __syncthreads();

  for (int64_t kc = 0; kc < nk; ++kc) {
    const bool more = kc + 1 < nk;
    if (more) load_tile(g, m0, n0, (kc + 1) * BK, tl);

    const uint8_t* stage = smem + (kc & 1) * kStage;
    Frag fp[2], fq[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      read_frag(stage, stage + 2 * kCodeTile, wm * 64 + 32 * i + r32, h, fp[i]);
      read_frag(stage + kCodeTile, stage + 2 * kCodeTile + kScaleTile, wn * 64 + 32 * i + r32, h, fq[i]);
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      half8_t a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        a[i] = dequant8_f16(fp[i].w[s], fp[i].s[s >> 1]);
        b[i] = dequant8_f16(fq[i].w[s], fq[i].s[s >> 1]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
    }

    if (more) store_tile(smem + ((kc + 1) & 1) * kStage, tl);
    __syncthreads();
  }

  // ---- epilogue: out = beta * addend + alpha * sgP * sgQ * acc
  const float scale = g.alpha * (*g.sg_p) * (*g.sg_q);
  const float beta = g.beta;
  const bool off_diag = ti < tj;
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * 64 + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
        const int64_t col = n0 + wn * 64 + 32 * j + r32;
        if (row >= g.M || col >= g.N) continue;
        if (SYM && !off_diag && row > col) continue;
        float v = scale * acc[i][j][r];
        if (g.addend) v = fmaf(beta, g.addend[row * g.N + col], v);
        g.out[row * g.N + col] = v;
        if (SYM && (off_diag || row < col)) g.out[col * g.N + row] = v;
        const uint32_t a = abs_bits(v);
        amax = a > amax ? a : amax;
      }
  if (g.amax_out) wave_amax_atomic(amax, g.amax_out);
}

}  // namespace

hipError_t launch_gemm(const GemmProblem& p, hipStream_t s) {
  if (p.symmetric) {
    const int64_t nt = (p.M + BM - 1) / BM;
    gemm_kernel<true><<<dim3((unsigned)(nt * (nt + 1) / 2)), kThreads, 0, s>>>(p);
  } else {
    dim3 grid((unsigned)((p.N + BN - 1) / BN), (unsigned)((p.M + BM - 1) / BM));
    gemm_kernel<false><<<grid, kThreads, 0, s>>>(p);
  }
  return hipGetLastError();
}

}  // namespace nvfp4
