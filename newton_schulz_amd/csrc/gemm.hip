// NVFP4 x NVFP4 -> FP32 GEMM with fused Newton–Schulz epilogues, gfx950.
//
// The three products of the NVFP4 NS iteration (Full-Stack FP4, arXiv
// 2607.04422, §3.4): A = qX qX^T, B = b A + c qA qA^T, X' = a X + qB qX16.
// Every one is C = P Q^T with both operands stored as packed E2M1 codes plus
// E4M3 scales blocked by 16 along the contraction axis K.
//
// Data path: packed codes and scale bytes (0.5625 B per element) go from
// global memory straight into LDS (global_load_lds, no staging registers);
// each lane then turns one 32-bit word of 8 codes and its block scale into
// 8 f16 values (exact: q*s has <= 6 significant bits inside the normal f16
// range) and feeds v_mfma_f32_32x32x16_f16 with FP32 accumulation.  The
// tensor scales s_g of both operands multiply the accumulator once in the
// epilogue.
//
// K order inside an MFMA: a product sums over K, so any permutation of K
// applied to both operands leaves it unchanged; both operands use the same
// map.  Stages are 256 wide when K % 256 == 0, else 128 wide.
//
// 256-wide stages (row lines): a 32-row group's stage is 32 rows x 128 code
// bytes, loaded eight whole rows (eight 128-byte lines) per DMA instruction
// and kept in LDS row by row with a chunk swizzle (row_swizzle below); lane l
// (row l%32, half h = l/32) consumes 16-byte chunks 4h .. 4h+3 of its row,
// one per quarter-stage, one word per MFMA step.
//
// 128-wide stages: lane l owns bytes [32h, 32h+32) of the row's 64 code
// bytes; MFMA step s of half-stage hs uses its word s of bytes
// [32h + 16hs, +16).  LDS is fragment-major: for each 32-row group and
// half-stage a 1 KB region holds lane l's 16 bytes at 16*l, exactly what
// both the DMA load of lane l writes and the fragment read of lane l reads.
// A DMA instruction then gathers 32 bytes from each of 32 rows, which moves
// data about four times slower than reading whole lines.
//
// Symmetric products compute only tiles that touch the upper triangle
// (row <= col); each element there is written once and mirrored.  Tiles
// left over after one per CU are split along K into parts whose FP32
// partials are summed in part order (deterministic): by the part that
// finishes last, inside the product kernel, when the whole tiles are long
// enough to hide that work, else by a second kernel; see FastArgs.
#include <cstddef>

#include "launch.hpp"
#include "nvfp4_device.hpp"


namespace nvfp4 {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kXcds = 8;   // MI355X: workgroups go round-robin to 8 XCDs
#ifndef NVFP4_CUS_PER_XCD
#define NVFP4_CUS_PER_XCD 32     // MI355X: 256 CUs in 8 XCDs
#endif
constexpr int kCus = NVFP4_CUS_PER_XCD;

// ===========================================================================
// Fast path: K % 128 == 0, DMA loads into fragment-major LDS.
// ===========================================================================

template <int WM_, int WN_, int FM_, int FN_, int NST_, int BK_>
struct Cfg {
  static constexpr int WM = WM_, WN = WN_, FM = FM_, FN = FN_;
  static constexpr int NST = NST_;                    // LDS stages in flight
  static constexpr int BK = BK_;                      // K elements per stage (128 or 256)
  static constexpr int kHalves = BK / 64;             // 16-byte lane slices per row per stage
  static_assert(BK == 128 || BK == 256, "BK must be 128 or 256");
  // BK = 256 loads whole 128-byte row lines (see row_swizzle); the narrower
  // stages load 32 rows x 16 bytes per instruction
  static constexpr bool kLines = BK == 256;
  static constexpr int kWaves = WM * WN;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int BM = WM * FM * 32, BN = WN * FN * 32;
  static constexpr int GP = BM / 32, GQ = BN / 32;   // 32-row groups per operand
  static constexpr int kGroups = GP + GQ;
  static constexpr int kRegions = kGroups * kHalves;  // 1 KB code regions per stage
  static constexpr int kCodeBytes = kRegions * 1024;
  static constexpr int kScaleGroupBytes = kLines ? 512 : 256;   // per 32-row group and stage
  static constexpr int kScaleBytes = kGroups * kScaleGroupBytes;
  static constexpr int kStage = kCodeBytes + kScaleBytes;
  static constexpr int kAcc = FM * FN * 16;           // accumulators per lane
  // two resident workgroups per CU unless the accumulators alone need more
  // than half the register file
#ifndef NVFP4_MIN_BLOCKS
  static constexpr int kMinBlocks = (kWaves <= 4 && kAcc <= 128) ? 2 : 1;
#else
  static constexpr int kMinBlocks = NVFP4_MIN_BLOCKS;
#endif
  // DMA instructions each wave issues per stage.  Regions are dealt out
  // round-robin; when they do not divide evenly, a wave with one fewer
  // repeats its previous load (same bytes to the same LDS address) so that
  // every wave waits on the same count.
  // Scale loads: one per group (4 bytes a lane), or with row lines one per
  // pair of groups (16 bytes a lane, 64 rows).
  static constexpr int kScaleRegions = kLines ? kGroups / 2 : kGroups;
  static_assert(!kLines || GP % 2 == 0, "row-line scale loads pair groups of one operand");
  static_assert(kRegions >= kWaves && kScaleRegions >= kWaves, "fewer regions than waves");
  static constexpr int kCodeLoads = (kRegions + kWaves - 1) / kWaves;
  static constexpr int kScaleLoads = (kScaleRegions + kWaves - 1) / kWaves;
  static constexpr int kLoadsPerWave = kCodeLoads + kScaleLoads;
};

// Schedule of one product (see plan_with): the tiles are cut into kXcds
// contiguous runs, one per XCD (tiles sharing operand panels share an L2).
// Within a run of n tiles, the first floor(n / cus) * cus are whole work
// units -- the same number for every CU -- and each of the remaining
// n mod cus tiles is split along K into `parts` units whose FP32 partials
// are summed in a fixed order (by the last part to finish or by a second
// kernel, see FastArgs), so the leftover work spreads over the CUs instead
// of doubling some of them.
#ifndef NVFP4_MAX_PARTS
#define NVFP4_MAX_PARTS 8
#endif
constexpr int kMaxParts = NVFP4_MAX_PARTS;   // K-parts of a split tile at most

struct FastArgs {
  GemmProblem g;
  int64_t TM, TN;       // tile grid
  int64_t tiles;
  float rcp_tm;         // 1 / TM, for the column-major tile order
  int parts;            // K-parts of a leftover tile (1: leftovers run whole)
  float* partials;
  uint32_t* counters;   // per split tile, K-parts finished; null: a second kernel sums
  int64_t bstride;      // bytes between the problems of a batched launch (grid y)
};

// Outputs of the problems of a batched launch, when given one by one (n > 0).
// The first argument of the product kernels, so that it sits at the start
// of the kernel-argument segment (explicit arguments are laid out in order
// at their natural alignment): entry y is then one scalar load from there,
// instead of all of them copied to registers or scratch.
struct OutTable {
  int n;
  float* outs[kMaxBatchOut];
};
static_assert(offsetof(OutTable, outs) == 8, "OutTable layout");

__device__ __forceinline__ float* table_out(int y) {
  typedef float* __attribute__((address_space(4))) const* KPtr;
  typedef const __attribute__((address_space(4))) uint8_t* KBytes;
  const KBytes k = (KBytes)__builtin_amdgcn_kernarg_segment_ptr();
  return ((KPtr)(k + offsetof(OutTable, outs)))[y];
}

template <class T>
__device__ __forceinline__ T* shift_bytes(T* p, int64_t off) {
  return p ? reinterpret_cast<T*>(reinterpret_cast<uintptr_t>(p) + off) : p;
}

// Problem blockIdx.y of a batched launch: every pointer moves by its
// offset (wave-uniform, so the operand bases stay in scalar registers).
// Workgroup (x, y) has linear id y * units + x, and units is a multiple of
// kXcds, so it runs on the XCD its unit has in a single launch.
template <bool RHTMAX>
__device__ __forceinline__ void select_problem(FastArgs& a, int nout) {
  const int64_t off = (int64_t)blockIdx.y * a.bstride;
  GemmProblem& g = a.g;
  g.codes_p = shift_bytes(g.codes_p, off);
  g.scales_p = shift_bytes(g.scales_p, off);
  g.sg_p = shift_bytes(g.sg_p, off);
  g.codes_q = shift_bytes(g.codes_q, off);
  g.scales_q = shift_bytes(g.scales_q, off);
  g.sg_q = shift_bytes(g.sg_q, off);
  g.addend = shift_bytes(g.addend, off);
  if (nout) {
    g.out = table_out((int)blockIdx.y);
  } else {
    g.out = shift_bytes(g.out, off);
  }
  g.amax_out = shift_bytes(g.amax_out, off);
  if constexpr (RHTMAX) {
    g.amax_out_c = shift_bytes(g.amax_out_c, off);
    g.clear_a = shift_bytes(g.clear_a, off);
    g.clear_b = shift_bytes(g.clear_b, off);
  }
  a.partials = shift_bytes(a.partials, off);
  a.counters = shift_bytes(a.counters, off);
}

// The last K-part of a split tile sums the parts inside the product kernel
// when a whole tile runs at least this many K-stages; the summing then
// overlaps the whole tiles' K-loops.  With fewer stages the summing CU
// slows the whole tile beside it by about what the second kernel costs
// (measured, against the reduce kernel: 3072^2 x 8192 (32 stages) gains
// 11 us, 3072^2 x 3072 (12 stages) 3 us).
#ifndef NVFP4_FIXUP_MIN_STAGES
#define NVFP4_FIXUP_MIN_STAGES 12
#endif

template <bool B>
struct BoolTag {
  static constexpr bool value = B;
};

struct Unit {
  int tile;             // tile index
  int part;             // K-part of a split tile (0 for a whole tile)
  int split;            // index among all split tiles, or -1 for a whole tile
};

// Scheduling arithmetic is 32-bit (tile counts stay far below 2^31) and
// wave-uniform, so it stays in scalar registers.
__device__ __forceinline__ void xcd_run(const FastArgs& a, int x, int& t0, int& n, int& whole) {
  const int tiles = (int)a.tiles;
  t0 = x * tiles / kXcds;
  n = (x + 1) * tiles / kXcds - t0;
  whole = a.parts > 1 ? n / kCus * kCus : n;
}

// Work unit of workgroup b (b % kXcds picks the XCD); false when none.
__device__ __forceinline__ bool unit_of(const FastArgs& a, int b, Unit& u) {
  const int x = b % kXcds, l = b / kXcds;
  int t0, n, whole;
  xcd_run(a, x, t0, n, whole);
  if (l < whole) {
    u.tile = t0 + l;
    u.part = 0;
    u.split = -1;
    return true;
  }
  const int r = l - whole;
  if (r >= (n - whole) * a.parts) return false;
  int base = 0;                           // split tiles of the XCDs before x
  for (int y = 0; y < x; ++y) {
    int ty, ny, wy;
    xcd_run(a, y, ty, ny, wy);
    base += ny - wy;
  }
  u.tile = t0 + whole + r / a.parts;
  u.part = r % a.parts;
  u.split = base + r / a.parts;
  return true;
}

// Tile of split tile number s (inverse of unit_of's numbering).
__device__ __forceinline__ int split_tile(const FastArgs& a, int s) {
  for (int x = 0; x < kXcds; ++x) {
    int t0, n, whole;
    xcd_run(a, x, t0, n, whole);
    if (s < n - whole) return t0 + whole + s;
    s -= n - whole;
  }
  return -1;
}

// Tile t of the grid: row-block I, col-block J.  Symmetric problems list only
// tiles whose first row is <= their last column, row by row.  32-bit,
// wave-uniform arithmetic without runtime divisions: every workgroup runs
// this before its first load.
template <int BM, int BN, bool SYM>
__device__ __forceinline__ void tile_of(const FastArgs& a, int t, int64_t& I, int64_t& J) {
  const int TM = (int)a.TM, TN = (int)a.TN;
  if constexpr (SYM) {
    for (int i = 0; i < TM; ++i) {
      const int jmin = (i * BM) / BN;   // first column block whose last column reaches row i*BM
      const int cnt = TN - jmin;
      if (cnt <= 0) continue;
      if (t < cnt) { I = i; J = jmin + t; return; }
      t -= cnt;
    }
    I = TM; J = 0;   // unreachable for t < tiles
  } else {
    // column-major (an XCD's run of tiles shares Q columns): J = t / TM from
    // the reciprocal, exact after one correction since t < 2^24
    int j = (int)((float)t * a.rcp_tm);
    int i = t - j * TM;
    if (i < 0) { --j; i += TM; } else if (i >= TM) { ++j; i -= TM; }
    I = i;
    J = j;
  }
}

// Global -> LDS DMA of 16 (or 4) bytes per lane: lane l's bytes land at LDS
// address lds + 16*l (4*l).  Written as inline asm so the compiler does not
// treat the asynchronous LDS write as pending before every later LDS read;
// the kernel orders it explicitly with s_waitcnt vmcnt + s_barrier.  The
// instruction has no register results; its address operands are read at
// issue.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ void dma16(const uint8_t* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(const uint8_t* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(base), "s"(lds)
               : "memory", "m0");
}

// Per-lane DMA sources of the regions this wave loads, as byte offsets from
// the operand's base at k = 0 (codes < 2^30 bytes, checked at the API); the
// base, advanced by each stage's K offset, is wave-uniform and lives in
// scalar registers.  Rows past the matrix edge are clamped to the last row:
// they feed only outputs that the epilogue masks.
template <class C>
struct StageSrc {
  uint32_t code[C::kCodeLoads];
  uint32_t scale[C::kScaleLoads];
};

template <class C>
__device__ __forceinline__ int code_region(int wave, int q) {
  const int r = wave + q * C::kWaves;
  return r < C::kRegions ? r : r - C::kWaves;
}
template <class C>
__device__ __forceinline__ int scale_group(int wave, int q) {
  const int r = wave + q * C::kWaves;
  return r < C::kScaleRegions ? r : r - C::kWaves;
}

// Row-line stages (BK = 256): a 32-row group's stage is 32 rows x 128 bytes
// (eight 16-byte chunks of 32 codes), stored in LDS row by row with chunk c
// of row r at position c ^ row_swizzle(r).  A DMA instruction then reads 8
// whole rows -- eight full 128-byte lines -- and the fragment reads below
// (16 consecutive lanes = 16 rows, one chunk each) hit 16 distinct 16-byte
// bank slots, as do any 8 consecutive lanes.
__device__ __forceinline__ int row_swizzle(int r) { return (r ^ (r >> 3)) & 7; }

// K map of a row-line stage: lane half h takes chunks 4h .. 4h+3; quarter
// qs of the stage feeds its four MFMA steps from chunk 4h + qs, one word
// (8 codes, two per byte) per step.  Scale block b of the stage covers
// chunk b / 2, so the lane's 8 scale bytes are blocks 8h .. 8h+7.

template <class C>
__device__ __forceinline__ void init_sources(const GemmProblem& g, int64_t m0, int64_t n0, int wave,
                                             int lane, StageSrc<C>& src) {
  const int64_t kb = g.K / 2, sb = g.K / 16;
  if constexpr (C::kLines) {
#pragma unroll
    for (int q = 0; q < C::kCodeLoads; ++q) {
      // region r: rows 8*(r%4) .. +7 of group r/4, lane = row * 8 + position
      const int r = code_region<C>(wave, q), grp = r / 4;
      const int rr = 8 * (r % 4) + (lane >> 3);
      const bool isP = grp < C::GP;
      int64_t row = (isP ? m0 + 32 * grp : n0 + 32 * (grp - C::GP)) + rr;
      const int64_t lim = isP ? g.M : g.N;
      row = row < lim ? row : lim - 1;
      src.code[q] = (uint32_t)(row * kb + 16 * ((lane & 7) ^ row_swizzle(rr)));
    }
#pragma unroll
    for (int q = 0; q < C::kScaleLoads; ++q) {
      // region r: groups 2r and 2r+1, one row (16 scale bytes) per lane
      const int grp = 2 * scale_group<C>(wave, q) + (lane >> 5);
      const bool isP = grp < C::GP;
      int64_t row = (isP ? m0 + 32 * grp : n0 + 32 * (grp - C::GP)) + (lane & 31);
      const int64_t lim = isP ? g.M : g.N;
      row = row < lim ? row : lim - 1;
      src.scale[q] = (uint32_t)(row * sb);
    }
    return;
  }
#pragma unroll
  for (int q = 0; q < C::kCodeLoads; ++q) {
    const int r = code_region<C>(wave, q), grp = r / C::kHalves, hs = r % C::kHalves;
    const bool isP = grp < C::GP;
    int64_t row = (isP ? m0 + 32 * grp : n0 + 32 * (grp - C::GP)) + (lane & 31);
    const int64_t lim = isP ? g.M : g.N;
    row = row < lim ? row : lim - 1;
    // lane half h owns bytes [h*BK/4, (h+1)*BK/4) of the row's BK/2 stage bytes
    src.code[q] = (uint32_t)(row * kb + (C::BK / 4) * (lane >> 5) + 16 * hs);
  }
#pragma unroll
  for (int q = 0; q < C::kScaleLoads; ++q) {
    const int grp = scale_group<C>(wave, q);
    const bool isP = grp < C::GP;
    int64_t row = (isP ? m0 + 32 * grp : n0 + 32 * (grp - C::GP)) + (lane & 31);
    const int64_t lim = isP ? g.M : g.N;
    row = row < lim ? row : lim - 1;
    // 8 scale bytes per row and stage, lane half h loads its 4
    src.scale[q] = (uint32_t)(row * sb + 4 * (lane >> 5));
  }
}

template <class C>
__device__ __forceinline__ void issue_stage(const GemmProblem& g, const StageSrc<C>& src, int64_t k0,
                                            uint8_t* stage, int wave) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(stage));
#pragma unroll
  for (int q = 0; q < C::kCodeLoads; ++q) {
    const int r = code_region<C>(wave, q);
    const uint8_t* op = (r / C::kHalves < C::GP ? g.codes_p : g.codes_q) + k0 / 2;
    dma16(op, src.code[q], base + (uint32_t)r * 1024u);
  }
#pragma unroll
  for (int q = 0; q < C::kScaleLoads; ++q) {
    const int sr = scale_group<C>(wave, q);
    if constexpr (C::kLines) {
      // groups 2sr (lanes 0-31) and 2sr+1 share one operand: GP is even
      const uint8_t* op = (2 * sr < C::GP ? g.scales_p : g.scales_q) + k0 / 16;
      dma16(op, src.scale[q], base + (uint32_t)C::kCodeBytes + (uint32_t)sr * 1024u);
    } else {
      const uint8_t* op = (sr < C::GP ? g.scales_p : g.scales_q) + k0 / 16;
      dma4(op, src.scale[q], base + (uint32_t)C::kCodeBytes + (uint32_t)sr * 256u);
    }
  }
}

struct EpCtx {
  float scale, beta;
  int N;
  int64_t m0, n0;       // tile origin
  int dr0, dc0;         // this lane's first row / column inside the tile
  bool fast;            // tile wholly inside the matrix and above the diagonal
  bool mirror;          // symmetric: store the transpose below the diagonal
};

template <class C, bool SYM>
__device__ __forceinline__ EpCtx epilogue_ctx(const GemmProblem& g, int64_t m0, int64_t n0, int wm,
                                              int wn, int lane) {
  EpCtx e;
  e.scale = g.alpha * (*g.sg_p) * (*g.sg_q);
  e.beta = g.beta;
  e.N = (int)g.N;
  e.m0 = m0;
  e.n0 = n0;
  e.dr0 = wm * C::FM * 32 + 4 * (lane >> 5);
  e.dc0 = wn * C::FN * 32 + (lane & 31);
  const bool inside = m0 + C::BM <= g.M && n0 + C::BN <= g.N;
  const bool upper = !SYM || (m0 + C::BM <= n0);        // every element has row < col
  e.fast = inside && upper;
  e.mirror = !(g.upper_only && m0 + C::BM <= n0);
  return e;
}

// The addend of one 32 x 32 block (i, j) of a wave's sub-tile in the MFMA
// output layout (0 outside the matrix or below a symmetric diagonal).
template <class C, bool SYM>
__device__ __forceinline__ void load_addend_block(const GemmProblem& g, const EpCtx& e, int i, int j,
                                                  float (&ad)[16]) {
  const int N = e.N;
  const float* atile = g.addend + e.m0 * g.N + e.n0;
  const int lo = e.dr0 * N + e.dc0;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int dr = i * 32 + 8 * (r >> 2) + (r & 3);
    const int64_t row = e.m0 + e.dr0 + dr, col = e.n0 + e.dc0 + j * 32;
    const bool ok = e.fast || (row < g.M && col < g.N && (!SYM || row <= col));
    ad[r] = ok ? atile[lo + dr * N + j * 32] : 0.0f;
  }
}

// The epilogue of one 32 x 32 block (i, j) of a wave's sub-tile, for the
// reduce kernel (v holds the block's 16 values per lane in the MFMA output
// layout, ad its addend); the same arithmetic as `epilogue` below, which
// keeps its own copy because sharing this one raises the product kernel's
// register count.
template <class C, bool SYM>
__device__ __forceinline__ void epilogue_block(const GemmProblem& g, const EpCtx& e, const floatx16& v16,
                                               const float (&ad)[16], int i, int j, uint32_t& amax) {
  const int N = e.N;
  // wave-uniform tile bases and 32-bit lane offsets (BM * N < 2^31)
  float* otile = g.out + e.m0 * g.N + e.n0;
  const bool atile = g.addend != nullptr;
  float* mtile = g.out + e.n0 * g.N + e.m0;           // mirror: (col, row)
  const int lo = e.dr0 * N + e.dc0, mo = e.dc0 * N + e.dr0;
  auto valid = [&](int dr) {
    if (e.fast) return true;
    const int64_t row = e.m0 + e.dr0 + dr, col = e.n0 + e.dc0 + j * 32;
    return row < g.M && col < g.N && (!SYM || row <= col);
  };
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float v4[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int r = 4 * q + t;
      const int dr = i * 32 + 8 * q + t;               // row offset from the lane's first row
      float v = e.scale * v16[r];
      if (atile) v = fmaf(e.beta, ad[r], v);
      if (valid(dr)) {
        otile[lo + dr * N + j * 32] = v;
        const uint32_t ab = abs_bits(v);
        amax = ab > amax ? ab : amax;
      }
      v4[t] = v;
    }
    if constexpr (SYM) {
      // mirror: rows dr..dr+3 of column c become 4 consecutive floats
      // (none for a tile above the diagonal of an upper_only product)
      const int moff = mo + (j * 32) * N + i * 32 + 8 * q;
      if (!e.mirror) {
        // lower triangle not stored
      } else if (e.fast) {
        *reinterpret_cast<float4*>(mtile + moff) = make_float4(v4[0], v4[1], v4[2], v4[3]);
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int64_t row = e.m0 + e.dr0 + i * 32 + 8 * q + t, col = e.n0 + e.dc0 + j * 32;
          if (row < g.M && col < g.N && row < col) mtile[moff + t] = v4[t];
        }
      }
    }
  }
}

// out = beta * addend + alpha * sgP * sgQ * acc for the tile at (m0, n0);
// symmetric products write row <= col and mirror row < col (with
// upper_only, only inside the tiles that touch the diagonal).  amax of the
// written values goes to amax_out.  Offsets inside a tile are 32-bit
// (BM * N < 2^31 is checked at the API); tiles wholly inside the matrix
// (and, if symmetric, wholly above the diagonal) skip the per-element tests.
//
// The addend values of this lane's outputs (MFMA output layout), loaded by
// the kernel while the tile's last K-stage still computes so that the
// epilogue finds them in registers; positions outside the matrix (or below
// the diagonal of a symmetric product) read as 0.
template <class C, bool SYM>
__device__ __forceinline__ void load_addend(const GemmProblem& g, int64_t m0, int64_t n0, int wm, int wn,
                                            int lane, float (&ad)[C::FM][C::FN][16]) {
  const int N = (int)g.N;
  const int64_t r0 = m0 + wm * C::FM * 32 + 4 * (lane >> 5);
  const int64_t c0 = n0 + wn * C::FN * 32 + (lane & 31);
  const float* abase = g.addend + r0 * g.N + c0;
  const bool fast = m0 + C::BM <= g.M && n0 + C::BN <= g.N && (!SYM || m0 + C::BM <= n0);
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int dr = i * 32 + 8 * (r >> 2) + (r & 3);
        const int64_t row = r0 + dr, col = c0 + j * 32;
        const bool ok = fast || (row < g.M && col < g.N && (!SYM || row <= col));
        ad[i][j][r] = ok ? abase[dr * N + j * 32] : 0.0f;
      }
}

// In place (addend == out) every position is read, by load_addend, before
// the lane that owns it stores it, and mirrored stores land below the
// diagonal, which no tile reads.
//
// KEEP (transformed maxima follow): acc keeps the written values, 0 outside
// the matrix, and no amax is published here.
template <class C, bool SYM, bool KEEP = false>
__device__ __forceinline__ void epilogue(const GemmProblem& g, floatx16 (&acc)[C::FM][C::FN],
                                         const float (&ad)[C::FM][C::FN][16], int64_t m0, int64_t n0,
                                         int wm, int wn, int lane) {
  const float scale = g.alpha * (*g.sg_p) * (*g.sg_q);
  const float beta = g.beta;
  const int h = lane >> 5, c32 = lane & 31;
  const int N = (int)g.N;
  const int64_t r0 = m0 + wm * C::FM * 32 + 4 * h;     // first row of this lane
  const int64_t c0 = n0 + wn * C::FN * 32 + c32;       // first column of this lane
  float* obase = g.out + r0 * g.N + c0;
  const bool add = g.addend != nullptr;
  float* mbase = g.out + c0 * g.N + r0;                // mirror: (col, row)
  const bool inside = m0 + C::BM <= g.M && n0 + C::BN <= g.N;
  const bool upper = !SYM || (m0 + C::BM <= n0);       // every element has row < col
  const bool mirror = !(upper && g.upper_only);
  auto valid = [&](int dr, int j) {
    if (inside && upper) return true;
    const int64_t row = r0 + dr, col = c0 + j * 32;
    return row < g.M && col < g.N && (!SYM || row <= col);
  };
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float v4[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int r = 4 * q + t;
          const int dr = i * 32 + 8 * q + t;           // row offset from r0
          float v = scale * acc[i][j][r];
          if (add) v = fmaf(beta, ad[i][j][r], v);
          if (valid(dr, j)) {
            obase[dr * N + j * 32] = v;
            const uint32_t ab = abs_bits(v);
            amax = ab > amax ? ab : amax;
          }
          if constexpr (KEEP) acc[i][j][r] = (r0 + dr < g.M && c0 + j * 32 < g.N) ? v : 0.0f;
          v4[t] = v;
        }
        if constexpr (SYM) {
          // mirror: rows r0+dr..+3 of column c become 4 consecutive floats
          const int moff = (j * 32) * N + i * 32 + 8 * q;
          if (!mirror) {
            // upper_only: lower triangle not stored
          } else if (inside && upper) {
            *reinterpret_cast<float4*>(mbase + moff) = make_float4(v4[0], v4[1], v4[2], v4[3]);
          } else {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const int64_t row = r0 + i * 32 + 8 * q + t, col = c0 + j * 32;
              if (row < g.M && col < g.N && row < col) mbase[moff + t] = v4[t];
            }
          }
        }
      }
    }
  if constexpr (!KEEP)
    if (g.amax_out) amax_publish_wave(amax, g.amax_out, g.amax_parts != 0);
}

// max |x H^r| over one 16-block x (raw float bits), as rht16 followed by
// the maximum of the magnitudes would give it: the same sign flips and FP32
// butterfly, with the final multiplication by 1/4 applied once to the
// largest magnitude (x -> RN(x / 4) is monotone and odd, so the largest of
// the rounded quarters is the rounded quarter of the largest; NaN stays NaN).
__device__ __forceinline__ uint32_t rht16_amax(const uint32_t (&v)[16], uint32_t mask) {
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
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const uint32_t a = abs_bits(__float_as_uint(f[j]));
    m = a > m ? a : m;
  }
  return __float_as_uint(__uint_as_float(m) * 0.25f);
}

// Workgroup barrier after this wave's LDS accesses have completed (global
// memory operations stay in flight).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Transformed maxima of the tile the epilogue just wrote (its values in acc,
// 0 outside the matrix), staged through the idle stage buffers as a
// BM x BN float tile: every 16-block of a row (and of a column) is multiplied
// by H^r in the operation order of the quantizer's own transform (rht16_amax),
// so the maxima are those of the tensor the quantizer encodes, bit for bit.
// Symmetric, upper-only products: a diagonal tile is completed from its
// upper triangle (the mirror the epilogue stores) and counts its rows; a
// tile above the diagonal counts its rows and its columns (the rows of its
// mirror), both into amax_out.  Otherwise rows go to amax_out and columns to
// amax_out_c.
template <class C, bool SYM>
__device__ __forceinline__ void rht_tile_maxima(const GemmProblem& g, const floatx16 (&acc)[C::FM][C::FN],
                                                int64_t m0, int64_t n0, int wm, int wn, int lane,
                                                uint8_t* smem) {
  constexpr int LD = C::BN + 4;   // row pitch in floats (16-byte aligned rows)
  static_assert((size_t)C::BM * LD * 4 <= (size_t)C::NST * C::kStage, "tile does not fit the stage buffers");
  float* T = reinterpret_cast<float*>(smem);
  const bool diag = SYM && m0 == n0;
  const int h = lane >> 5, c32 = lane & 31;
  // Barriers that order LDS only: __syncthreads' workgroup fence would also
  // wait for the epilogue's global stores, which nothing here reads.  Every
  // wave is done with the stage buffers here (their DMA writes were waited
  // for in the last K-stage, their reads fed the MFMAs).
  lds_barrier();
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int dr = wm * C::FM * 32 + i * 32 + 8 * (r >> 2) + (r & 3) + 4 * h;
        const int dc = wn * C::FN * 32 + j * 32 + c32;
        const float v = acc[i][j][r];
        if (!diag || dr <= dc) T[dr * LD + dc] = v;
        if (diag && dr < dc) T[dc * LD + dr] = v;
      }
  lds_barrier();
  uint32_t mr = 0, mc = 0;
  const int tid = (int)threadIdx.x;
  constexpr int kRowBlocks = C::BM * (C::BN / 16), kColBlocks = (C::BM / 16) * C::BN;
  for (int b = tid; b < kRowBlocks; b += C::kThreads) {
    const int row = b / (C::BN / 16), cb = b % (C::BN / 16);
    uint32_t v[16];
#pragma unroll
    for (int e = 0; e < 16; e += 4) {
      const float4 w = *reinterpret_cast<const float4*>(T + row * LD + 16 * cb + e);
      v[e] = __float_as_uint(w.x);
      v[e + 1] = __float_as_uint(w.y);
      v[e + 2] = __float_as_uint(w.z);
      v[e + 3] = __float_as_uint(w.w);
    }
    const uint32_t a = rht16_amax(v, g.rht_mask);
    mr = a > mr ? a : mr;
  }
  if (!diag) {
    for (int b = tid; b < kColBlocks; b += C::kThreads) {
      const int col = b % C::BN, rb = b / C::BN;
      uint32_t v[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) v[e] = __float_as_uint(T[(16 * rb + e) * LD + col]);
      const uint32_t a = rht16_amax(v, g.rht_mask);
      mc = a > mc ? a : mc;
    }
  }
  if constexpr (SYM) {
    mr = mc > mr ? mc : mr;
    if (g.amax_out) amax_publish_wave(mr, g.amax_out, g.amax_parts != 0);
  } else {
    if (g.amax_out) amax_publish_wave(mr, g.amax_out, g.amax_parts != 0);
    if (g.amax_out_c) amax_publish_wave(mc, g.amax_out_c, g.amax_parts != 0);
  }
}

// FP32 partials of a K-part: per (block b = i*FN + j, quarter q) a run of
// kThreads float4 (lane-major), so that a reader of one block and one wave
// loads contiguous kilobytes.
template <class C>
__device__ __forceinline__ size_t partial_index(int b, int q, int thread) {
  return ((size_t)(b * 4 + q) * C::kThreads + thread) * 4;
}

// FIXUP: the last K-part of a split tile sums the parts (a.counters set);
// otherwise gemm_reduce_kernel does.  Two instantiations, so that products
// without split tiles keep the plain kernel's code.
// BATCH: one problem per grid row (select_problem); a separate
// instantiation, so that single launches keep the plain kernel's code.
// `t` must stay the first parameter: table_out reads it at offset 0 of the
// kernel-argument segment.
// RHTMAX: transformed maxima instead of max |out| (rht_tile_maxima); a
// separate instantiation, so that the other launches keep their code.
template <class C, bool SYM, bool FIXUP, bool BATCH, bool RHTMAX = false>
__global__ __launch_bounds__(C::kThreads, C::kMinBlocks) void gemm_fast_kernel(const OutTable t, FastArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::NST * C::kStage];
  __shared__ uint32_t last_part;
  if constexpr (BATCH) select_problem<RHTMAX>(a, t.n);
  const GemmProblem& g = a.g;
  if constexpr (RHTMAX) {
    if (blockIdx.x == 0) {
      if (g.clear_a) amax_clear(g.clear_a);
      if (g.clear_b) amax_clear(g.clear_b);
    }
  }

  // ---- work unit: a whole tile or a K-part of a leftover tile (unit_of)
  Unit un;
  if (!unit_of(a, (int)blockIdx.x, un)) return;
  const int nparts = un.split < 0 ? 1 : a.parts;
  int64_t I, J;
  tile_of<C::BM, C::BN, SYM>(a, un.tile, I, J);
  const int64_t m0 = I * C::BM, n0 = J * C::BN;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / C::WN, wn = wave % C::WN;

  floatx16 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  StageSrc<C> src;
  init_sources<C>(g, m0, n0, wave, lane, src);

  const int64_t nk_all = g.K / C::BK;
  const int64_t kc0 = nk_all * un.part / nparts, kc1 = nk_all * (un.part + 1) / nparts;


  float ad[C::FM][C::FN][16];   // the addend, loaded during the last stage

  // prologue: stages kc0 .. kc0 + NST - 2 in flight
#pragma unroll
  for (int p = 0; p < C::NST - 1; ++p)
    if (kc0 + p < kc1) issue_stage<C>(g, src, (kc0 + p) * C::BK, smem + p * C::kStage, wave);

  // one K-stage; the last (peeled, so that the addend registers are live
  // only there) also fetches the epilogue's addend
  auto stage = [&](int64_t kc, auto last) {
    // wait for this wave's loads of stage kc (later stages may stay in
    // flight), then for every wave's; the barrier also retires all reads of
    // the buffer the next issue overwrites
    if (kc + C::NST - 2 < kc1) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"((C::NST - 2) * C::kLoadsPerWave) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();
    if (kc + C::NST - 1 < kc1)
      issue_stage<C>(g, src, (kc + C::NST - 1) * C::BK,
                     smem + ((kc - kc0 + C::NST - 1) % C::NST) * C::kStage, wave);
    // the last stage: fetch the epilogue's addend while it computes (no
    // later stage waits on vmcnt, so these loads delay nothing)
    if constexpr (decltype(last)::value)
      if (un.split < 0 && g.addend) load_addend<C, SYM>(g, m0, n0, wm, wn, lane, ad);
    const uint8_t* st = smem + ((kc - kc0) % C::NST) * C::kStage;

    // this lane's scale dword per fragment: blocks 4h..4h+3 of the stage
    // (BK = 128), as E4M3 bytes; with row lines (BK = 256) two dwords,
    // blocks 8h..8h+7
    uint32_t sp[C::FM], sq[C::FN], sp1[C::FM], sq1[C::FN];
    if constexpr (C::kLines) {
      const int so = 16 * (lane & 31) + 8 * (lane >> 5);
#pragma unroll
      for (int i = 0; i < C::FM; ++i) {
        const uint2 w = *reinterpret_cast<const uint2*>(st + C::kCodeBytes + (wm * C::FM + i) * 512 + so);
        sp[i] = w.x;
        sp1[i] = w.y;
      }
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        const uint2 w = *reinterpret_cast<const uint2*>(st + C::kCodeBytes + (C::GP + wn * C::FN + j) * 512 + so);
        sq[j] = w.x;
        sq1[j] = w.y;
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
        sp[i] = *reinterpret_cast<const uint32_t*>(st + C::kCodeBytes + (wm * C::FM + i) * 256 + 4 * lane);
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
        sq[j] = *reinterpret_cast<const uint32_t*>(st + C::kCodeBytes + (C::GP + wn * C::FN + j) * 256 + 4 * lane);
    }

#pragma unroll
    for (int hs = 0; hs < C::kHalves; ++hs) {
      uint4 cp[C::FM], cq[C::FN];
      half2_t spf[C::FM], sqf[C::FN];   // the half-stage's two block scales as f16
      if constexpr (C::kLines) {
        // chunk 4h + hs of row lane%32, at its swizzled position
        const int lo = 128 * (lane & 31) + 16 * ((4 * (lane >> 5) + hs) ^ row_swizzle(lane & 31));
#pragma unroll
        for (int i = 0; i < C::FM; ++i) {
          cp[i] = *reinterpret_cast<const uint4*>(st + (wm * C::FM + i) * 4096 + lo);
          spf[i] = scale_pair2_f16(hs < 2 ? sp[i] : sp1[i], hs & 1);
        }
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
          cq[j] = *reinterpret_cast<const uint4*>(st + (C::GP + wn * C::FN + j) * 4096 + lo);
          sqf[j] = scale_pair2_f16(hs < 2 ? sq[j] : sq1[j], hs & 1);
        }
      } else {
#pragma unroll
        for (int i = 0; i < C::FM; ++i) {
          cp[i] = *reinterpret_cast<const uint4*>(st + ((wm * C::FM + i) * C::kHalves + hs) * 1024 + 16 * lane);
          spf[i] = scale_pair2_f16(sp[i], hs);
        }
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
          cq[j] = *reinterpret_cast<const uint4*>(st + ((C::GP + wn * C::FN + j) * C::kHalves + hs) * 1024 + 16 * lane);
          sqf[j] = scale_pair2_f16(sq[j], hs);
        }
      }
      // software pipeline: step s + 1 is dequantized while step s multiplies
      half8_t av[C::FM], bv[C::FN];
#pragma unroll
      for (int i = 0; i < C::FM; ++i) av[i] = dequant8_f16(cp[i].x, splat_lo(spf[i]));
#pragma unroll
      for (int j = 0; j < C::FN; ++j) bv[j] = dequant8_f16(cq[j].x, splat_lo(sqf[j]));
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        half8_t an[C::FM], bn[C::FN];
        if (s < 3) {
#pragma unroll
          for (int i = 0; i < C::FM; ++i) {
            const uint32_t w = s == 0 ? cp[i].y : s == 1 ? cp[i].z : cp[i].w;
            an[i] = dequant8_f16(w, s + 1 < 2 ? splat_lo(spf[i]) : splat_hi(spf[i]));
          }
#pragma unroll
          for (int j = 0; j < C::FN; ++j) {
            const uint32_t w = s == 0 ? cq[j].y : s == 1 ? cq[j].z : cq[j].w;
            bn[j] = dequant8_f16(w, s + 1 < 2 ? splat_lo(sqf[j]) : splat_hi(sqf[j]));
          }
        }
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
          for (int j = 0; j < C::FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
        if (s < 3) {
#pragma unroll
          for (int i = 0; i < C::FM; ++i) av[i] = an[i];
#pragma unroll
          for (int j = 0; j < C::FN; ++j) bv[j] = bn[j];
        }
      }
    }
  };
  for (int64_t kc = kc0; kc < kc1 - 1; ++kc) stage(kc, BoolTag<false>{});
  stage(kc1 - 1, BoolTag<true>{});

  if (un.split >= 0) {
    if constexpr (!FIXUP) {
      float* part = a.partials + ((size_t)un.split * a.parts + un.part) * C::kAcc * C::kThreads;
      // gemm_reduce_kernel sums the parts in order and runs the epilogue (a
      // kernel boundary makes the partials visible without cache flushes)
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *reinterpret_cast<float4*>(part + partial_index<C>(i * C::FN + j, q, threadIdx.x)) =
                make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                            acc[i][j][4 * q + 3]);
      return;
    } else {
      // Summed here by the part that finishes last.  The partials move with
      // the sc1 cache policy -- coherent at device scope: a store completes at
      // the point all XCDs read through and a load reads from there, never a
      // stale line of the reader's L2 -- so no L2 writeback or invalidation is
      // needed.  Each part's stores complete (vmcnt 0) before it counts itself
      // done with a device-scope atomic; the part that sees every other one
      // done loads their partials after that.  In the LLVM AMDGPU memory
      // model for gfx942/gfx950 an sc1 load or store is what a relaxed
      // (monotonic) agent-scope atomic load or store lowers to, and an
      // agent-scope release or acquire adds to the vmcnt wait only an L2
      // writeback (buffer_wbl2 sc1) or invalidate (buffer_inv sc1) for data
      // NOT accessed that way.  Every access to the partials is of that kind,
      // so the wait plus the atomic give the ordering a release/acquire pair
      // would.  Making the counter update acq_rel instead (same results)
      // measured 53.5 -> 58.6 us on the 3072^2 x 3072 product and 90 -> 93 us
      // on the 3072^2 x 8192 one: the whole-L2 writeback and invalidate are
      // paid per split tile.
      constexpr int kSc1 = 16;                          // cache-policy bit sc1
      typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
      const uint32_t part_bytes = (uint32_t)(C::kAcc * C::kThreads * 4);
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          a.partials + (size_t)un.split * a.parts * C::kAcc * C::kThreads, (short)0,
          (int)(part_bytes * (uint32_t)a.parts), 0x00020000);   // raw buffer, 32-bit data format
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const u32x4 w = {__float_as_uint(acc[i][j][4 * q]), __float_as_uint(acc[i][j][4 * q + 1]),
                             __float_as_uint(acc[i][j][4 * q + 2]), __float_as_uint(acc[i][j][4 * q + 3])};
            __builtin_amdgcn_raw_buffer_store_b128(
                w, rs, (int)(un.part * part_bytes + 4 * partial_index<C>(i * C::FN + j, q, threadIdx.x)),
                0, kSc1);
          }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();                                  // every wave's partial is stored
      if (threadIdx.x == 0) {
        const uint32_t done = __hip_atomic_fetch_add(a.counters + un.split, 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        const bool last = done == (uint32_t)(a.parts - 1);
        // every other part has counted itself: leave the counter zero for the
        // next launch
        if (last) __hip_atomic_store(a.counters + un.split, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last_part = last ? 1u : 0u;
      }
      __syncthreads();
      if (last_part == 0u) return;
      // part by part in part order: a part's whole partial (16 loads in
      // flight) is added to the running sum; this part's own values come
      // from registers.  sum = p0, then sum += p1, += p2, ... as
      // gemm_reduce_kernel adds them.
      floatx16 sum[C::FM][C::FN];
      for (int p = 0; p < a.parts; ++p) {
        floatx16 v[C::FM][C::FN];
        if (p == un.part) {
#pragma unroll
          for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int j = 0; j < C::FN; ++j) v[i][j] = acc[i][j];
        } else {
#pragma unroll
          for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int j = 0; j < C::FN; ++j)
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(
                    rs, (int)(p * part_bytes + 4 * partial_index<C>(i * C::FN + j, q, threadIdx.x)),
                    0, kSc1);
#pragma unroll
                for (int t = 0; t < 4; ++t) v[i][j][4 * q + t] = __uint_as_float(w[t]);
              }
        }
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
          for (int j = 0; j < C::FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) sum[i][j][r] = p == 0 ? v[i][j][r] : sum[i][j][r] + v[i][j][r];
      }
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) acc[i][j] = sum[i][j];
      if (g.addend) load_addend<C, SYM>(g, m0, n0, wm, wn, lane, ad);
    }
  }
  if constexpr (RHTMAX) {
    epilogue<C, SYM, true>(g, acc, ad, m0, n0, wm, wn, lane);
    rht_tile_maxima<C, SYM>(g, acc, m0, n0, wm, wn, lane, smem);
  } else {
    epilogue<C, SYM>(g, acc, ad, m0, n0, wm, wn, lane);
  }
}

// One wave per workgroup: block (i, j) of wave w's sub-tile of split tile
// s, summed over the K-parts in part order, then that block's epilogue.
// Workgroups: split tiles x waves x FM x FN, so the partials stream in
// with many loads in flight.
template <class C, bool SYM, bool BATCH>   // `t` first, as in gemm_fast_kernel
__global__ __launch_bounds__(64) void gemm_reduce_kernel(const OutTable t, FastArgs a) {
  constexpr int kBlocks = C::FM * C::FN;
  if constexpr (BATCH) select_problem<false>(a, t.n);
  const int bid = (int)blockIdx.x;
  const int s = bid / (C::kWaves * kBlocks), rem = bid % (C::kWaves * kBlocks);
  const int w = rem / kBlocks, b = rem % kBlocks, i = b / C::FN, j = b % C::FN;
  const int tile = split_tile(a, s);
  if (tile < 0) return;
  int64_t I, J;
  tile_of<C::BM, C::BN, SYM>(a, tile, I, J);
  const int lane = threadIdx.x & 63;
  const int thread = w * 64 + lane;                 // the lane's thread in the product kernel
  const float* base = a.partials + (size_t)s * a.parts * C::kAcc * C::kThreads;
  const EpCtx e = epilogue_ctx<C, SYM>(a.g, I * C::BM, J * C::BN, w / C::WN, w % C::WN, lane);
  // every load first (addend, then all parts), so that the block costs one
  // memory round trip; then the sum in part order
  float ad[16];
  if (a.g.addend) load_addend_block<C, SYM>(a.g, e, i, j, ad);
  float4 u[kMaxParts][4];
#pragma unroll
  for (int p = 0; p < kMaxParts; ++p)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (p < a.parts)
        u[p][q] = *reinterpret_cast<const float4*>(base + (size_t)p * C::kAcc * C::kThreads +
                                                   partial_index<C>(b, q, thread));
  floatx16 v;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float4 t = u[0][q];
#pragma unroll
    for (int p = 1; p < kMaxParts; ++p)
      if (p < a.parts) {
        t.x += u[p][q].x; t.y += u[p][q].y; t.z += u[p][q].z; t.w += u[p][q].w;
      }
    v[4 * q] = t.x; v[4 * q + 1] = t.y; v[4 * q + 2] = t.z; v[4 * q + 3] = t.w;
  }
  uint32_t amax = 0;
  epilogue_block<C, SYM>(a.g, e, v, ad, i, j, amax);
  if (a.g.amax_out) amax_publish_wave(amax, a.g.amax_out, a.g.amax_parts != 0);
}

// ===========================================================================
// General path: any K that is a multiple of 16 (register-staged loads with
// zero fill past K).  128 x 128 tile, 4 waves of 64 x 64.
// ===========================================================================

constexpr int GBM = 128, GBN = 128, GBK = 128, GThreads = 256;
constexpr int kCodeStride = GBK / 2 + 16;
constexpr int kScaleStride = 12;
constexpr int kCodeTile = GBM * kCodeStride;
constexpr int kScaleTile = GBM * kScaleStride;
constexpr int kGStage = 2 * kCodeTile + 2 * kScaleTile;

struct TileLoad {
  uint2 pc[4], qc[4];
  uint32_t ps, qs;
};

__device__ __forceinline__ void load_tile(const GemmProblem& g, int64_t m0, int64_t n0, int64_t k0,
                                          TileLoad& t) {
  const int tid = threadIdx.x;
  const int64_t kb = g.K / 2;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = tid + GThreads * i;
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
  const int row = tid >> 1, part = tid & 1;
  const int64_t sb = g.K / 16;
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

__device__ __forceinline__ void store_tile(uint8_t* stage, const TileLoad& t) {
  const int tid = threadIdx.x;
  uint8_t* sp = stage;
  uint8_t* sq = stage + kCodeTile;
  uint8_t* sps = stage + 2 * kCodeTile;
  uint8_t* sqs = sps + kScaleTile;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = tid + GThreads * i;
    const int row = idx >> 3, chunk = idx & 7;
    *reinterpret_cast<uint2*>(sp + row * kCodeStride + chunk * 8) = t.pc[i];
    *reinterpret_cast<uint2*>(sq + row * kCodeStride + chunk * 8) = t.qc[i];
  }
  const int row = tid >> 1, part = tid & 1;
  *reinterpret_cast<uint32_t*>(sps + row * kScaleStride + part * 4) = t.ps;
  *reinterpret_cast<uint32_t*>(sqs + row * kScaleStride + part * 4) = t.qs;
}

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

template <bool SYM>
__global__ __launch_bounds__(GThreads, 2) void gemm_general_kernel(GemmProblem g) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kGStage];
  int64_t ti, tj;
  if constexpr (SYM) {
    const int64_t nt = (g.M + GBM - 1) / GBM;
    int64_t rem = blockIdx.x, r = 0;
    while (rem >= nt - r) { rem -= nt - r; ++r; }
    ti = r;
    tj = r + rem;
  } else {
    // one-dimensional grid, row-major over tiles (no 65535 cap on tile rows)
    const uint32_t tn = (uint32_t)((g.N + GBN - 1) / GBN);
    ti = blockIdx.x / tn;
    tj = blockIdx.x % tn;
  }
  const int64_t m0 = ti * GBM, n0 = tj * GBN;
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

  const int64_t nk = (g.K + GBK - 1) / GBK;
  TileLoad tl;
  load_tile(g, m0, n0, 0, tl);
  store_tile(smem, tl);
  __syncthreads();
  for (int64_t kc = 0; kc < nk; ++kc) {
    const bool more = kc + 1 < nk;
    if (more) load_tile(g, m0, n0, (kc + 1) * GBK, tl);
    const uint8_t* stage = smem + (kc & 1) * kGStage;
    Frag fp[2], fq[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      read_frag(stage, stage + 2 * kCodeTile, wm * 64 + 32 * i + r32, h, fp[i]);
      read_frag(stage + kCodeTile, stage + 2 * kCodeTile + kScaleTile, wn * 64 + 32 * i + r32, h, fq[i]);
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      half8_t av[2], bv[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        av[i] = dequant8_f16(fp[i].w[s], fp[i].s[s >> 1]);
        bv[i] = dequant8_f16(fq[i].w[s], fq[i].s[s >> 1]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
    if (more) store_tile(smem + ((kc + 1) & 1) * kGStage, tl);
    __syncthreads();
  }

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
  if (g.amax_out) amax_publish_wave(amax, g.amax_out, g.amax_parts != 0);
}

// ---------------------------------------------------------------- plans ----

// Two tile shapes: 128 x 128 (four 64 x 64 waves), and 64 x 128 (two waves)
// for products with short K whose 128 x 128 tiles would leave most of the
// GPU's workgroup slots empty.  With 128-wide stages the small tiles lose on
// long K (more operand re-reads) and win on short K.
#ifndef NVFP4_FAST_NST
#define NVFP4_FAST_NST 2
#endif
#ifndef NVFP4_BIG_SHAPE
#define NVFP4_BIG_SHAPE 2, 2, 2, 2
#endif
// K % 256 == 0 runs 128 x 128 tiles with 256-wide row-line stages: a DMA
// instruction that reads whole 128-byte lines moves its kilobyte about four
// times faster than one that gathers 32 bytes from each of 32 rows
// (measured: 9.6 TB/s gathered vs 37 TB/s from L2 over all CUs), which
// makes the short-K products fast on the big tiles too (qA qA^T at 3072^2:
// 55 us vs 63 us on the 64 x 128 tiles).  Other multiples of 128 keep the
// 128-wide stages and the tile choice below.
using BigCfg = Cfg<NVFP4_BIG_SHAPE, NVFP4_FAST_NST, 256>;
using BigCfg128 = Cfg<NVFP4_BIG_SHAPE, NVFP4_FAST_NST, 128>;
using SmallCfg128 = Cfg<1, 2, 2, 2, NVFP4_FAST_NST, 128>;
#ifndef NVFP4_SMALL_BELOW
#define NVFP4_SMALL_BELOW 512   // big-tile count below which the small tiles run
#endif
#ifndef NVFP4_SMALL_MAX_K
#define NVFP4_SMALL_MAX_K 4096  // ... when K is at most this
#endif

// Leftover tiles (see FastArgs) are split into at most cus / leftovers
// parts, each of at least NVFP4_MIN_PART_STAGES K-stages, so that every CU
// gets at most one part; products whose tiles divide evenly over the CUs of
// each XCD run unsplit.
#ifndef NVFP4_MIN_PART_K
#define NVFP4_MIN_PART_K 1024    // K per part at least
#endif

int64_t sym_tiles(int64_t TM, int64_t TN, int64_t BM, int64_t BN) {
  int64_t t = 0;
  for (int64_t i = 0; i < TM; ++i) {
    const int64_t jmin = i * BM - BN + 1 <= 0 ? 0 : (i * BM) / BN;
    if (jmin < TN) t += TN - jmin;
  }
  return t;
}

template <class C>
GemmPlan plan_with(int64_t M, int64_t N, int64_t K, bool symmetric, bool allow_split, int cfg) {
  GemmPlan p{};
  p.fast = true;
  p.cfg = cfg;
  p.TM = (M + C::BM - 1) / C::BM;
  p.TN = (N + C::BN - 1) / C::BN;
  p.tiles = symmetric ? sym_tiles(p.TM, p.TN, C::BM, C::BN) : p.TM * p.TN;
  const int cus = kCus;
  // leftover tiles of the busiest XCD run, and the units per XCD
  int64_t left_max = 0, split_tiles = 0;
  for (int x = 0; x < kXcds; ++x) {
    const int64_t n = (int64_t)(x + 1) * p.tiles / kXcds - (int64_t)x * p.tiles / kXcds;
    left_max = n % cus > left_max ? n % cus : left_max;
    split_tiles += n % cus;
  }
  int parts = 1;
  const int64_t stages = K / C::BK;
  // split only where a leftover would double a CU's work (at most one whole
  // tile per CU); with two or more the reduce pass costs more than it saves
  // (measured: 3072^2 x 8192 with one whole tile per CU gains 22 us, 3072^2
  // x 3072 with two loses 9 us)
  const bool one_per_cu = p.tiles / kXcds < 2 * cus;
  if (allow_split && left_max > 0 && one_per_cu) {
    int64_t q = cus / left_max;
    if (q > NVFP4_MAX_PARTS) q = NVFP4_MAX_PARTS;
    if (q > K / NVFP4_MIN_PART_K) q = K / NVFP4_MIN_PART_K;
    if (q > stages) q = stages;
    parts = q >= 2 ? (int)q : 1;
  }
  p.splits = parts;
  int64_t per_xcd = 0;
  for (int x = 0; x < kXcds; ++x) {
    const int64_t n = (int64_t)(x + 1) * p.tiles / kXcds - (int64_t)x * p.tiles / kXcds;
    const int64_t whole = parts > 1 ? n / cus * cus : n;
    const int64_t u = whole + (n - whole) * parts;
    per_xcd = u > per_xcd ? u : per_xcd;
  }
  p.units = per_xcd * kXcds;            // the grid
  p.split_tiles = parts > 1 ? split_tiles : 0;
  p.fixup = parts > 1 && stages >= NVFP4_FIXUP_MIN_STAGES &&
            (size_t)p.split_tiles * sizeof(uint32_t) <= kGemmCounterBytes;
  if (parts > 1) {
    const size_t part = (size_t)p.split_tiles * parts * C::kAcc * C::kThreads * sizeof(float);
    p.partial_bytes = (part + 255) / 256 * 256;
    p.ws_bytes = kGemmCounterBytes + p.partial_bytes;
  }
  return p;
}

__global__ void zero_counters_kernel(uint32_t* c, int n) {
  for (int i = (int)threadIdx.x; i < n; i += (int)blockDim.x) c[i] = 0u;
}

template <class C>
hipError_t launch_with(const GemmProblem& g, const GemmPlan& p, void* ws, bool zero_counters,
                       hipStream_t s) {
  FastArgs a;
  a.g = g;
  a.TM = p.TM;
  a.TN = p.TN;
  a.tiles = p.tiles;
  a.rcp_tm = 1.0f / (float)p.TM;
  a.parts = p.splits;
  a.partials = p.splits > 1 ? reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + kGemmCounterBytes)
                            : nullptr;
  a.counters = p.fixup ? static_cast<uint32_t*>(ws) : nullptr;
  a.bstride = g.batch > 1 ? g.batch_stride : 0;
  OutTable t{};
  if (g.batch > 1 && g.out_each) {
    if (g.batch > kMaxBatchOut) return hipErrorInvalidValue;
    t.n = g.batch;
    for (int i = 0; i < g.batch; ++i) t.outs[i] = g.out_each[i];
  }
  if (g.batch > 1 && zero_counters) return hipErrorInvalidValue;
  if (p.fixup && zero_counters) {
    zero_counters_kernel<<<1, 256, 0, s>>>(a.counters, (int)p.split_tiles);
    const hipError_t ez = hipGetLastError();
    if (ez != hipSuccess) return ez;
  }
  const dim3 grid((unsigned)p.units, (unsigned)g.batch);
  const bool b = g.batch > 1;
#define NVFP4_FAST(SY, FX)                                                              \
  do {                                                                                  \
    if (b) gemm_fast_kernel<C, SY, FX, true><<<grid, C::kThreads, 0, s>>>(t, a);        \
    else gemm_fast_kernel<C, SY, FX, false><<<grid, C::kThreads, 0, s>>>(t, a);         \
  } while (0)
#define NVFP4_RHT(SY, FX)                                                               \
  do {                                                                                  \
    if (b) gemm_fast_kernel<C, SY, FX, true, true><<<grid, C::kThreads, 0, s>>>(t, a);  \
    else gemm_fast_kernel<C, SY, FX, false, true><<<grid, C::kThreads, 0, s>>>(t, a);   \
  } while (0)
  if (g.rht_on) {
    // transformed maxima: 128 x 128 row-line tiles, no second summing
    // kernel (plan_rht_maxima)
    if constexpr (C::kLines && C::BM == 128 && C::BN == 128) {
      if (p.splits > 1 && !p.fixup) return hipErrorInvalidValue;
      if (g.symmetric && p.fixup) NVFP4_RHT(true, true);
      else if (g.symmetric) NVFP4_RHT(true, false);
      else if (p.fixup) NVFP4_RHT(false, true);
      else NVFP4_RHT(false, false);
      return hipGetLastError();
    } else {
      return hipErrorInvalidValue;
    }
  }
  if (g.symmetric && p.fixup) NVFP4_FAST(true, true);
  else if (g.symmetric) NVFP4_FAST(true, false);
  else if (p.fixup) NVFP4_FAST(false, true);
  else NVFP4_FAST(false, false);
#undef NVFP4_FAST
#undef NVFP4_RHT
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1 || p.fixup) return e;
  const dim3 rgrid((unsigned)(p.split_tiles * C::kWaves * C::FM * C::FN), (unsigned)g.batch);
  if (g.symmetric && b) gemm_reduce_kernel<C, true, true><<<rgrid, 64, 0, s>>>(t, a);
  else if (g.symmetric) gemm_reduce_kernel<C, true, false><<<rgrid, 64, 0, s>>>(t, a);
  else if (b) gemm_reduce_kernel<C, false, true><<<rgrid, 64, 0, s>>>(t, a);
  else gemm_reduce_kernel<C, false, false><<<rgrid, 64, 0, s>>>(t, a);
  return hipGetLastError();
}

}  // namespace

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, bool symmetric, bool allow_split) {
  if (K % 128 != 0) {
    GemmPlan p{};
    p.fast = false;
    p.splits = 1;
    return p;
  }
  if (K % 256 == 0) return plan_with<BigCfg>(M, N, K, symmetric, allow_split, 0);
  const GemmPlan big = plan_with<BigCfg128>(M, N, K, symmetric, allow_split, 2);
  if (big.tiles >= NVFP4_SMALL_BELOW || K > NVFP4_SMALL_MAX_K) return big;
  return plan_with<SmallCfg128>(M, N, K, symmetric, allow_split, 3);
}

hipError_t launch_gemm(const GemmProblem& g, const GemmPlan& p, void* ws, bool zero_counters,
                       hipStream_t s) {
  if (g.batch < 1 || (g.batch > 1 && (!p.fast || g.batch_stride <= 0))) return hipErrorInvalidValue;
  if (g.rht_on && !plan_rht_maxima(p)) return hipErrorInvalidValue;
  if (!p.fast) {
    if (g.symmetric) {
      const int64_t nt = (g.M + GBM - 1) / GBM;
      gemm_general_kernel<true><<<dim3((unsigned)(nt * (nt + 1) / 2)), GThreads, 0, s>>>(g);
    } else {
      const int64_t tiles = ((g.N + GBN - 1) / GBN) * ((g.M + GBM - 1) / GBM);
      if (tiles > INT32_MAX) return hipErrorInvalidValue;
      gemm_general_kernel<false><<<dim3((unsigned)tiles), GThreads, 0, s>>>(g);
    }
    return hipGetLastError();
  }
  switch (p.cfg) {
    case 0: return launch_with<BigCfg>(g, p, ws, zero_counters, s);
    case 2: return launch_with<BigCfg128>(g, p, ws, zero_counters, s);
    default: return launch_with<SmallCfg128>(g, p, ws, zero_counters, s);
  }
}

}  // namespace nvfp4
