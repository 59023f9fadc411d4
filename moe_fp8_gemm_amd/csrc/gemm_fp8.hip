// FP8 (E4M3) GEMM with fine-grained block scaling for gfx950: dense, M-grouped
// contiguous and M-grouped masked variants share one persistent kernel template.
//
// What is computed (pages on DeepGEMM): D(bf16) = A . B^T, NT layout.  A has
// one fp32 scale per row per 128-wide K block, B one per 128x128 block
// (page "GitHub 推荐…DeepGEMM…", 问题判断).  The partial product of each K block
// comes out of the matrix cores un-scaled and is multiplied by sa*sb and added
// into an fp32 accumulator on the vector ALUs (two-level accumulation: page
// juejin.cn, sections 3 and 4(1); page "GitHub 推荐…", 创新之处).  Grouping is on
// M only (page juejin.cn, section 3); tiles of all groups are handed out by a
// single persistent scheduler (page juejin.cn, section 4(4), unified tile
// scheduler with rasterisation for L2 reuse).
//
// gfx950 design (not the pages' Hopper design):
//  * One v_mfma_f32_16x16x128_f8f6f4 consumes exactly one 128-wide scale block,
//    so every MFMA result is a complete K-block partial: it is promoted right
//    away (4 FMAs per lane) and needs no second accumulator set.
//  * Operands are swapped in the MFMA: B rows feed the A port, A rows the B
//    port.  A lane's four result registers then belong to ONE row of D, so a
//    lane needs one sa value per 16-row sub-tile, and its 4*NS columns are
//    made contiguous by the order in which B rows are placed in LDS
//    ("fragment order"), which turns the epilogue into 16-byte stores.
//  * Global -> LDS by direct-to-LDS DMA (global_load_lds_dwordx4), one
//    __shared__ buffer per pipeline stage so that the compiler's LDS-DMA
//    wait tracking distinguishes stages; STAGES-1 K blocks are in flight while
//    one is consumed.  Rows are XOR-swizzled in 16-byte slots to keep the
//    fragment reads free of bank conflicts.
//  * Persistent grid of one workgroup per CU; the tile index sequence is remapped
//    so that the 32 workgroups of one XCD work on neighbouring tiles (L2 per XCD).
#include "dgfp8_internal.h"

namespace dgfp8 {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define DG_GAS __attribute__((address_space(1)))
#define DG_LAS __attribute__((address_space(3)))

constexpr int kKBlock = 128;      // width of a scale block along K == K of one MFMA
constexpr int kMaxMaskedGroups = 1024;
constexpr int kGroupM = 8;        // raster: tiles of kGroupM consecutive M-tiles sweep N together

// s_waitcnt immediate (gfx9 encoding): vmcnt <= vm, lgkmcnt == 0, expcnt unconstrained.
template <int VM>
struct WaitVmLgkm0 {
  static constexpr int value = (VM & 0xF) | ((VM >> 4) << 14) | (0x7 << 4) | (0x0 << 8);
};

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

__device__ __forceinline__ void dma16(const void* g, DG_LAS void* l) {
  __builtin_amdgcn_global_load_lds((DG_GAS void*)g, l, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* g, DG_LAS void* l) {
  __builtin_amdgcn_global_load_lds((DG_GAS void*)g, l, 4, 0, 0);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs; overflow gives inf).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return bf16_rne(lo) | (bf16_rne(hi) << 16);
}

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int STAGES_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, STAGES = STAGES_;
  static constexpr int kWaves = WAVES_M * WAVES_N;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int MS = WM / 16, NS = WN / 16;
  static constexpr int kAChunks = BM * kKBlock / 1024;  // 1 KB DMA chunk = 8 rows x 128 B
  static constexpr int kBChunks = BN * kKBlock / 1024;
  static constexpr int kAChunksPerWave = kAChunks / kWaves;
  static constexpr int kBChunksPerWave = kBChunks / kWaves;
  static constexpr int kNSB = BN >= 128 ? BN / 128 : 1;  // B scales per tile and K block
  static constexpr int kSAPerWave = BM / kWaves;
  static constexpr int kLoadsPerStage = kAChunksPerWave + kBChunksPerWave + 1;
  static constexpr int kScaleFloats = BM + 4;
  static_assert(kAChunks % kWaves == 0 && kBChunks % kWaves == 0, "chunks per wave");
  static_assert(kSAPerWave + kNSB <= 64, "scale DMA of the last wave");
  static_assert(WN <= 128 && 128 % WN == 0, "a wave's columns lie in one 128-column scale block");
  static_assert(NS % 2 == 0, "epilogue stores 8 columns at a time");
  static_assert(STAGES >= 2 && STAGES <= 4, "stages");
};

// One LDS buffer per (config, stage, kind): distinct variables, so the compiler's
// LDS-DMA dependency tracking keeps the stages apart.
template <class C, int S>
__device__ __forceinline__ DG_LAS uint8_t* lds_a() {
  __shared__ __attribute__((aligned(1024))) uint8_t buf[C::BM * kKBlock];
  return (DG_LAS uint8_t*)buf;
}
template <class C, int S>
__device__ __forceinline__ DG_LAS uint8_t* lds_b() {
  __shared__ __attribute__((aligned(1024))) uint8_t buf[C::BN * kKBlock];
  return (DG_LAS uint8_t*)buf;
}
template <class C, int S>
__device__ __forceinline__ DG_LAS float* lds_s() {
  __shared__ __attribute__((aligned(16))) float buf[C::kScaleFloats];
  return (DG_LAS float*)buf;
}

// Per-tile state of one workgroup (all values wave-uniform except the pointers).
template <class C>
struct Tile {
  const uint8_t* a_src[C::kAChunksPerWave];   // this lane's A source at K block 0
  const uint8_t* b_src[C::kBChunksPerWave];   // this lane's B source at K block 0
  const float* sa_src;                        // this lane's scale source at K block 0 (or null)
  int64_t s_kstride;                          // K-block stride of that scale source
};

template <class C, int S>
__device__ __forceinline__ void issue_stage(const Tile<C>& t, int kb) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  DG_LAS uint8_t* la = lds_a<C, S>();
  DG_LAS uint8_t* lb = lds_b<C, S>();
  DG_LAS float* ls = lds_s<C, S>();
  const int64_t koff = (int64_t)kb * kKBlock;
#pragma unroll
  for (int j = 0; j < C::kAChunksPerWave; ++j)
    dma16(t.a_src[j] + koff, la + (wave * C::kAChunksPerWave + j) * 1024);
#pragma unroll
  for (int j = 0; j < C::kBChunksPerWave; ++j)
    dma16(t.b_src[j] + koff, lb + (wave * C::kBChunksPerWave + j) * 1024);
  // Scales: wave w fetches sa of rows [w*kSAPerWave, +kSAPerWave); the last wave's
  // next kNSB lanes fetch the B scales, which land at ls[BM + j].
  const int active = C::kSAPerWave + (wave == C::kWaves - 1 ? C::kNSB : 0);
  if (lane < active) dma4(t.sa_src + kb * t.s_kstride, ls + wave * C::kSAPerWave);
}

// Consume one stage: MS x NS MFMAs, each promoted at once into acc.
template <class C, int S>
__device__ __forceinline__ void compute_stage(f32x4 (&acc)[C::MS][C::NS], int wr, int wc) {
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15;
  const int q = lane >> 4;
  DG_LAS uint8_t* la = lds_a<C, S>();
  DG_LAS uint8_t* lb = lds_b<C, S>();
  DG_LAS float* ls = lds_s<C, S>();

  const float sb = ls[C::BM + (wc * C::WN) / 128];
  i32x8 bf[C::NS];
#pragma unroll
  for (int t = 0; t < C::NS; ++t) {
    const int row = wc * C::WN + t * 16 + r16;
    DG_LAS uint8_t* base = lb + row * kKBlock;
    const i32x4 lo = *(DG_LAS i32x4*)(base + (((2 * q) ^ swz(row)) << 4));
    const i32x4 hi = *(DG_LAS i32x4*)(base + (((2 * q + 1) ^ swz(row)) << 4));
    bf[t] = (i32x8){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  }
#pragma unroll
  for (int ms = 0; ms < C::MS; ++ms) {
    const int row = wr * C::WM + ms * 16 + r16;
    DG_LAS uint8_t* base = la + row * kKBlock;
    const i32x4 lo = *(DG_LAS i32x4*)(base + (((2 * q) ^ swz(row)) << 4));
    const i32x4 hi = *(DG_LAS i32x4*)(base + (((2 * q + 1) ^ swz(row)) << 4));
    const i32x8 af = (i32x8){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    const float s = ls[row] * sb;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < C::NS; ++t) {
      // A port <- B rows (n), B port <- A rows (m): result lane l, reg r is
      // D[m = row of lane l%16][n = 4*(l/16)+r-th row of fragment t].
      const f32x4 p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[t], af, zero, 0, 0, 0, 0, 0, 0);
      acc[ms][t][0] = __builtin_fmaf(p[0], s, acc[ms][t][0]);
      acc[ms][t][1] = __builtin_fmaf(p[1], s, acc[ms][t][1]);
      acc[ms][t][2] = __builtin_fmaf(p[2], s, acc[ms][t][2]);
      acc[ms][t][3] = __builtin_fmaf(p[3], s, acc[ms][t][3]);
    }
  }
}

// Wait until this wave's DMA for the stage about to be read has landed (with
// `later` younger stages still allowed in flight), then barrier so that every
// wave's share has landed too.  lgkmcnt(0) also retires this wave's LDS reads
// of the stage the next prefetch will overwrite.
template <class C>
__device__ __forceinline__ void wait_stage(int later) {
  constexpr int L = C::kLoadsPerStage;
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (C::STAGES == 4) {
    if (later >= 2) __builtin_amdgcn_s_waitcnt(WaitVmLgkm0<2 * L>::value);
    else if (later == 1) __builtin_amdgcn_s_waitcnt(WaitVmLgkm0<L>::value);
    else __builtin_amdgcn_s_waitcnt(WaitVmLgkm0<0>::value);
  } else if constexpr (C::STAGES == 3) {
    if (later >= 1) __builtin_amdgcn_s_waitcnt(WaitVmLgkm0<L>::value);
    else __builtin_amdgcn_s_waitcnt(WaitVmLgkm0<0>::value);
  } else {
    __builtin_amdgcn_s_waitcnt(WaitVmLgkm0<0>::value);
  }
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// One pipeline step for K block kb held in stage S; prefetches kb + STAGES - 1.
template <class C, int S>
__device__ __forceinline__ void step(const Tile<C>& t, f32x4 (&acc)[C::MS][C::NS], int kb, int kblocks,
                                     int wr, int wc) {
  // Stages issued after kb's and possibly still in flight: kb+1 .. kb+STAGES-2.
  const int left = kblocks - 1 - kb;
  wait_stage<C>(left < C::STAGES - 2 ? left : C::STAGES - 2);
  constexpr int SN = (S + C::STAGES - 1) % C::STAGES;
  if (kb + C::STAGES - 1 < kblocks) issue_stage<C, SN>(t, kb + C::STAGES - 1);
  compute_stage<C, S>(acc, wr, wc);
}

struct TileCoord {
  int mt, nt, group;   // M tile (within the group for masked), N tile, group (or -1: skip)
};

__device__ __forceinline__ int remap_for_xcd(int b, int grid) {
  // Consecutive workgroup ids go to different XCDs (round-robin dispatch); give
  // each XCD a contiguous run of the tile sequence instead.
  return (grid % 8 == 0) ? (b % 8) * (grid / 8) + b / 8 : b;
}

__device__ __forceinline__ void raster(int t, int tiles_m, int tiles_n, int& mt, int& nt) {
  const int per_group = kGroupM * tiles_n;
  const int gid = t / per_group;
  const int first_m = gid * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  const int in = t - gid * per_group;
  mt = first_m + in % gm;
  nt = in / gm;
}

template <class C, int V>
__global__ void __launch_bounds__(C::kThreads)
__attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_kernel(GemmParams p) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wr = wave / C::WAVES_N;
  const int wc = wave % C::WAVES_N;
  const int kblocks = (int)(p.k / kKBlock);
  const int tiles_n = (int)((p.n + C::BN - 1) / C::BN);
  const int64_t n_sblocks = (p.n + 127) / 128;

  // ---- tile space
  __shared__ int masked_prefix[V == kMasked ? kMaxMaskedGroups + 1 : 1];
  int tiles_m = 0, num_tiles = 0;
  if constexpr (V == kMasked) {
    // Exclusive prefix of per-group M-tile counts, from masked_m on the device.
    if (wave == 0) {
      constexpr int kPer = kMaxMaskedGroups / 64;
      int cnt[kPer];
      int sum = 0;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int g = lane * kPer + i;
        int mm = 0;
        if (g < p.num_groups) mm = p.masked_m[g];
        mm = mm < 0 ? 0 : (mm > p.m ? (int)p.m : mm);
        cnt[i] = (mm + C::BM - 1) / C::BM;
        sum += cnt[i];
      }
      int incl = sum;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off, 64);
        if (lane >= off) incl += v;
      }
      int run = incl - sum;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        masked_prefix[lane * kPer + i] = run;
        run += cnt[i];
      }
      if (lane == 63) masked_prefix[kMaxMaskedGroups] = incl;
    }
    __syncthreads();
    num_tiles = masked_prefix[kMaxMaskedGroups] * tiles_n;
  } else {
    tiles_m = (int)((p.m + C::BM - 1) / C::BM);
    num_tiles = tiles_m * tiles_n;
  }

  for (int tile = remap_for_xcd(blockIdx.x, gridDim.x); tile < num_tiles; tile += gridDim.x) {
    // ---- decode the tile
    int mt, nt, g = 0;
    int64_t m_limit = p.m;   // rows of A that exist (for clamping) / may be written
    if constexpr (V == kMasked) {
      // group: largest g with prefix[g] * tiles_n <= tile
      int lo = 0, hi = p.num_groups;          // invariant: prefix[lo]*tn <= tile < prefix[hi]*tn
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (masked_prefix[mid] * tiles_n <= tile) lo = mid; else hi = mid;
      }
      g = lo;
      const int mtiles_g = masked_prefix[g + 1] - masked_prefix[g];
      const int local = tile - masked_prefix[g] * tiles_n;
      nt = local / mtiles_g;
      mt = local % mtiles_g;
      int mm = p.masked_m[g];
      mm = mm < 0 ? 0 : (mm > p.m ? (int)p.m : mm);
      m_limit = mm;
    } else {
      raster(tile, tiles_m, tiles_n, mt, nt);
      if constexpr (V == kContiguous) {
        g = p.m_indices[(int64_t)mt * C::BM];
        if (g < 0) continue;                  // whole block is padding
      }
    }
    const int64_t m0 = (int64_t)mt * C::BM;
    const int64_t n0 = (int64_t)nt * C::BN;

    const uint8_t* A = p.a + (V == kMasked ? (int64_t)g * p.a_gs : 0);
    const float* SFA = p.sfa + (V == kMasked ? (int64_t)g * p.sfa_gs : 0);
    const uint8_t* B = p.b + (V != kDense ? (int64_t)g * p.b_gs : 0);
    const float* SFB = p.sfb + (V != kDense ? (int64_t)g * p.sfb_gs : 0);
    const int64_t a_rows = p.m;   // rows of A present in memory (per group when masked)

    // ---- per-lane DMA sources at K block 0
    Tile<C> t;
#pragma unroll
    for (int j = 0; j < C::kAChunksPerWave; ++j) {
      const int prow = (wave * C::kAChunksPerWave + j) * 8 + (lane >> 3);
      int64_t row = m0 + prow;
      row = row < a_rows ? row : a_rows - 1;
      t.a_src[j] = A + row * p.lda + (((lane & 7) ^ swz(prow)) << 4);
    }
#pragma unroll
    for (int j = 0; j < C::kBChunksPerWave; ++j) {
      const int prow = (wave * C::kBChunksPerWave + j) * 8 + (lane >> 3);
      const int wcol = prow / C::WN;
      const int pl = prow % C::WN;
      const int ft = pl / 16, fi = pl % 16;
      int64_t col = n0 + wcol * C::WN + 4 * C::NS * (fi / 4) + 4 * ft + (fi % 4);
      col = col < p.n ? col : p.n - 1;
      t.b_src[j] = B + col * p.ldb + (((lane & 7) ^ swz(prow)) << 4);
    }
    if (lane < C::kSAPerWave) {
      int64_t row = m0 + wave * C::kSAPerWave + lane;
      row = row < a_rows ? row : a_rows - 1;
      t.sa_src = SFA + row * p.sfa_sm;
      t.s_kstride = p.sfa_sk;
    } else {
      int64_t nb = n0 / 128 + (lane - C::kSAPerWave);
      nb = nb < n_sblocks ? nb : n_sblocks - 1;
      t.sa_src = SFB + nb * p.sfb_sn;
      t.s_kstride = p.sfb_sk;
    }

    f32x4 acc[C::MS][C::NS];
#pragma unroll
    for (int i = 0; i < C::MS; ++i)
#pragma unroll
      for (int j = 0; j < C::NS; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

    // ---- pipeline: all waves are done with the previous tile's stages here
    __builtin_amdgcn_s_waitcnt(WaitVmLgkm0<0>::value);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    issue_stage<C, 0>(t, 0);
    if (C::STAGES >= 3 && 1 < kblocks) issue_stage<C, 1 % C::STAGES>(t, 1);
    if (C::STAGES >= 4 && 2 < kblocks) issue_stage<C, 2 % C::STAGES>(t, 2);

    for (int kb = 0; kb < kblocks; kb += C::STAGES) {
      step<C, 0>(t, acc, kb, kblocks, wr, wc);
      if (kb + 1 < kblocks) step<C, 1 % C::STAGES>(t, acc, kb + 1, kblocks, wr, wc);
      if constexpr (C::STAGES >= 3)
        if (kb + 2 < kblocks) step<C, 2 % C::STAGES>(t, acc, kb + 2, kblocks, wr, wc);
      if constexpr (C::STAGES >= 4)
        if (kb + 3 < kblocks) step<C, 3 % C::STAGES>(t, acc, kb + 3, kblocks, wr, wc);
    }

    // ---- epilogue: bf16 RNE, 16-byte stores of 8 consecutive columns
    uint16_t* D = p.d + (V == kMasked ? (int64_t)g * p.d_gs : 0);
    const int r16 = lane & 15;
    const int q = lane >> 4;
#pragma unroll
    for (int ms = 0; ms < C::MS; ++ms) {
      const int64_t row = m0 + wr * C::WM + ms * 16 + r16;
      bool ok = row < m_limit;
      if constexpr (V == kContiguous) ok = ok && (p.m_indices[row] >= 0);
      if (!ok) continue;
      uint16_t* drow = D + row * p.ldd;
#pragma unroll
      for (int j = 0; j < C::NS / 2; ++j) {
        const int64_t col = n0 + wc * C::WN + 4 * C::NS * q + 8 * j;
        if (col < p.n) {
          const f32x4 x0 = acc[ms][2 * j];
          const f32x4 x1 = acc[ms][2 * j + 1];
          u32x4 v;
          v.x = pack_bf16x2(x0[0], x0[1]);
          v.y = pack_bf16x2(x0[2], x0[3]);
          v.z = pack_bf16x2(x1[0], x1[1]);
          v.w = pack_bf16x2(x1[2], x1[3]);
          *(u32x4*)(drow + col) = v;
        }
      }
    }
  }
}

using CfgLarge = Cfg<128, 256, 2, 2, 3>;
using CfgMid = Cfg<128, 128, 2, 2, 4>;

template <class C>
hipError_t launch_cfg(Variant v, const GemmParams& p, int grid, hipStream_t stream) {
  dim3 block(C::kThreads);
  switch (v) {
    case kDense: hipLaunchKernelGGL((gemm_kernel<C, kDense>), dim3(grid), block, 0, stream, p); break;
    case kContiguous: hipLaunchKernelGGL((gemm_kernel<C, kContiguous>), dim3(grid), block, 0, stream, p); break;
    case kMasked: hipLaunchKernelGGL((gemm_kernel<C, kMasked>), dim3(grid), block, 0, stream, p); break;
  }
  return hipGetLastError();
}

}  // namespace

InstanceInfo instance_info(GemmInstance inst) {
  switch (inst) {
    case kInstLarge: return {CfgLarge::BM, CfgLarge::BN};
    case kInstMid: return {CfgMid::BM, CfgMid::BN};
    default: return {0, 0};
  }
}

hipError_t launch_gemm(GemmInstance inst, Variant v, const GemmParams& p, int grid, hipStream_t stream) {
  switch (inst) {
    case kInstLarge: return launch_cfg<CfgLarge>(v, p, grid, stream);
    case kInstMid: return launch_cfg<CfgMid>(v, p, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dgfp8
