// Internal declarations shared by the host API and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dgfp8.h"

namespace dgfp8 {

// kDenseSplitK: dense GEMM whose K range is split over several workgroups per
// output tile (small M); partial sums go through a workspace.
// kContiguousSplitK: the contiguous GEMM on the 128-row blocks listed on the
// device (contig_mode 2), with a K split the kernel derives from the number of
// listed blocks (see contig_split_units).
enum Variant : int { kDense = 0, kContiguous = 1, kMasked = 2, kDenseSplitK = 3, kContiguousSplitK = 4 };

// Everything a GEMM launch needs.  Pointers are device addresses; strides are
// in elements (bytes for the E4M3 operands).
struct GemmParams {
  const uint8_t* a;
  int64_t lda, a_gs;              // a_gs: group stride (masked)
  const float* sfa;
  int64_t sfa_sm, sfa_sk, sfa_gs;
  const uint8_t* b;
  int64_t ldb, b_gs;
  const float* sfb;
  int64_t sfb_sn, sfb_sk, sfb_gs;
  uint16_t* d;
  int64_t ldd, d_gs;
  const float* c;                 // dense only: fp32 addend [m, n] (row stride ldc), or null
  int64_t ldc;
  const int32_t* m_indices;       // contiguous
  const int32_t* masked_m;        // masked
  int64_t m;                      // dense: M, contiguous: m_total, masked: max_m
  int64_t n, k;
  int num_groups;
  // split-K only: fp32 partial tiles [tiles][splits][BM*BN] and one arrival
  // counter per output tile (zero on entry, left zero on exit)
  float* ws;
  int* counters;
  int splits;
  int kb_per_split;
  // scale format: 0 = fp32 scales, 1 = packed UE8M0 (int32 words holding the
  // exponents of 4 consecutive K blocks; sfa/sfb then point at those words)
  int sf_packed;
  // contiguous only: 0 = a tile per BM-row block; 1 = 256-row tiles on pairs of
  // consecutive blocks of one group; 2 = 128-row tiles on the blocks no pair
  // covers (tile lists built on the device from m_indices)
  int contig_mode;
  // kContiguousSplitK only: the K split s is the largest with
  // (listed blocks) x (N tiles) x s <= contig_split_units, at most `splits`
  // (and at most the K blocks); the workspace holds contig_split_units partial
  // tiles.  A host constant, so the split never depends on the grid width.
  int contig_split_units;
};

// Largest number of 128-row blocks (m_total / 128) a paired contiguous plan takes.
constexpr int kMaxContigPairBlocks = 2048;

// Kernel instances the host can pick (see gemm_fp8.hip for the tile shapes).
enum GemmInstance : int {
  kInstLarge = 0,     // 128 x 256 output tiles, 8 waves, 3-stage LDS pipeline
  kInstMid = 1,       // 128 x 128 output tiles, 8 waves, 3-stage LDS pipeline
  kInstHuge = 2,      // 256 x 256 output tiles, 8 waves, 2-stage LDS pipeline (dense, masked)
  kInstSkinny128 = 3, // 128 x 64 output tiles, 8 waves, 4-stage LDS pipeline (small M, usually split over K)
  kInstSkinny64 = 4,  // 64 x 64 output tiles, 8 waves, 4-stage LDS pipeline (M <= 64, usually split over K)
  kInstDecode = 5,    // 64 x 256 output tiles, 8 waves side by side, 3-stage LDS pipeline (masked, few rows)
  kInstTall = 6,      // 192 x 256 output tiles, 8 waves, 2-stage LDS pipeline (dense, fills the device where 256x256 does not)
  kNumInstances
};

struct InstanceInfo {
  int bm, bn;
  int occ;   // workgroups resident per CU (persistent grid = CUs * occ)
};
InstanceInfo instance_info(GemmInstance inst);

hipError_t launch_gemm(GemmInstance inst, Variant v, const GemmParams& p, int grid,
                       hipStream_t stream);

struct CastParams {
  const void* x;
  int64_t ldx;
  uint8_t* q;
  int64_t ldq;
  float* sf;
  int64_t sf_s0, sf_s1;           // per-token: (row, kblock); per-block: (nblock, kblock)
  int64_t rows, k;
  int ue8m0;
};

hipError_t launch_per_token_cast(const CastParams& p, bool input_fp32, int num_cus,
                                 hipStream_t stream);
hipError_t launch_per_block_cast(const CastParams& p, hipStream_t stream);

// fp32 scales -> packed UE8M0 words (see dg_pack_ue8m0).
struct PackParams {
  const float* sf;
  int64_t sf_s0, sf_s1;           // element (i, kb) at sf[i * sf_s0 + kb * sf_s1]
  int32_t* out;
  int64_t out_s0, out_s1;         // word (i, w) at out[i * out_s0 + w * out_s1]
  int64_t rows, kblocks;
};
hipError_t launch_pack_ue8m0(const PackParams& p, int num_cus, hipStream_t stream);

}  // namespace dgfp8
