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
//    lane needs one sa value per 16-row sub-tile.  The order in which B rows
//    are placed in LDS ("fragment order") gives each lane 8 consecutive
//    columns per fragment pair, and the 4 lanes of a row adjacent groups of
//    8, so that every epilogue store writes 64 contiguous bytes per row.
//  * Global -> LDS by direct-to-LDS DMA (global_load_lds_dwordx4) into three
//    LDS stages: while K block kb is multiplied, the DMAs of kb+1 and kb+2 are
//    in flight.  The DMAs are waited for explicitly (s_waitcnt vmcnt) and the
//    stage hand-over uses an LDS-only barrier.  Rows are XOR-swizzled in
//    16-byte slots to keep the fragment reads free of bank conflicts.
//  * Persistent grid of one workgroup per CU; the tile index sequence is remapped
//    so that the 32 workgroups of one XCD work on neighbouring tiles (L2 per XCD).
#include "dgfp8_device.h"

namespace dgfp8 {
namespace {

constexpr int kMaxMaskedGroups = 1024;
constexpr int kGroupM = 8;        // raster: tiles of kGroupM consecutive M-tiles sweep N together

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int STAGES_, int BBUF_ = 2, int OCC_ = 1>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int kStages = STAGES_;   // LDS stages; K blocks in flight = kStages - 1
  static constexpr int kBBuf = BBUF_;       // B fragments held in registers (streamed)
  static constexpr int kOcc = OCC_;         // workgroups resident per CU
  static constexpr bool kPackedSf = false;  // scales: fp32 (false) or packed UE8M0 (see SfCfg)
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
  // Scale slots: wave w's DMA fills ls[64w + lane]; lane < kSAPerWave holds the A
  // scale of tile row w*kSAPerWave + lane, the last wave's lanes kSAPerWave + j
  // hold the B scale of 128-column block j.  Other lanes land in unused slots.
  static constexpr int kScaleFloats = 64 * kWaves;
  static constexpr int kMfmas = MS * NS;
  static_assert(kAChunks % kWaves == 0 && kBChunks % kWaves == 0, "chunks per wave");
  static_assert(kSAPerWave + kNSB <= 64, "scale DMA of the last wave");
  static_assert(WN <= 128 && 128 % WN == 0, "a wave's columns lie in one 128-column scale block");
  static_assert(NS % 2 == 0, "epilogue stores 8 columns at a time");
  static_assert(kStages >= 2 && kStages <= 8, "pipeline depth");
  static_assert((kStages - 2) * kLoadsPerStage <= 63, "vmcnt range of the stage wait");
};

// A tile configuration whose scales come as packed UE8M0 exponents: one int32
// holds the 8-bit biased exponents of 4 consecutive K blocks, little-endian
// (page "GitHub 推荐…DeepGEMM…", 可复用的模式与技巧, UE8M0 int32 packing).  An
// exponent byte is exactly the block-scaled MFMA's E8M0 scale operand, so these
// kernels have no mantissa arithmetic at all: no rescale, no epilogue factor.
template <class Base, bool kPacked>
struct SfCfg : Base {
  static constexpr bool kPackedSf = kPacked;
};

// LDS buffers, one array of kStages stages per (config, variant, kind): every
// kernel owns its buffers.  The stage index is a run-time value.
template <class C, int V>
__device__ __forceinline__ DG_LAS uint8_t* lds_a(int stage) {
  __shared__ __attribute__((aligned(1024))) uint8_t buf[C::kStages * C::BM * kKBlock];
  return (DG_LAS uint8_t*)buf + stage * (C::BM * kKBlock);
}
template <class C, int V>
__device__ __forceinline__ DG_LAS uint8_t* lds_b(int stage) {
  __shared__ __attribute__((aligned(1024))) uint8_t buf[C::kStages * C::BN * kKBlock];
  return (DG_LAS uint8_t*)buf + stage * (C::BN * kKBlock);
}
template <class C, int V>
__device__ __forceinline__ DG_LAS float* lds_s(int stage) {
  __shared__ __attribute__((aligned(16))) float buf[C::kStages * C::kScaleFloats];
  return (DG_LAS float*)buf + stage * C::kScaleFloats;
}

// DMA sources of one tile.  Bases are wave-uniform (scalar registers); per-lane
// parts are 32-bit byte offsets, so the loads use the saddr + voffset form.
template <class C>
struct TileSrc {
  const uint8_t* a_base;
  const uint8_t* b_base;
  uint32_t a_off[C::kAChunksPerWave];
  uint32_t b_off[C::kBChunksPerWave];
  const float* s_src;       // this lane's scale word at K block 0 (A row scale or B block scale)
  int64_t s_kstride;
  int kb0;                  // absolute index of the unit's first K block (split-K), for packed scales
};

// DMA instruction d (0 <= d < kLoadsPerStage) of this wave's share of K block kb
// into LDS stage st: A chunks first, then B chunks, then the scales.
template <class C, int V>
__device__ __forceinline__ void issue_dma_part(const TileSrc<C>& t, int kb, int st, int wave, int lane, int d) {
  constexpr int NA = C::kAChunksPerWave, NB = C::kBChunksPerWave;
  (void)lane;
  if (d < NA) {
    dma16(t.a_base + (int64_t)kb * kKBlock, t.a_off[d], lds_addr(lds_a<C, V>(st)) + (wave * NA + d) * 1024);
  } else if (d < NA + NB) {
    const int j = d - NA;
    dma16(t.b_base + (int64_t)kb * kKBlock, t.b_off[j], lds_addr(lds_b<C, V>(st)) + (wave * NB + j) * 1024);
  } else {
    // fp32: one word per K block (s_src already points at the unit's first
    // block); packed: one word per 4 K blocks, indexed by the absolute block.
    const int64_t w = C::kPackedSf ? (int64_t)((t.kb0 + kb) >> 2) : (int64_t)kb;
    dma4(t.s_src + w * t.s_kstride, lds_addr(lds_s<C, V>(st)) + wave * 64 * 4);
  }
}

template <class C, int V>
__device__ __forceinline__ void issue_dma(const TileSrc<C>& t, int kb, int st, int wave, int lane) {
#pragma unroll
  for (int d = 0; d < C::kLoadsPerStage; ++d) issue_dma_part<C, V>(t, kb, st, wave, lane, d);
}


// Scale application.  A row's scale product c = sa * sb for a K block is
// applied as c = 2^e * m, m in [1, 2) carrying the sign.  The block-scaled
// MFMA multiplies the K block's products by 2^e exactly through its E8M0
// operands: the B-row port (one per wave) always gets 2^-63, and the A-row
// port (per lane: lane l supplies row l%16, the row its results belong to)
// gets the biased exponent of q = sa * (sb * 2^63) = c * 2^63, so that
// 2^-63 * 2^(exponent of q) = 2^e.  The accumulator is kept in units of the
// current mantissa m: before a K block's MFMAs it is rescaled by m_prev / m,
// and the epilogue multiplies by the last m.  The MFMA therefore accumulates
// straight into acc, and no VALU instruction waits on an MFMA result inside
// the K loop (with power-of-two scales every ratio is 1).
//   Special values come out of q on their own: a zero scale gives q = 0,
// exponent 0, weight 2^-190, and the block's contribution (below 2^-165)
// rounds away, so it adds exactly nothing, as the definition says.  A
// subnormal scale is applied exactly as long as the product is at least
// 2^-189 (q is then normal).  An infinite or NaN scale, or a product of 2^65
// or more, makes q infinite or NaN, exponent 255, which the MFMA reads as
// NaN.
// Register state of one K block: A fragments, streamed B fragments, scale
// exponents and the accumulator rescale ratios.
template <class C>
struct BlockRegs {
  i32x8 af[C::MS];
  i32x8 bf[C::kBBuf];
  int ea[C::MS];
  int eb;
  float ratio[C::MS];
};

// Raw scales of the K block in stage st that this lane needs: the wave's B
// scale and the A scale of its row in each 16-row sub-tile.
template <class C, int V>
__device__ __forceinline__ void read_scales(float& sb, float (&sa)[C::MS], int st, int wr, int wc, int r16) {
  DG_LAS float* ls = lds_s<C, V>(st);
  sb = ls[(C::kWaves - 1) * 64 + C::kSAPerWave + (wc * C::WN) / 128];
#pragma unroll
  for (int ms = 0; ms < C::MS; ++ms) {
    const int row = wr * C::WM + ms * 16 + r16;
    sa[ms] = ls[(row / C::kSAPerWave) * 64 + row % C::kSAPerWave];
  }
}

// E8M0 exponents and accumulator rescale ratios of a K block from its raw
// scales.  mant: per-row mantissa product the accumulator is expressed in
// (carried across K blocks).
// keep: leave mant unchanged (the block is not used; its registers are).
// kb_abs: absolute K block index (selects the byte of a packed scale word).
template <class C>
__device__ __forceinline__ void scale_math(BlockRegs<C>& r, float (&mant)[C::MS], float sb, const float (&sa)[C::MS],
                                           int kb_abs, bool keep = false) {
  if constexpr (C::kPackedSf) {
    const int sh = (kb_abs & 3) * 8;
    r.eb = (int)((__builtin_bit_cast(uint32_t, sb) >> sh) & 0xFFu);
#pragma unroll
    for (int ms = 0; ms < C::MS; ++ms) r.ea[ms] = (int)((__builtin_bit_cast(uint32_t, sa[ms]) >> sh) & 0xFFu);
    return;
  }
  r.eb = kBRowScaleE8M0;
  const float sb63 = sb * 0x1p63f;   // exact unless sb >= 2^65 (then q is inf or NaN)
#pragma unroll
  for (int ms = 0; ms < C::MS; ++ms) {
    const float q = sa[ms] * sb63;
    r.ea[ms] = scale_exponent(q);
    const float m = scale_mantissa(q);
    r.ratio[ms] = mant[ms] * __builtin_amdgcn_rcpf(m);
    mant[ms] = keep ? mant[ms] : m;
  }
}

// off0/off1: this lane's byte offsets of its two 16-byte slots inside a 16-row
// fragment (the same for A and B fragments).
template <class C, int V>
__device__ __forceinline__ i32x8 read_a(int ms, int st, int wr, uint32_t off0, uint32_t off1) {
  return read_frag(lds_a<C, V>(st) + (wr * C::WM + ms * 16) * kKBlock, off0, off1);
}
template <class C, int V>
__device__ __forceinline__ i32x8 read_b(int t, int st, int wc, uint32_t off0, uint32_t off1) {
  return read_frag(lds_b<C, V>(st) + (wc * C::WN + t * 16) * kKBlock, off0, off1);
}

// All register state of the K block in stage 0 (first block of a tile).
template <class C, int V>
__device__ __forceinline__ void load_block(BlockRegs<C>& r, float (&mant)[C::MS], uint32_t off0, uint32_t off1,
                                           int wr, int wc, int r16, int kb_abs) {
  float sb, sa[C::MS];
  read_scales<C, V>(sb, sa, 0, wr, wc, r16);
#pragma unroll
  for (int ms = 0; ms < C::MS; ++ms) r.af[ms] = read_a<C, V>(ms, 0, wr, off0, off1);
#pragma unroll
  for (int t = 0; t < C::kBBuf - 1; ++t) r.bf[t] = read_b<C, V>(t, 0, wc, off0, off1);
  scale_math(r, mant, sb, sa, kb_abs);
}

// Pipeline of one K block kb (stage S = kb % kStages).  MFMA j: B fragment
// t = j / MS outer, A fragment ms = j % MS inner; B fragment t + kBBuf - 1 is
// read while t is used.  The block's last MS MFMAs (fragment NS - 1) form the
// tail.  After the tail's first MFMA every LDS read of stage S is done, so the
// wave waits for its DMA of kb + 1 and passes the block barrier B(kb+1): every
// wave's DMA of kb + 1 has landed and every wave is done reading stage S.  The
// rest of the tail then reads block kb + 1's scales, first B fragments and A
// fragments into the registers the tail frees (A fragment ms right after its
// last MFMA), and starts the DMA of block kb + kStages into stage S.  That DMA
// is finished in the head of the next step, one instruction per MFMA.  The
// next block's first MFMA therefore finds its operands loaded: the barrier and
// the LDS latency overlap the tail MFMAs.
//
// DMA accounting: block x's DMA (kLoadsPerStage instructions per wave) is
// issued in the tail of step x - kStages and the head of step x - kStages + 1;
// a tile's first kStages - 1 blocks and the tail part of block kStages - 1 come
// from the tile prologue.  At B(y) every block before y + kStages - 1 has been
// fully issued, so kStages - 2 younger blocks may stay in flight.  Past the
// tile's last block the DMA re-loads the last block (a harmless reload into a
// free stage) so that every count stays the same.
template <class C>
struct Pipe {
  static constexpr int kJB = C::kMfmas - C::MS;                     // first tail MFMA
  static constexpr int kTailDma = (C::MS - 1 < C::kLoadsPerStage) ? C::MS - 1 : C::kLoadsPerStage;
  static constexpr int kHeadDma = C::kLoadsPerStage - kTailDma;
  // With two stages the head part must land within this same block: issue it
  // early, one instruction per MFMA; with more stages spread it out.
  static constexpr int kHeadSpan = C::kStages == 2 ? (kHeadDma < kJB + 1 ? kHeadDma : kJB + 1) : kJB + 1;
  static constexpr int kHeadGap = kHeadDma > 0 && kHeadSpan / kHeadDma > 0 ? kHeadSpan / kHeadDma : 1;
  static_assert(C::NS % C::kBBuf == 0, "the tail's B fragment must not share a slot with the prefetched ones");
};

template <class C>
__device__ __forceinline__ void wait_block_dma() {
  __builtin_amdgcn_s_waitcnt(WaitVmLgkm0<(C::kStages - 2) * C::kLoadsPerStage>::value);
}

// One MFMA of the block: acc[ms][t] += 2^(eb + ea[ms]) * (B frag t) x (A frag ms),
// then the accumulator two MFMAs ahead is rescaled to this block's mantissa
// (its 4 multiplies run while this MFMA executes, and that MFMA does not wait
// out the VALU-write -> MFMA-read hazard).
template <class C, int J>
__device__ __forceinline__ void mfma_one(f32x4 (&acc)[C::MS][C::NS], BlockRegs<C>& r) {
  constexpr int t = J / C::MS, ms = J % C::MS;
  // A port <- B rows (n), B port <- A rows (m): result lane l, reg r is
  // D[m = row l%16 of A fragment ms][n = row 4*(l/16)+r of B fragment t].
  acc[ms][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(r.bf[t % C::kBBuf], r.af[ms], acc[ms][t], 0, 0, 0,
                                                                r.eb, 0, r.ea[ms]);
  if constexpr (!C::kPackedSf && J + 2 < C::kMfmas)
    rescale(acc[(J + 2) % C::MS][(J + 2) / C::MS], r.ratio[(J + 2) % C::MS]);
}

// Head of step kb (stage st): MFMAs 0 .. kJB, the head part of block kbd's DMA
// into stage sd, and the streamed B fragment reads.
template <class C, int V>
__device__ __forceinline__ void head(f32x4 (&acc)[C::MS][C::NS], BlockRegs<C>& r, int st, int sd, uint32_t off0,
                                     uint32_t off1, int wc, const TileSrc<C>& tsrc, int kbd, int wave, int lane) {
  using P = Pipe<C>;
  if constexpr (!C::kPackedSf) {
    rescale(acc[0][0], r.ratio[0]);
    if constexpr (C::kMfmas > 1) rescale(acc[1 % C::MS][1 / C::MS], r.ratio[1 % C::MS]);
  }
  static_for<0, P::kJB + 1>([&](auto jc) {
    constexpr int J = decltype(jc)::value;
    __builtin_amdgcn_sched_barrier(0);
    mfma_one<C, J>(acc, r);
    constexpr int t = J / C::MS, ms = J % C::MS, tn = t + C::kBBuf - 1;
    if constexpr (ms == 0 && tn < C::NS) r.bf[tn % C::kBBuf] = read_b<C, V>(tn, st, wc, off0, off1);
    if constexpr (J % P::kHeadGap == 0 && J / P::kHeadGap < P::kHeadDma)
      issue_dma_part<C, V>(tsrc, kbd, sd, wave, lane, P::kTailDma + J / P::kHeadGap);
  });
  __builtin_amdgcn_sched_barrier(0);
  if constexpr ((P::kJB + 1 + P::kHeadGap - 1) / P::kHeadGap < P::kHeadDma) {
#pragma unroll
    for (int d = (P::kJB + 1 + P::kHeadGap - 1) / P::kHeadGap; d < P::kHeadDma; ++d)
      issue_dma_part<C, V>(tsrc, kbd, sd, wave, lane, P::kTailDma + d);
  }
}

// Tail of step kb (next block's stage SN): barrier B(kb+1), prefetch of block
// kb+1 into the freed registers, tail part of block kbd's DMA into S.  The
// tile's last block runs the same code (no branch in the pipeline: it would
// cost the in-place accumulation its registers); its "next block" is whatever
// stage SN holds, and last leaves the mantissa state alone.
template <class C, int V>
__device__ __forceinline__ void tail(f32x4 (&acc)[C::MS][C::NS], float (&mant)[C::MS], BlockRegs<C>& r, int st,
                                     int sn, uint32_t off0, uint32_t off1, int wr, int wc, int r16,
                                     const TileSrc<C>& tsrc, int kbd, int wave, int lane, bool last, int kb_next) {
  using P = Pipe<C>;
  wait_block_dma<C>();
  lds_barrier();
  float sb, sa[C::MS];
  read_scales<C, V>(sb, sa, sn, wr, wc, r16);
#pragma unroll
  for (int t = 0; t < C::kBBuf - 1; ++t) r.bf[t] = read_b<C, V>(t, sn, wc, off0, off1);
  r.af[0] = read_a<C, V>(0, sn, wr, off0, off1);
  static_for<0, C::MS - 1>([&](auto uc) {
    constexpr int U = decltype(uc)::value;
    __builtin_amdgcn_sched_barrier(0);
    mfma_one<C, P::kJB + 1 + U>(acc, r);
    r.af[U + 1] = read_a<C, V>(U + 1, sn, wr, off0, off1);
    if constexpr (U < P::kTailDma) issue_dma_part<C, V>(tsrc, kbd, st, wave, lane, U);
  });
  __builtin_amdgcn_sched_barrier(0);
  scale_math(r, mant, sb, sa, tsrc.kb0 + kb_next, last);
}

// One K block kb in stage st = kb % kStages (see Pipe).
template <class C, int V>
__device__ __forceinline__ void step(const TileSrc<C>& t, f32x4 (&acc)[C::MS][C::NS], float (&mant)[C::MS],
                                     BlockRegs<C>& r, int kb, int st, int kblocks, int wave, int lane, uint32_t off0,
                                     uint32_t off1, int wr, int wc, int r16) {
  const int sn = st + 1 == C::kStages ? 0 : st + 1;   // stage of kb + 1
  const int sp = st == 0 ? C::kStages - 1 : st - 1;   // stage of kb - 1 (freed at B(kb))
  const int kbh = kb + C::kStages - 1;                 // block whose DMA head part goes into sp
  head<C, V>(acc, r, st, sp, off0, off1, wc, t, kbh < kblocks ? kbh : kblocks - 1, wave, lane);
  const int kbt = kb + C::kStages;                     // block whose DMA tail part goes into st
  tail<C, V>(acc, mant, r, st, sn, off0, off1, wr, wc, r16, t, kbt < kblocks ? kbt : kblocks - 1, wave, lane,
             kb + 1 >= kblocks, kb + 1);
}

// Step of a wave none of whose rows is written (rows past M, contiguous
// padding, masked rows past masked_m): it issues its share of the tile's DMA
// and passes the block barrier at the same points as step(), nothing else.
template <class C, int V>
__device__ __forceinline__ void idle_step(const TileSrc<C>& t, int kb, int st, int kblocks, int wave, int lane) {
  using P = Pipe<C>;
  const int sp = st == 0 ? C::kStages - 1 : st - 1;
  const int kbh = kb + C::kStages - 1;
#pragma unroll
  for (int d = 0; d < P::kHeadDma; ++d)
    issue_dma_part<C, V>(t, kbh < kblocks ? kbh : kblocks - 1, sp, wave, lane, P::kTailDma + d);
  wait_block_dma<C>();
  lds_barrier();
  const int kbt = kb + C::kStages;
#pragma unroll
  for (int d = 0; d < P::kTailDma; ++d) issue_dma_part<C, V>(t, kbt < kblocks ? kbt : kblocks - 1, st, wave, lane, d);
}

// Tile prologue DMA (all stages free): blocks 0 .. kStages-2 in full and the
// tail part of block kStages-1.
template <class C, int V>
__device__ __forceinline__ void tile_dma(const TileSrc<C>& t, int kblocks, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < C::kStages - 1; ++i) issue_dma<C, V>(t, i < kblocks ? i : kblocks - 1, i, wave, lane);
  constexpr int kL = C::kStages - 1;
#pragma unroll
  for (int d = 0; d < Pipe<C>::kTailDma; ++d)
    issue_dma_part<C, V>(t, kL < kblocks ? kL : kblocks - 1, kL, wave, lane, d);
}

// B(0).  Only younger instructions than block 0's DMA may remain in flight:
// the rest of the prologue DMA, and possibly stores of the previous tile
// (issued after it; waiting for some of them is harmless).
template <class C>
__device__ __forceinline__ void tile_wait() {
  __builtin_amdgcn_s_waitcnt(WaitVmLgkm0<(C::kStages - 2) * C::kLoadsPerStage + Pipe<C>::kTailDma>::value);
  lds_barrier();
}

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

// Contiguous layout, device-side tile list (one wave; graph-safe, the host never
// reads m_indices).  A 128-row block belongs to the group m_indices holds at
// its first row (-1: padding, no tile).  Consecutive blocks of one group form a
// segment; from each segment's start, blocks are taken in pairs (a 256-row
// tile) and an odd segment ends in a single block.  mode 1 lists the first
// block of every pair, mode 2 every single block; the two launches of a plan
// together cover every non-padding block exactly once.  Each lane walks 32
// consecutive blocks; a max-scan over lanes hands each lane the start of the
// segment its first block belongs to.
constexpr int kMaxContigBlocks = kMaxContigPairBlocks;

__device__ void contig_tile_list(const GemmParams& p, int lane, DG_LAS int16_t* list, DG_LAS int* count) {
  constexpr int kPer = kMaxContigBlocks / 64;
  const int nb = (int)(p.m / kKBlock);
  const int b0 = lane * kPer;
  auto group_of = [&](int b) -> int { return b >= 0 && b < nb ? p.m_indices[(int64_t)b * kKBlock] : -1; };
  int g[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) g[i] = group_of(b0 + i);
  const int gprev = group_of(b0 - 1), gnext = group_of(b0 + kPer);
  int last = -1;   // last segment start in this lane's blocks
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int prev = i ? g[i - 1] : gprev;
    if (g[i] >= 0 && g[i] != prev) last = b0 + i;
  }
  int incl = last;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off, 64);
    if (lane >= off) incl = max(incl, v);
  }
  int start = __shfl_up(incl, 1, 64);
  if (lane == 0) start = -1;
  uint32_t pick = 0;
  int n = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int b = b0 + i;
    const int prev = i ? g[i - 1] : gprev;
    if (g[i] < 0) continue;
    if (g[i] != prev) start = b;
    if (((b - start) & 1) == 0) {
      const bool pair = (i + 1 < kPer ? g[i + 1] : gnext) == g[i];
      if (pair == (p.contig_mode == 1)) {
        pick |= 1u << i;
        ++n;
      }
    }
  }
  int run = n;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(run, off, 64);
    if (lane >= off) run += v;
  }
  int pos = run - n;
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    if ((pick >> i) & 1u) list[pos++] = (int16_t)(b0 + i);
  if (lane == 63) *count = run;
}

template <class C, int V>
__global__ void __launch_bounds__(C::kThreads)
__attribute__((amdgpu_waves_per_eu(C::kWaves * C::kOcc / 4, C::kWaves * C::kOcc / 4)))
gemm_kernel(GemmParams p) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wr = wave / C::WAVES_N;
  const int wc = wave % C::WAVES_N;
  const int r16 = lane & 15;
  const int q = lane >> 4;
  const int kblocks = (int)(p.k / kKBlock);
  const int tiles_n = (int)((p.n + C::BN - 1) / C::BN);
  const int64_t n_sblocks = (p.n + 127) / 128;
  // This lane's two 16-byte slots (logical slots 2q, 2q+1) inside any 16-row fragment.
  const uint32_t off0 = r16 * kKBlock + (((2 * q) ^ swz16(r16)) << 4);
  const uint32_t off1 = r16 * kKBlock + (((2 * q + 1) ^ swz16(r16)) << 4);

  // ---- tile space
  constexpr bool kSplit = V == kDenseSplitK || V == kContiguousSplitK;
  constexpr bool kContig = V == kContiguous || V == kContiguousSplitK;
  __shared__ int masked_prefix[V == kMasked ? kMaxMaskedGroups + 1 : 1];
  int tiles_m = 0, num_tiles = 0;
  // K split of a split variant: units (tile, split) with kb_per_split K blocks each
  int splits = kSplit ? p.splits : 1;
  int kb_per_split = p.kb_per_split;
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
    num_tiles = tiles_m * tiles_n * splits;
  }
  __shared__ int16_t contig_list[kContig ? kMaxContigBlocks : 1];
  __shared__ int contig_count;
  if constexpr (kContig) {
    if (p.contig_mode != 0) {
      if (wave == 0) contig_tile_list(p, lane, (DG_LAS int16_t*)contig_list, (DG_LAS int*)&contig_count);
      __syncthreads();
      tiles_m = contig_count;
      if constexpr (V == kContiguousSplitK) {
        // As many splits as keep the units within contig_split_units (every
        // workgroup computes the same value from the same list).
        const int tiles = tiles_m * tiles_n;
        int s = tiles > 0 ? p.contig_split_units / tiles : 1;
        s = s < p.splits ? s : p.splits;
        s = s < kblocks ? s : kblocks;
        s = s > 1 ? s : 1;
        kb_per_split = (kblocks + s - 1) / s;
        splits = (kblocks + kb_per_split - 1) / kb_per_split;
      }
      num_tiles = tiles_m * tiles_n * splits;
    }
  }

  // Tile state: position, group, K blocks and DMA sources.  okmask bit ms:
  // this lane's row of sub-tile ms is written.  The epilogue's global loads
  // (m_indices, masked_m) are done and consumed here, before the next tile's
  // DMAs are issued: the compiler does not know of those DMAs, and a wait for
  // a load placed after them would wait for them too.
  struct Tile {
    int mt, nt, g, split, kbs;
    int m0;                 // first row of the tile (per group when masked)
    uint32_t okmask;
    TileSrc<C> src;
  };
  auto decode = [&](int tile, Tile& s) -> bool {
      int mt, nt, g = 0, split = 0;
      int64_t m_limit = p.m;   // rows that may be written
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
      } else if constexpr (kSplit) {
        // consecutive units are the splits of one output tile: they run together
        split = tile % splits;
        raster(tile / splits, tiles_m, tiles_n, mt, nt);
      } else {
        raster(tile, tiles_m, tiles_n, mt, nt);
      }
      int64_t m0 = (int64_t)mt * C::BM;
      if constexpr (kContig) {
        if (p.contig_mode != 0) m0 = (int64_t)contig_list[mt] * kKBlock;   // listed block
        g = p.m_indices[m0];
        if (g < 0) return false;                // whole block is padding
      }
      const int64_t n0 = (int64_t)nt * C::BN;
      const int64_t a_rows = p.m;   // rows of A present in memory (per group when masked)

      // Per-lane index math of this tile is done on a copy of the lane id that the
      // compiler cannot see through, so that it is recomputed per tile instead of
      // being hoisted out of the tile loop and kept live (or spilled) for the
      // whole kernel.
      int tl = lane;
      asm volatile("" : "+v"(tl));

      // ---- DMA sources: uniform bases, per-lane 32-bit offsets (host checks they fit)
      TileSrc<C>& t = s.src;
      t.kb0 = 0;
      t.a_base = p.a + (V == kMasked ? (int64_t)g * p.a_gs : 0);
      t.b_base = p.b + (V != kDense ? (int64_t)g * p.b_gs : 0);
#pragma unroll
      for (int j = 0; j < C::kAChunksPerWave; ++j) {
        const int prow = (wave * C::kAChunksPerWave + j) * 8 + (tl >> 3);
        int64_t row = m0 + prow;
        row = row < a_rows ? row : a_rows - 1;
        t.a_off[j] = (uint32_t)(row * p.lda) + (((tl & 7) ^ swz16(prow)) << 4);
      }
#pragma unroll
      for (int j = 0; j < C::kBChunksPerWave; ++j) {
        // LDS row prow of the B stage holds, in fragment order, column
        // n0 + wcol*WN + 32*(ft/2) + 8*(fi/4) + 4*(ft%2) + fi%4 (ft = fragment,
        // fi = row in it).  Result lane group q = fi/4 then holds, from the
        // fragment pair (2j, 2j+1), the 8 columns 32j + 8q .. 32j + 8q + 7: one
        // store instruction writes 64 contiguous bytes of each of 16 rows.
        const int prow = (wave * C::kBChunksPerWave + j) * 8 + (tl >> 3);
        const int wcol = prow / C::WN;
        const int pl = prow % C::WN;
        const int ft = pl / 16, fi = pl % 16;
        int64_t col = n0 + wcol * C::WN + 32 * (ft / 2) + 8 * (fi / 4) + 4 * (ft % 2) + (fi % 4);
        col = col < p.n ? col : p.n - 1;
        t.b_off[j] = (uint32_t)(col * p.ldb) + (((tl & 7) ^ swz16(prow)) << 4);
      }
      {
        const float* SFA = p.sfa + (V == kMasked ? (int64_t)g * p.sfa_gs : 0);
        const float* SFB = p.sfb + (V != kDense ? (int64_t)g * p.sfb_gs : 0);
        // Every lane points at a valid scale (the DMA is unconditional; see
        // kScaleFloats).  Lanes whose slot is not used repeat the address of the
        // wave's first A row, so that the load touches no cache line beyond those
        // holding the scales the tile needs.
        const int j = tl - C::kSAPerWave;
        if (wave == C::kWaves - 1 && j >= 0 && j < C::kNSB) {
          int64_t nb = n0 / 128 + j;
          nb = nb < n_sblocks ? nb : n_sblocks - 1;
          t.s_src = SFB + nb * p.sfb_sn;
          t.s_kstride = p.sfb_sk;
        } else {
          int64_t row = m0 + wave * C::kSAPerWave + (tl < C::kSAPerWave ? tl : 0);
          row = row < a_rows ? row : a_rows - 1;
          t.s_src = SFA + row * p.sfa_sm;
          t.s_kstride = p.sfa_sk;
        }
      }

      int kbs = kblocks;   // K blocks of this unit
      if constexpr (kSplit) {
        const int kb0 = split * kb_per_split;
        kbs = min(kb_per_split, kblocks - kb0);
        t.a_base += (int64_t)kb0 * kKBlock;
        t.b_base += (int64_t)kb0 * kKBlock;
        if constexpr (!C::kPackedSf) t.s_src += (int64_t)kb0 * t.s_kstride;
        t.kb0 = kb0;
      }
    // All of these are wave-uniform; say so, so that they stay in scalar
    // registers across the tile loop.
    t.a_base = uniform_ptr(t.a_base);
    t.b_base = uniform_ptr(t.b_base);
    s.mt = __builtin_amdgcn_readfirstlane(mt);
    s.m0 = __builtin_amdgcn_readfirstlane((int)m0);
    s.nt = __builtin_amdgcn_readfirstlane(nt);
    s.g = __builtin_amdgcn_readfirstlane(g);
    s.split = __builtin_amdgcn_readfirstlane(split);
    s.kbs = __builtin_amdgcn_readfirstlane(kbs);
    uint32_t okm = 0;
#pragma unroll
    for (int ms = 0; ms < C::MS; ++ms) {
      const int64_t row = m0 + wr * C::WM + ms * 16 + (tl & 15);
      bool ok = row < m_limit;
      if constexpr (kContig) ok = ok && (p.m_indices[row] >= 0);
      okm |= (ok ? 1u : 0u) << ms;
    }
    s.okmask = okm;
    return true;
  };
  // First tile at or after `tile` (stride gridDim.x) that is not skipped.
  auto next_tile = [&](int tile, Tile& s) -> int {
    for (; tile < num_tiles; tile += gridDim.x)
      if (decode(tile, s)) break;
    return tile;
  };
  auto prologue = [&](const Tile& s) { tile_dma<C, V>(s.src, s.kbs, wave, lane); };

  // bf16 RNE, 16-byte stores of 8 consecutive columns; dense variants add the
  // optional fp32 addend C first (D = C + A.B^T, rounded once).
  auto store_tile = [&](const Tile& s, f32x4 (&acc)[C::MS][C::NS]) {
    uint16_t* D = p.d + (V == kMasked ? (int64_t)s.g * p.d_gs : 0);
    const int er16 = lane & 15, eq = lane >> 4;
    const int64_t m0 = s.m0, n0 = (int64_t)s.nt * C::BN;
#pragma unroll
    for (int ms = 0; ms < C::MS; ++ms) {
      if (!((s.okmask >> ms) & 1u)) continue;
      uint16_t* drow = D + (m0 + wr * C::WM + ms * 16 + er16) * p.ldd;
#pragma unroll
      for (int j = 0; j < C::NS / 2; ++j) {
        const int64_t col = n0 + wc * C::WN + 32 * j + 8 * eq;
        if (col < p.n) {
          f32x4 x0 = acc[ms][2 * j];
          f32x4 x1 = acc[ms][2 * j + 1];
          if constexpr (V == kDense || V == kDenseSplitK) {
            if (p.c) {
              const float* crow = p.c + (m0 + wr * C::WM + ms * 16 + er16) * p.ldc + col;
              x0 += *(const f32x4*)crow;
              x1 += *(const f32x4*)(crow + 4);
            }
          }
          u32x4 v;
          v.x = pack_bf16x2(x0[0], x0[1]);
          v.y = pack_bf16x2(x0[2], x0[3]);
          v.z = pack_bf16x2(x1[0], x1[1]);
          v.w = pack_bf16x2(x1[2], x1[3]);
          *(u32x4*)(drow + col) = v;
        }
      }
    }
  };
  // First tile of round r (tiles r*grid .. r*grid + grid - 1).  A round that
  // the dense tiles fill only in part is spread evenly over the 8 XCDs (each
  // takes a contiguous run of about a eighth of it) instead of filling the
  // first XCDs and leaving the others idle; the full rounds keep the
  // contiguous per-XCD runs of remap_for_xcd.  Only the tile-to-workgroup map
  // changes: every tile is still run once, by one workgroup.
  auto round_start = [&](int r) -> int {
    const int grid = (int)gridDim.x, t0 = r * grid;
    if (V == kDense && grid % 8 == 0 && t0 < num_tiles && num_tiles - t0 < grid) {
      const int rem = num_tiles - t0, q = rem >> 3, extra = rem & 7;
      const int x = (int)blockIdx.x & 7, j = (int)blockIdx.x >> 3;
      const int cnt = q + (x < extra ? 1 : 0);
      return j < cnt ? t0 + x * q + min(x, extra) + j : num_tiles;
    }
    return t0 < num_tiles ? t0 + remap_for_xcd((int)blockIdx.x, grid) : num_tiles;
  };
  int rnd = 0;
  Tile cur;
  int tile = next_tile(round_start(0), cur);
  if (tile < num_tiles) prologue(cur);
  while (tile < num_tiles) {
    f32x4 acc[C::MS][C::NS];
    float mant[C::MS];
#pragma unroll
    for (int i = 0; i < C::MS; ++i) {
      mant[i] = 1.0f;
#pragma unroll
      for (int j = 0; j < C::NS; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }

    // ---- main loop over K blocks, LDS stage = kb % kStages.  A wave none of
    // whose rows is written only keeps the DMA and barrier schedule.
    tile_wait<C>();
    int st = 0;
    if (__builtin_amdgcn_ballot_w64(cur.okmask != 0) != 0) {
      BlockRegs<C> r;
      load_block<C, V>(r, mant, off0, off1, wr, wc, r16, cur.src.kb0);
#pragma nounroll
      for (int kb = 0; kb < cur.kbs; ++kb) {
        step<C, V>(cur.src, acc, mant, r, kb, st, cur.kbs, wave, lane, off0, off1, wr, wc, r16);
        st = st + 1 == C::kStages ? 0 : st + 1;
      }
    } else {
#pragma nounroll
      for (int kb = 0; kb < cur.kbs; ++kb) {
        idle_step<C, V>(cur.src, kb, st, cur.kbs, wave, lane);
        st = st + 1 == C::kStages ? 0 : st + 1;
      }
    }

    // ---- epilogue: back from mantissa units
    if constexpr (!C::kPackedSf) {
#pragma unroll
      for (int ms = 0; ms < C::MS; ++ms)
#pragma unroll
        for (int j = 0; j < C::NS; ++j) acc[ms][j] *= mant[ms];
    }
    Tile nxt;
    const int ntile = next_tile(V == kDense ? round_start(++rnd) : tile + (int)gridDim.x, nxt);
    if (kSplit && splits > 1) {
      // Publish this unit's partial tile, count arrivals; the last unit of the
      // output tile adds all partials in split order (deterministic whatever the
      // arrival order) and writes D.  Partials are kept in register order, not
      // as a matrix: the 4 floats of acc[ms][j] of lane l of wave w sit at float
      // ((w * MS * NS + ms * NS + j) * 64 + l) * 4 of the split's region, so that
      // each 16-byte store or load instruction covers 1 KB contiguous.  The
      // units of one tile may run on different XCDs, whose L2 caches are not
      // coherent with each other for plain accesses: the partials move with
      // device-scope (sc1) buffer accesses, written through to and read from the
      // device-coherent level, which avoids the L2-wide writeback and invalidate
      // that a device-scope fence costs.  The buffer's size bounds every access.
      const int tile_mn = cur.mt * tiles_n + cur.nt;
      constexpr int kTileFloats = C::BM * C::BN;
      const __amdgpu_buffer_rsrc_t part = __builtin_amdgcn_make_buffer_rsrc(
          p.ws + (int64_t)tile_mn * splits * kTileFloats, 0, splits * kTileFloats * 4, kRawBufferFlags);
      const int lane_off = ((wave * C::kMfmas) * 64 + lane) * 16;   // bytes, (ms, j) = (0, 0)
#pragma unroll
      for (int ms = 0; ms < C::MS; ++ms)
#pragma unroll
        for (int j = 0; j < C::NS; ++j)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[ms][j]), part,
                                                 lane_off + (ms * C::NS + j) * 1024,
                                                 cur.split * kTileFloats * 4, kScopeDevice);
      // every partial store has been acknowledged before the arrival is counted
      __builtin_amdgcn_s_waitcnt(WaitVmLgkm0<0>::value);
      __shared__ int last_flag;
      __syncthreads();
      if (threadIdx.x == 0)
        last_flag = __hip_atomic_fetch_add(p.counters + tile_mn, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                    splits - 1;
      __syncthreads();
      if (last_flag) {
#pragma unroll
        for (int ms = 0; ms < C::MS; ++ms)
#pragma unroll
          for (int j = 0; j < C::NS; ++j) acc[ms][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
        // Splits in batches: every load of a batch is issued before the first
        // add, so one memory round trip serves the whole batch; the adds then
        // run in split order.
        constexpr int kBatch = 32 / (C::kMfmas * 4) > 0 ? 32 / (C::kMfmas * 4) : 1;
        for (int sp0 = 0; sp0 < splits; sp0 += kBatch) {
          f32x4 v[kBatch][C::MS][C::NS];
#pragma unroll
          for (int b = 0; b < kBatch; ++b)
#pragma unroll
            for (int ms = 0; ms < C::MS; ++ms)
#pragma unroll
              for (int j = 0; j < C::NS; ++j)
                v[b][ms][j] = sp0 + b < splits
                                  ? __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                                  part, lane_off + (ms * C::NS + j) * 1024,
                                                                  (sp0 + b) * kTileFloats * 4, kScopeDevice))
                                  : (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int b = 0; b < kBatch; ++b)
#pragma unroll
            for (int ms = 0; ms < C::MS; ++ms)
#pragma unroll
              for (int j = 0; j < C::NS; ++j)
                if (sp0 + b < splits) acc[ms][j] += v[b][ms][j];
        }
        // ready for the next call
        if (threadIdx.x == 0) __hip_atomic_store(p.counters + tile_mn, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        store_tile(cur, acc);
      }
      // every wave is done with this unit's LDS stages and its DMAs have landed
      __builtin_amdgcn_s_waitcnt(WaitVmLgkm0<0>::value);
      lds_barrier();
      if (ntile < num_tiles) prologue(nxt);
    } else {
      // Every wave is done reading this tile's LDS stages, and the DMAs its
      // last steps re-issued into them have landed (only those are
      // outstanding here): issue the next tile's first DMAs, then convert and
      // store this tile while they are in flight.
      __builtin_amdgcn_s_waitcnt(WaitVmLgkm0<0>::value);
      lds_barrier();
      if ((V == kDense || V == kDenseSplitK) && p.c) {
        // The addend's loads must come before the next tile's DMAs: a wait for
        // them placed after those DMAs would wait for the DMAs too.
        store_tile(cur, acc);
        if (ntile < num_tiles) prologue(nxt);
      } else {
        if (ntile < num_tiles) prologue(nxt);
        store_tile(cur, acc);
      }
    }
    cur = nxt;
    tile = ntile;
  }
  // Tail steps re-issue the last K block's DMA into free stages: let them land
  // before this workgroup's LDS can be handed to another one.
  __builtin_amdgcn_s_waitcnt(WaitVmLgkm0<0>::value);
}

using CfgHuge = Cfg<256, 256, 4, 2, 2, 2>;
using CfgSkinny128 = Cfg<128, 64, 4, 2, 4>;
using CfgSkinny64 = Cfg<64, 64, 4, 2, 4>;
using CfgLarge = Cfg<128, 256, 2, 4, 3>;
using CfgMid = Cfg<128, 128, 2, 4, 3>;
// Masked decode (few rows per group): one 64-row wave band across 256 columns.
using CfgDecode = Cfg<64, 256, 1, 8, 3>;
// Three quarters of the 256x256 tile (48-row wave bands): more tiles where the
// 256x256 grid leaves CUs idle (N = 2112: 198 tiles instead of 144 at M = 4096).
using CfgTall = Cfg<192, 256, 4, 2, 2>;

// Variants compiled per configuration: bit v of Mask set = variant v available.
template <class C, int Mask>
hipError_t launch_variant(Variant v, const GemmParams& p, int grid, hipStream_t stream) {
  dim3 block(C::kThreads);
  if (!((Mask >> v) & 1)) return hipErrorInvalidValue;
  switch (v) {
    case kDense:
      if constexpr ((Mask >> kDense) & 1) hipLaunchKernelGGL((gemm_kernel<C, kDense>), dim3(grid), block, 0, stream, p);
      break;
    case kContiguous:
      if constexpr ((Mask >> kContiguous) & 1)
        hipLaunchKernelGGL((gemm_kernel<C, kContiguous>), dim3(grid), block, 0, stream, p);
      break;
    case kMasked:
      if constexpr ((Mask >> kMasked) & 1) hipLaunchKernelGGL((gemm_kernel<C, kMasked>), dim3(grid), block, 0, stream, p);
      break;
    case kDenseSplitK:
      if constexpr ((Mask >> kDenseSplitK) & 1)
        hipLaunchKernelGGL((gemm_kernel<C, kDenseSplitK>), dim3(grid), block, 0, stream, p);
      break;
    case kContiguousSplitK:
      if constexpr ((Mask >> kContiguousSplitK) & 1)
        hipLaunchKernelGGL((gemm_kernel<C, kContiguousSplitK>), dim3(grid), block, 0, stream, p);
      break;
  }
  return hipGetLastError();
}

template <class C, int Mask>
hipError_t launch_cfg(Variant v, const GemmParams& p, int grid, hipStream_t stream) {
  return p.sf_packed ? launch_variant<SfCfg<C, true>, Mask>(v, p, grid, stream)
                     : launch_variant<C, Mask>(v, p, grid, stream);
}

constexpr int kAll = (1 << kDense) | (1 << kContiguous) | (1 << kMasked) | (1 << kDenseSplitK) |
                     (1 << kContiguousSplitK);
constexpr int kDenseAndSplit = (1 << kDense) | (1 << kDenseSplitK);

}  // namespace

InstanceInfo instance_info(GemmInstance inst) {
  switch (inst) {
    case kInstHuge: return {CfgHuge::BM, CfgHuge::BN, CfgHuge::kOcc};
    case kInstSkinny128: return {CfgSkinny128::BM, CfgSkinny128::BN, CfgSkinny128::kOcc};
    case kInstSkinny64: return {CfgSkinny64::BM, CfgSkinny64::BN, CfgSkinny64::kOcc};
    case kInstLarge: return {CfgLarge::BM, CfgLarge::BN, CfgLarge::kOcc};
    case kInstMid: return {CfgMid::BM, CfgMid::BN, CfgMid::kOcc};
    case kInstDecode: return {CfgDecode::BM, CfgDecode::BN, CfgDecode::kOcc};
    case kInstTall: return {CfgTall::BM, CfgTall::BN, CfgTall::kOcc};
    default: return {0, 0, 0};
  }
}

hipError_t launch_gemm(GemmInstance inst, Variant v, const GemmParams& p, int grid, hipStream_t stream) {
  switch (inst) {
    case kInstHuge: return launch_cfg<CfgHuge, (1 << kDense) | (1 << kMasked) | (1 << kContiguous)>(v, p, grid, stream);
    case kInstSkinny128: return launch_cfg<CfgSkinny128, kDenseAndSplit>(v, p, grid, stream);
    case kInstSkinny64: return launch_cfg<CfgSkinny64, kDenseAndSplit>(v, p, grid, stream);
    case kInstLarge: return launch_cfg<CfgLarge, kAll>(v, p, grid, stream);
    case kInstMid: return launch_cfg<CfgMid, kAll>(v, p, grid, stream);
    case kInstDecode: return launch_cfg<CfgDecode, (1 << kMasked)>(v, p, grid, stream);
    case kInstTall: return launch_cfg<CfgTall, (1 << kDense)>(v, p, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dgfp8
