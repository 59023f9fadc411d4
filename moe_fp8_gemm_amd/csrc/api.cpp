// Host side of the C ABI: argument validation (the caller's faults come back as
// status codes, in the spirit of the host assertions the pages describe: page
// "GitHub 推荐…DeepGEMM…", 解法哲学 and 可复用的模式与技巧 on layout validation),
// choice of a compiled kernel instance, and launch on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstdint>
#include <initializer_list>

#include "dgfp8_internal.h"

#define DG_EXPORT extern "C" __attribute__((visibility("default")))

namespace dgfp8 {
namespace {

constexpr int kContiguousAlignment = 128;
constexpr int kMaxMaskedGroups = 1024;
constexpr int kMaxDevices = 64;

int g_num_cus_override = 0;
int g_contig_plan = 0;   // 0: cost model, 1: paired plan, 2: one tile per 128-row block
int g_dense_inst = -1;   // forced dense instance (-1: cost model) and its K splits
int g_dense_splits = 1;
int g_device_cus[kMaxDevices] = {0};

// Compute units of the current device (ignores the override).
int hw_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  if (g_device_cus[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    g_device_cus[dev] = v;
  }
  return g_device_cus[dev];
}

// Width of the persistent grid.
int device_cus() { return g_num_cus_override > 0 ? g_num_cus_override : hw_cus(); }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Strides (elements) and sizes no real buffer comes near: 2^40.  Rejecting
// larger ones keeps every product of two of them inside int64 (in this file
// and in the kernels' 64-bit offset arithmetic).
constexpr int64_t kMaxStride = (int64_t)1 << 40;
bool strides_ok(std::initializer_list<int64_t> v) {
  for (int64_t x : v)
    if (x > kMaxStride) return false;
  return true;
}

// Checks shared by the three GEMM variants.
dg_status check_common(const void* a, int64_t lda, const void* sfa, int64_t sfa_sm, int64_t sfa_sk,
                       const void* b, int64_t ldb, const void* sfb, int64_t sfb_sn, int64_t sfb_sk,
                       const void* d, int64_t ldd, int64_t n, int64_t k) {
  if (!a || !b || !d || !sfa || !sfb) return DG_ERROR_INVALID_VALUE;
  if (n < 0 || k < 0) return DG_ERROR_INVALID_VALUE;
  if (sfa_sm < 0 || sfa_sk < 0 || sfb_sn < 0 || sfb_sk < 0) return DG_ERROR_INVALID_VALUE;
  if (lda < k || ldb < k || ldd < n) return DG_ERROR_INVALID_VALUE;
  if (!strides_ok({lda, ldb, ldd, sfa_sm, sfa_sk, sfb_sn, sfb_sk, n, k})) return DG_ERROR_NOT_SUPPORTED;
  if (k == 0 || k % 128 != 0) return DG_ERROR_NOT_SUPPORTED;
  if (n % 8 != 0 || ldd % 8 != 0) return DG_ERROR_NOT_SUPPORTED;
  if (lda % 16 != 0 || ldb % 16 != 0) return DG_ERROR_NOT_SUPPORTED;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(d, 16)) return DG_ERROR_NOT_SUPPORTED;
  if (!aligned(sfa, 4) || !aligned(sfb, 4)) return DG_ERROR_NOT_SUPPORTED;
  return DG_SUCCESS;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Static instance choice: estimated time = rounds of persistent tiles x tile
// area x a per-instance cost factor (relative cycles per output element,
// measured on MI355X: bigger tiles move fewer bytes through L2 and LDS per FLOP).
double area_factor(GemmInstance inst) {
  return inst == kInstHuge ? 1.0 : inst == kInstTall ? 1.13 : inst == kInstLarge ? 1.2 : 1.5;
}

double instance_cost(GemmInstance inst, int64_t m_rows, int64_t groups_m_tiles_hint, int64_t n, int cus) {
  const InstanceInfo info = instance_info(inst);
  const int64_t tiles = (groups_m_tiles_hint > 0 ? groups_m_tiles_hint : ceil_div(m_rows, info.bm)) *
                        ceil_div(n, info.bn);
  const int64_t rounds = ceil_div(tiles, cus);
  return (double)rounds * info.bm * info.bn * area_factor(inst);
}

GemmInstance choose_dense(int64_t m, int64_t n, int cus) {
  GemmInstance best = kInstMid;
  double best_cost = instance_cost(kInstMid, m, 0, n, cus);
  for (GemmInstance inst : {kInstLarge, kInstHuge, kInstTall}) {
    const double c = instance_cost(inst, m, 0, n, cus);
    if (c < best_cost) { best = inst; best_cost = c; }
  }
  return best;
}

// ---- split-K for small M (too few output tiles to keep the CUs streaming B)
//
// Workspace layout (caller-owned): a fixed block of kSplitCounters int32
// arrival counters (one per output tile; zero before first use, left zero by
// every completed call), then the fp32 partial tiles [tiles][splits][BM*BN].
// The counter block never moves, so one workspace serves problems of any shape.

constexpr int kSplitCounters = 1 << 16;
constexpr int64_t kSplitCounterBytes = kSplitCounters * 4;     // 256 KiB
constexpr int64_t kMaxSplitPartialBytes = 64ll << 20;           // plans larger than this are not considered

struct DensePlan {
  GemmInstance inst;
  int64_t tiles;      // output tiles
  int splits;         // 1: plain dense kernel
  int kb_per_split;
};

DensePlan make_plan(GemmInstance inst, int64_t m, int64_t n, int64_t kblocks, int64_t splits) {
  const InstanceInfo info = instance_info(inst);
  DensePlan plan{inst, ceil_div(m, info.bm) * ceil_div(n, info.bn), 1, (int)kblocks};
  if (splits > 1) {
    plan.kb_per_split = (int)ceil_div(kblocks, splits);
    plan.splits = (int)ceil_div(kblocks, plan.kb_per_split);
  }
  return plan;
}

// Estimated time of a small-M plan (seconds).  Every unit (output tile, or its
// share of K when split) pays a start-up cost, then a per-K-block cost of its
// instance; a split unit also publishes an fp32 partial tile, and the last unit
// of each tile reads all of them back.  Units run in rounds of one per CU.  The
// constants are fitted to MI355X timings of the dense LLM-layer shapes with
// M in {64, 128, 256}, operands in HBM; the plans they pick are within a few
// percent of the best measured plan on each of those shapes.
double plan_seconds(const DensePlan& pl, int cus) {
  constexpr double kUnitStart = 4.3e-6;
  constexpr double kReduceBytesPerSec = 27.6e9;
  double per_kb = 0.0, split_cost = 0.0;
  switch (pl.inst) {
    case kInstSkinny64: per_kb = 0.54e-6; split_cost = 1.6e-6; break;
    case kInstSkinny128: per_kb = 0.69e-6; split_cost = 0.7e-6; break;
    case kInstMid: per_kb = 0.89e-6; split_cost = 0.0; break;
    case kInstLarge: per_kb = 1.06e-6; split_cost = 80e-6; break;   // never worth splitting
    default: per_kb = 2.0e-6; split_cost = 80e-6; break;
  }
  const InstanceInfo info = instance_info(pl.inst);
  const int64_t units = pl.tiles * pl.splits;
  const double rounds = (double)ceil_div(units, cus);
  const double unit = kUnitStart + pl.kb_per_split * per_kb + (pl.splits > 1 ? split_cost : 0.0);
  double t = rounds * unit;
  if (pl.splits > 1) t += pl.splits * (double)info.bm * info.bn * 4 / kReduceBytesPerSec;
  return t;
}

constexpr int kMinKbPerSplit = 2;   // at least 256 of K per unit

// Dense plan: the plain instance choice, unless it leaves more than half of the
// CUs idle; then the cheapest (instance, split) pair by plan_seconds (the CU
// count is a parameter so that the plan, and with it the summation order, does
// not depend on the grid-width override).
DensePlan plan_dense(int64_t m, int64_t n, int64_t k, int cus, bool allow_split) {
  const int64_t kblocks = k / 128;
  if (g_dense_inst >= 0) {
    const int64_t s = allow_split ? std::min<int64_t>(g_dense_splits, kblocks) : 1;
    const DensePlan forced = make_plan((GemmInstance)g_dense_inst, m, n, kblocks, s);
    // one arrival counter per output tile
    if (forced.splits > 1 && forced.tiles > kSplitCounters) return make_plan(forced.inst, m, n, kblocks, 1);
    return forced;
  }
  const DensePlan plain = make_plan(choose_dense(m, n, cus), m, n, kblocks, 1);
  if (plain.tiles * 2 > cus) return plain;
  DensePlan best = plain;
  double best_t = plan_seconds(plain, cus);
  for (GemmInstance inst : {kInstSkinny64, kInstSkinny128, kInstMid, kInstLarge}) {
    const InstanceInfo info = instance_info(inst);
    if (inst == kInstSkinny64 && m > 64) continue;
    const int64_t tiles = ceil_div(m, info.bm) * ceil_div(n, info.bn);
    const int64_t max_splits = allow_split && tiles <= kSplitCounters ? kblocks / kMinKbPerSplit : 1;
    for (int64_t s = 1; s <= max_splits || s == 1; ++s) {
      if (s > 1 && tiles * s * info.bm * info.bn * (int64_t)sizeof(float) > kMaxSplitPartialBytes) break;
      const DensePlan pl = make_plan(inst, m, n, kblocks, s);
      if (pl.splits != s && s > 1) continue;   // same as a smaller split count
      const double t = plan_seconds(pl, cus);
      if (t < best_t) { best = pl; best_t = t; }
    }
  }
  return best;
}

// Workspace bytes a plan needs (0 for an unsplit plan).
int64_t plan_workspace_bytes(const DensePlan& pl) {
  if (pl.splits <= 1) return 0;
  const InstanceInfo info = instance_info(pl.inst);
  return kSplitCounterBytes + pl.tiles * pl.splits * (int64_t)info.bm * info.bn * (int64_t)sizeof(float);
}

// Contiguous layout: the group of a tile is read per 128 rows, so BM = 128.
GemmInstance choose_contiguous(int64_t m_total, int64_t n, int cus) {
  return instance_cost(kInstLarge, m_total, 0, n, cus) <= instance_cost(kInstMid, m_total, 0, n, cus)
             ? kInstLarge : kInstMid;
}

// Contiguous plan.  When the tiles of the chosen instance end in a thinly
// filled last round, the M tiles of the whole rounds run in one launch and the
// rows left over in a second launch of 128x128 tiles, which spreads them over
// twice as many CUs.  A row's result does not depend on its tile, so the split
// changes no bits.
struct ContigPlan {
  GemmInstance head, tail;
  int64_t head_rows;   // rows of the first launch (m_total: one launch)
};

// Estimated cost (same units as instance_cost) of a contiguous plan.
double contig_plan_cost(const ContigPlan& pl, int64_t m_total, int64_t n, int cus);

ContigPlan plan_contiguous(int64_t m_total, int64_t n, int cus) {
  const GemmInstance inst = choose_contiguous(m_total, n, cus);
  ContigPlan pl{inst, inst, m_total};
  const InstanceInfo hi = instance_info(inst);
  const int64_t tiles_n = ceil_div(n, hi.bn);
  const int64_t slots = (int64_t)cus * hi.occ;
  const int64_t tiles = (m_total / hi.bm) * tiles_n;
  const int64_t head_rows = (tiles / slots) * slots / tiles_n * hi.bm;
  if (inst == kInstMid || head_rows <= 0 || head_rows >= m_total) return pl;
  const double round = (double)hi.bm * hi.bn * area_factor(inst);
  const double whole = instance_cost(inst, m_total, 0, n, cus);
  // a fifth of a round for the second launch's start and ramp
  const double split = instance_cost(inst, head_rows, 0, n, cus) + instance_cost(kInstMid, m_total - head_rows, 0, n, cus) +
                       0.2 * round;
  if (split < whole) {
    pl.tail = kInstMid;
    pl.head_rows = head_rows;
  }
  return pl;
}

double contig_plan_cost(const ContigPlan& pl, int64_t m_total, int64_t n, int cus) {
  if (pl.head_rows >= m_total) return instance_cost(pl.head, m_total, 0, n, cus);
  return instance_cost(pl.head, pl.head_rows, 0, n, cus) + instance_cost(pl.tail, m_total - pl.head_rows, 0, n, cus) +
         0.2 * instance_info(pl.head).bm * instance_info(pl.head).bn * area_factor(pl.head);
}

// Split of the paired plan's second launch (the blocks no pair covers): the
// kernel picks s = min(cap, units / (listed blocks x N tiles)) on the device, so
// the partial tiles never exceed `units` (the CU count, as for the dense
// split-K plans).  Needs one arrival counter per (listed block, N tile) for up
// to min(groups, blocks) listed blocks.
struct ContigSplit {
  bool ok;          // the split is possible for this problem
  int units, cap;
  int64_t ws_bytes; // workspace it needs
};

ContigSplit contig_split(GemmInstance si, int64_t nblocks, int64_t n, int64_t k, int num_groups, int cus) {
  const InstanceInfo info = instance_info(si);
  ContigSplit cs{false, cus * info.occ, (int)std::min<int64_t>(k / 128 / kMinKbPerSplit, 64), 0};
  const int64_t max_listed = std::min<int64_t>(num_groups, nblocks);
  cs.ok = cs.cap >= 2 && max_listed * ceil_div(n, info.bn) <= kSplitCounters;
  cs.ws_bytes = kSplitCounterBytes + (int64_t)cs.units * info.bm * info.bn * (int64_t)sizeof(float);
  return cs;
}

// Paired contiguous plan (see grouped_contiguous).  The host does not know the
// routing, so the pair count is estimated: half of the groups end in a single
// block.  Returns the instance for the single blocks and the estimated cost;
// with `split`, the single blocks' launch splits K over the idle CUs.
GemmInstance paired_singles_instance(int64_t nblocks, int64_t n, int64_t k, int num_groups, int cus, bool split,
                                     double* cost) {
  const double singles = (double)std::min<int64_t>(num_groups, nblocks) / 2.0;
  const int64_t single_rows = (int64_t)(singles + 0.5) * 128;
  const int64_t pair_rows = (nblocks * 128 - single_rows) / 256 * 256;
  const GemmInstance si = instance_cost(kInstMid, single_rows, 0, n, cus) <=
                                  instance_cost(kInstLarge, single_rows, 0, n, cus)
                              ? kInstMid : kInstLarge;
  const InstanceInfo info = instance_info(si);
  const double round = (double)info.bm * info.bn * area_factor(si);
  double singles_cost = instance_cost(si, single_rows, 0, n, cus);
  const ContigSplit cs = contig_split(si, nblocks, n, k, num_groups, cus);
  if (split && cs.ok && single_rows > 0) {
    // s splits: ceil(tiles * s / cus) rounds of 1/s of a tile's K each, plus a
    // tenth of a round for the partial-tile hand-off
    const int64_t tiles = single_rows / 128 * ceil_div(n, info.bn);
    const int64_t sp = std::max<int64_t>(1, std::min<int64_t>(cs.cap, cs.units / std::max<int64_t>(tiles, 1)));
    if (sp > 1) singles_cost = (double)ceil_div(tiles * sp, cus) * round / (double)sp + 0.1 * round;
  }
  if (cost) *cost = instance_cost(kInstHuge, pair_rows, 0, n, cus) + singles_cost + 0.2 * round;
  return si;
}

dg_status launch(GemmInstance inst, Variant v, const GemmParams& p, int64_t tile_bound, hipStream_t stream) {
  const int64_t slots = (int64_t)device_cus() * instance_info(inst).occ;
  int64_t grid = tile_bound < slots ? tile_bound : slots;
  if (grid <= 0) return DG_SUCCESS;
  if (tile_bound > INT_MAX) return DG_ERROR_NOT_SUPPORTED;
  return launch_gemm(inst, v, p, (int)grid, stream) == hipSuccess ? DG_SUCCESS : DG_ERROR_LAUNCH;
}

// The kernels address one group's operand rows with 32-bit byte offsets.
bool offsets_fit(int64_t rows_a, int64_t lda, int64_t n, int64_t ldb) {
  // rows * ld <= 2^32 - 1, written so that no product can overflow
  const int64_t lim = (int64_t)UINT32_MAX;
  return lda > 0 && ldb > 0 && rows_a <= lim / lda && n <= lim / ldb;
}

// Sizes the planner's integer arithmetic is written for: every product it
// forms stays far below 2^63.  Larger problems cannot pass offsets_fit either,
// so the size and plan queries report them as never split / not supported.
constexpr int64_t kMaxDim = (int64_t)1 << 31;
bool dims_ok(int64_t m, int64_t n, int64_t k) { return m <= kMaxDim && n <= kMaxDim && k <= kMaxDim; }

}  // namespace
}  // namespace dgfp8

using namespace dgfp8;

DG_EXPORT const char* dg_status_string(dg_status status) {
  switch (status) {
    case DG_SUCCESS: return "DG_SUCCESS";
    case DG_ERROR_INVALID_VALUE: return "DG_ERROR_INVALID_VALUE";
    case DG_ERROR_NOT_SUPPORTED: return "DG_ERROR_NOT_SUPPORTED";
    case DG_ERROR_MISALIGNED_LAYOUT: return "DG_ERROR_MISALIGNED_LAYOUT";
    case DG_ERROR_LAUNCH: return "DG_ERROR_LAUNCH";
    case DG_ERROR_SCRATCH_LIMIT: return "DG_ERROR_SCRATCH_LIMIT";
  }
  return "DG_ERROR_UNKNOWN";
}

DG_EXPORT dg_status dg_set_dense_plan(int instance, int splits) {
  if (instance < 0) {
    g_dense_inst = -1;
    g_dense_splits = 1;
    return DG_SUCCESS;
  }
  if (instance >= kNumInstances || splits < 1) return DG_ERROR_INVALID_VALUE;
  // the 64 x 256 instance serves masked groups only; 256 x 256 and 192 x 256
  // have no split-K variant
  if (instance == kInstDecode) return DG_ERROR_NOT_SUPPORTED;
  if ((instance == kInstHuge || instance == kInstTall) && splits > 1) return DG_ERROR_NOT_SUPPORTED;
  if (splits > kSplitCounters) return DG_ERROR_NOT_SUPPORTED;
  g_dense_inst = instance;
  g_dense_splits = splits;
  return DG_SUCCESS;
}

DG_EXPORT size_t dg_fp8_gemm_nt_workspace_size(int64_t m, int64_t n, int64_t k) {
  if (m <= 0 || n <= 0 || k <= 0 || k % 128 != 0 || !dims_ok(m, n, k)) return 0;
  return (size_t)plan_workspace_bytes(plan_dense(m, n, k, hw_cus(), true));
}

DG_EXPORT dg_status dg_fp8_gemm_nt_tile_config(int64_t m, int64_t n, int64_t k, size_t ws_bytes, int* block_m,
                                               int* block_n, int* splits) {
  if (!block_m || !block_n || !splits) return DG_ERROR_INVALID_VALUE;
  if (m <= 0 || n <= 0 || k <= 0) return DG_ERROR_INVALID_VALUE;
  if (k % 128 != 0 || !dims_ok(m, n, k)) return DG_ERROR_NOT_SUPPORTED;
  DensePlan plan = plan_dense(m, n, k, hw_cus(), ws_bytes > 0);
  if ((int64_t)ws_bytes < plan_workspace_bytes(plan)) plan = plan_dense(m, n, k, hw_cus(), false);
  const InstanceInfo info = instance_info(plan.inst);
  *block_m = info.bm;
  *block_n = info.bn;
  *splits = plan.splits;
  return DG_SUCCESS;
}

namespace {

// Scale words of either format are 4 bytes: the kernels take them through the
// same pointers, the format selects how a K block finds its scale.
const float* sf_ptr(const void* p) { return static_cast<const float*>(p); }

dg_status gemm_nt(const void* a, int64_t lda, const void* sfa, int64_t sfa_sm, int64_t sfa_sk, const void* b,
                  int64_t ldb, const void* sfb, int64_t sfb_sn, int64_t sfb_sk, void* d, int64_t ldd, int64_t m,
                  int64_t n, int64_t k, void* ws, size_t ws_bytes, void* stream, bool packed,
                  const float* c = nullptr, int64_t ldc = 0) {
  if (m < 0 || n < 0 || k < 0) return DG_ERROR_INVALID_VALUE;
  if (m == 0 || n == 0) return DG_SUCCESS;
  dg_status st = check_common(a, lda, sfa, sfa_sm, sfa_sk, b, ldb, sfb, sfb_sn, sfb_sk, d, ldd, n, k);
  if (st != DG_SUCCESS) return st;
  if (!offsets_fit(m, lda, n, ldb)) return DG_ERROR_NOT_SUPPORTED;
  if (ws && !aligned(ws, 16)) return DG_ERROR_NOT_SUPPORTED;
  GemmParams p{};
  p.a = static_cast<const uint8_t*>(a); p.lda = lda;
  p.sfa = sf_ptr(sfa); p.sfa_sm = sfa_sm; p.sfa_sk = sfa_sk;
  p.b = static_cast<const uint8_t*>(b); p.ldb = ldb;
  p.sfb = sf_ptr(sfb); p.sfb_sn = sfb_sn; p.sfb_sk = sfb_sk;
  p.d = static_cast<uint16_t*>(d); p.ldd = ldd;
  p.c = c; p.ldc = ldc;
  p.m = m; p.n = n; p.k = k; p.num_groups = 1;
  p.sf_packed = packed ? 1 : 0;
  // The plan (and so the summation order) follows the hardware CU count, never
  // the grid-width override, so results do not depend on the override.  A
  // split plan runs only when the caller's workspace holds it.
  DensePlan plan = plan_dense(m, n, k, hw_cus(), ws != nullptr);
  const int64_t need = plan_workspace_bytes(plan);
  if (need > 0 && (int64_t)ws_bytes < need) plan = plan_dense(m, n, k, hw_cus(), false);
  if (plan.splits > 1) {
    p.counters = static_cast<int*>(ws);
    p.ws = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + kSplitCounterBytes);
    p.splits = plan.splits;
    p.kb_per_split = plan.kb_per_split;
    return launch(plan.inst, kDenseSplitK, p, plan.tiles * plan.splits, static_cast<hipStream_t>(stream));
  }
  return launch(plan.inst, kDense, p, plan.tiles, static_cast<hipStream_t>(stream));
}

}  // namespace

DG_EXPORT dg_status dg_fp8_gemm_nt_ws(const void* a, int64_t lda, const float* sfa, int64_t sfa_sm, int64_t sfa_sk,
                                      const void* b, int64_t ldb, const float* sfb, int64_t sfb_sn, int64_t sfb_sk,
                                      void* d, int64_t ldd, int64_t m, int64_t n, int64_t k, void* ws,
                                      size_t ws_bytes, void* stream) {
  return gemm_nt(a, lda, sfa, sfa_sm, sfa_sk, b, ldb, sfb, sfb_sn, sfb_sk, d, ldd, m, n, k, ws, ws_bytes, stream,
                 false);
}

DG_EXPORT dg_status dg_fp8_gemm_nt_acc(const void* a, int64_t lda, const float* sfa, int64_t sfa_sm,
                                       int64_t sfa_sk, const void* b, int64_t ldb, const float* sfb, int64_t sfb_sn,
                                       int64_t sfb_sk, const float* c, int64_t ldc, void* d, int64_t ldd, int64_t m,
                                       int64_t n, int64_t k, void* ws, size_t ws_bytes, void* stream) {
  if (m > 0 && n > 0) {
    if (!c || ldc < n) return DG_ERROR_INVALID_VALUE;
    if (ldc % 4 != 0 || !aligned(c, 16)) return DG_ERROR_NOT_SUPPORTED;
  }
  return gemm_nt(a, lda, sfa, sfa_sm, sfa_sk, b, ldb, sfb, sfb_sn, sfb_sk, d, ldd, m, n, k, ws, ws_bytes, stream,
                 false, c, ldc);
}

DG_EXPORT dg_status dg_fp8_gemm_nt_ue8m0(const void* a, int64_t lda, const int32_t* sfa, int64_t sfa_sm,
                                         int64_t sfa_sk, const void* b, int64_t ldb, const int32_t* sfb,
                                         int64_t sfb_sn, int64_t sfb_sk, void* d, int64_t ldd, int64_t m, int64_t n,
                                         int64_t k, void* ws, size_t ws_bytes, void* stream) {
  return gemm_nt(a, lda, sfa, sfa_sm, sfa_sk, b, ldb, sfb, sfb_sn, sfb_sk, d, ldd, m, n, k, ws, ws_bytes, stream,
                 true);
}

DG_EXPORT dg_status dg_fp8_gemm_nt(const void* a, int64_t lda, const float* sfa, int64_t sfa_sm, int64_t sfa_sk,
                                   const void* b, int64_t ldb, const float* sfb, int64_t sfb_sn, int64_t sfb_sk,
                                   void* d, int64_t ldd, int64_t m, int64_t n, int64_t k, void* stream) {
  return dg_fp8_gemm_nt_ws(a, lda, sfa, sfa_sm, sfa_sk, b, ldb, sfb, sfb_sn, sfb_sk, d, ldd, m, n, k, nullptr, 0,
                           stream);
}

namespace {

// Which contiguous plan runs (see grouped_contiguous).  Paired or not, and the
// split, follow the problem, the hardware CU count and the workspace bytes
// available, never the grid-width override: the split changes the summation
// order of the rows it covers.  The one-launch-or-two choice of the unpaired
// plan follows the grid width (it changes no bit).
struct ContigDecision {
  bool paired, split;
  GemmInstance single;
  ContigPlan plain;   // the unpaired plan for the current grid width
};

ContigDecision decide_contiguous(int64_t m_total, int64_t n, int64_t k, int num_groups, size_t ws_bytes) {
  const int cus = hw_cus();
  const int64_t nblocks = m_total / kContiguousAlignment;
  ContigDecision dec{false, false, kInstMid, plan_contiguous(m_total, n, device_cus())};
  if (nblocks > kMaxContigPairBlocks || g_contig_plan == 2) return dec;
  const GemmInstance si_est = paired_singles_instance(nblocks, n, k, num_groups, cus, false, nullptr);
  const ContigSplit cs = contig_split(si_est, nblocks, n, k, num_groups, cus);
  const bool split = cs.ok && (int64_t)ws_bytes >= cs.ws_bytes;
  double paired_cost = 0.0;
  dec.single = paired_singles_instance(nblocks, n, k, num_groups, cus, split, &paired_cost);
  // the model must predict a clear gain: within 10% the two plans measure alike
  dec.paired = g_contig_plan == 1 ||
               paired_cost < 0.9 * contig_plan_cost(plan_contiguous(m_total, n, cus), m_total, n, cus);
  dec.split = dec.paired && split;
  return dec;
}

dg_status grouped_contiguous(const void* a, int64_t lda, const void* sfa, int64_t sfa_sm, int64_t sfa_sk,
                             const void* b, int64_t ldb, int64_t b_group_stride, const void* sfb, int64_t sfb_sn,
                             int64_t sfb_sk, int64_t sfb_group_stride, void* d, int64_t ldd,
                             const int32_t* m_indices, int64_t m_total, int64_t n, int64_t k, int num_groups,
                             void* ws, size_t ws_bytes, void* stream, bool packed) {
  if (m_total < 0 || n < 0 || k < 0 || num_groups < 1) return DG_ERROR_INVALID_VALUE;
  if (b_group_stride < 0 || sfb_group_stride < 0) return DG_ERROR_INVALID_VALUE;
  if (m_total % kContiguousAlignment != 0) return DG_ERROR_MISALIGNED_LAYOUT;
  if (m_total == 0 || n == 0) return DG_SUCCESS;
  if (!m_indices) return DG_ERROR_INVALID_VALUE;
  dg_status st = check_common(a, lda, sfa, sfa_sm, sfa_sk, b, ldb, sfb, sfb_sn, sfb_sk, d, ldd, n, k);
  if (st != DG_SUCCESS) return st;
  if (b_group_stride % 16 != 0 || !aligned(m_indices, 4)) return DG_ERROR_NOT_SUPPORTED;
  if (!strides_ok({b_group_stride, sfb_group_stride, m_total})) return DG_ERROR_NOT_SUPPORTED;
  if (!offsets_fit(m_total, lda, n, ldb)) return DG_ERROR_NOT_SUPPORTED;
  if (ws && !aligned(ws, 16)) return DG_ERROR_NOT_SUPPORTED;
  GemmParams p{};
  p.a = static_cast<const uint8_t*>(a); p.lda = lda;
  p.sfa = sf_ptr(sfa); p.sfa_sm = sfa_sm; p.sfa_sk = sfa_sk;
  p.b = static_cast<const uint8_t*>(b); p.ldb = ldb; p.b_gs = b_group_stride;
  p.sfb = sf_ptr(sfb); p.sfb_sn = sfb_sn; p.sfb_sk = sfb_sk; p.sfb_gs = sfb_group_stride;
  p.d = static_cast<uint16_t*>(d); p.ldd = ldd;
  p.m_indices = m_indices;
  p.m = m_total; p.n = n; p.k = k; p.num_groups = num_groups;
  p.sf_packed = packed ? 1 : 0;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  // Paired plan: when the groups average at least two 128-row blocks, pairs of
  // consecutive blocks of one group run as 256-row tiles (the largest, most
  // efficient tile) and the blocks left over as 128-row tiles in a second
  // launch.  Both launches find their tiles on the device from m_indices, so
  // the plan needs no host read and stays graph-capturable.  Each row's result
  // is computed the same way whatever its tile, so no bit changes.
  //
  // With a workspace the second launch splits K over the CUs its few tiles
  // leave idle (the split is chosen on the device from the listed blocks).
  // The plan follows the hardware CU count, never the grid-width override, so
  // the results (which the split's summation order affects) do not depend on
  // the override.
  const int64_t nblocks = m_total / kContiguousAlignment;
  const ContigDecision dec = decide_contiguous(m_total, n, k, num_groups, ws != nullptr ? ws_bytes : 0);
  if (dec.paired) {
    const InstanceInfo hi = instance_info(kInstHuge);
    GemmParams pp = p;
    pp.contig_mode = 1;
    st = launch(kInstHuge, kContiguous, pp, (nblocks / 2) * ceil_div(n, hi.bn), s);
    if (st != DG_SUCCESS) return st;
    GemmParams ps = p;
    ps.contig_mode = 2;
    const int64_t tiles_bound = std::min<int64_t>(num_groups, nblocks) * ceil_div(n, instance_info(dec.single).bn);
    if (dec.split) {
      const ContigSplit cs = contig_split(dec.single, nblocks, n, k, num_groups, hw_cus());
      ps.counters = static_cast<int*>(ws);
      ps.ws = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + kSplitCounterBytes);
      ps.splits = cs.cap;
      ps.kb_per_split = (int)(k / 128);
      ps.contig_split_units = cs.units;
      return launch(dec.single, kContiguousSplitK, ps, std::max<int64_t>(tiles_bound, cs.units), s);
    }
    return launch(dec.single, kContiguous, ps, tiles_bound, s);
  }
  const ContigPlan pl = dec.plain;
  const InstanceInfo hi = instance_info(pl.head);
  GemmParams ph = p;
  ph.m = pl.head_rows;
  st = launch(pl.head, kContiguous, ph, (pl.head_rows / hi.bm) * ceil_div(n, hi.bn), s);
  if (st != DG_SUCCESS || pl.head_rows == m_total) return st;
  // The rest of the rows: the same problem seen from row head_rows on.
  const int64_t r0 = pl.head_rows;
  const InstanceInfo ti = instance_info(pl.tail);
  GemmParams pt = p;
  pt.a += r0 * lda;
  pt.sfa += r0 * sfa_sm;
  pt.d += r0 * ldd;
  pt.m_indices += r0;
  pt.m = m_total - r0;
  return launch(pl.tail, kContiguous, pt, (pt.m / ti.bm) * ceil_div(n, ti.bn), s);
}

}  // namespace

DG_EXPORT dg_status dg_m_grouped_fp8_gemm_nt_contiguous(
    const void* a, int64_t lda, const float* sfa, int64_t sfa_sm, int64_t sfa_sk,
    const void* b, int64_t ldb, int64_t b_group_stride,
    const float* sfb, int64_t sfb_sn, int64_t sfb_sk, int64_t sfb_group_stride,
    void* d, int64_t ldd, const int32_t* m_indices, int64_t m_total,
    int64_t n, int64_t k, int num_groups, void* stream) {
  return grouped_contiguous(a, lda, sfa, sfa_sm, sfa_sk, b, ldb, b_group_stride, sfb, sfb_sn, sfb_sk,
                            sfb_group_stride, d, ldd, m_indices, m_total, n, k, num_groups, nullptr, 0, stream,
                            false);
}

DG_EXPORT dg_status dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0(
    const void* a, int64_t lda, const int32_t* sfa, int64_t sfa_sm, int64_t sfa_sk,
    const void* b, int64_t ldb, int64_t b_group_stride,
    const int32_t* sfb, int64_t sfb_sn, int64_t sfb_sk, int64_t sfb_group_stride,
    void* d, int64_t ldd, const int32_t* m_indices, int64_t m_total,
    int64_t n, int64_t k, int num_groups, void* stream) {
  return grouped_contiguous(a, lda, sfa, sfa_sm, sfa_sk, b, ldb, b_group_stride, sfb, sfb_sn, sfb_sk,
                            sfb_group_stride, d, ldd, m_indices, m_total, n, k, num_groups, nullptr, 0, stream,
                            true);
}

DG_EXPORT size_t dg_m_grouped_fp8_gemm_nt_contiguous_workspace_size(int64_t m_total, int64_t n, int64_t k,
                                                                    int num_groups) {
  if (m_total <= 0 || n <= 0 || k <= 0 || k % 128 != 0 || num_groups < 1) return 0;
  if (m_total % kContiguousAlignment != 0 || !dims_ok(m_total, n, k)) return 0;
  const ContigDecision dec = decide_contiguous(m_total, n, k, num_groups, (size_t)INT64_MAX);
  if (!dec.split) return 0;
  return (size_t)contig_split(dec.single, m_total / kContiguousAlignment, n, k, num_groups, hw_cus()).ws_bytes;
}

DG_EXPORT dg_status dg_m_grouped_fp8_gemm_nt_contiguous_ws(
    const void* a, int64_t lda, const float* sfa, int64_t sfa_sm, int64_t sfa_sk,
    const void* b, int64_t ldb, int64_t b_group_stride,
    const float* sfb, int64_t sfb_sn, int64_t sfb_sk, int64_t sfb_group_stride,
    void* d, int64_t ldd, const int32_t* m_indices, int64_t m_total,
    int64_t n, int64_t k, int num_groups, void* ws, size_t ws_bytes, void* stream) {
  return grouped_contiguous(a, lda, sfa, sfa_sm, sfa_sk, b, ldb, b_group_stride, sfb, sfb_sn, sfb_sk,
                            sfb_group_stride, d, ldd, m_indices, m_total, n, k, num_groups, ws, ws_bytes, stream,
                            false);
}

DG_EXPORT dg_status dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0_ws(
    const void* a, int64_t lda, const int32_t* sfa, int64_t sfa_sm, int64_t sfa_sk,
    const void* b, int64_t ldb, int64_t b_group_stride,
    const int32_t* sfb, int64_t sfb_sn, int64_t sfb_sk, int64_t sfb_group_stride,
    void* d, int64_t ldd, const int32_t* m_indices, int64_t m_total,
    int64_t n, int64_t k, int num_groups, void* ws, size_t ws_bytes, void* stream) {
  return grouped_contiguous(a, lda, sfa, sfa_sm, sfa_sk, b, ldb, b_group_stride, sfb, sfb_sn, sfb_sk,
                            sfb_group_stride, d, ldd, m_indices, m_total, n, k, num_groups, ws, ws_bytes, stream,
                            true);
}

namespace {

dg_status grouped_masked(const void* a, int64_t lda, int64_t a_group_stride, const void* sfa, int64_t sfa_sm,
                         int64_t sfa_sk, int64_t sfa_group_stride, const void* b, int64_t ldb, int64_t b_group_stride,
                         const void* sfb, int64_t sfb_sn, int64_t sfb_sk, int64_t sfb_group_stride, void* d,
                         int64_t ldd, int64_t d_group_stride, const int32_t* masked_m, int num_groups, int64_t max_m,
                         int64_t n, int64_t k, int64_t expected_m, void* stream, bool packed) {
  if (max_m < 0 || n < 0 || k < 0 || num_groups < 1) return DG_ERROR_INVALID_VALUE;
  if (a_group_stride < 0 || sfa_group_stride < 0 || b_group_stride < 0 || sfb_group_stride < 0 ||
      d_group_stride < 0)
    return DG_ERROR_INVALID_VALUE;
  if (num_groups > kMaxMaskedGroups) return DG_ERROR_NOT_SUPPORTED;
  if (max_m == 0 || n == 0) return DG_SUCCESS;
  if (!masked_m) return DG_ERROR_INVALID_VALUE;
  dg_status st = check_common(a, lda, sfa, sfa_sm, sfa_sk, b, ldb, sfb, sfb_sn, sfb_sk, d, ldd, n, k);
  if (st != DG_SUCCESS) return st;
  if (a_group_stride % 16 != 0 || b_group_stride % 16 != 0 || d_group_stride % 8 != 0 || !aligned(masked_m, 4))
    return DG_ERROR_NOT_SUPPORTED;
  if (!strides_ok({a_group_stride, sfa_group_stride, b_group_stride, sfb_group_stride, d_group_stride, max_m}))
    return DG_ERROR_NOT_SUPPORTED;
  if (!offsets_fit(max_m, lda, n, ldb)) return DG_ERROR_NOT_SUPPORTED;
  GemmParams p{};
  p.a = static_cast<const uint8_t*>(a); p.lda = lda; p.a_gs = a_group_stride;
  p.sfa = sf_ptr(sfa); p.sfa_sm = sfa_sm; p.sfa_sk = sfa_sk; p.sfa_gs = sfa_group_stride;
  p.b = static_cast<const uint8_t*>(b); p.ldb = ldb; p.b_gs = b_group_stride;
  p.sfb = sf_ptr(sfb); p.sfb_sn = sfb_sn; p.sfb_sk = sfb_sk; p.sfb_gs = sfb_group_stride;
  p.d = static_cast<uint16_t*>(d); p.ldd = ldd; p.d_gs = d_group_stride;
  p.masked_m = masked_m;
  p.m = max_m; p.n = n; p.k = k; p.num_groups = num_groups;
  p.sf_packed = packed ? 1 : 0;
  // Each group's B is streamed once per M tile: a 256-row tile covers groups
  // of up to 256 rows in one pass.  When the caller expects few rows per group
  // (decode: expected_m <= 64), 64-row tiles stage a quarter of the A rows and
  // leave LDS for a third stage.  expected_m is a hint only: every instance
  // computes each output element with the same operations in the same order,
  // so the results are the same bits whichever instance runs.
  const GemmInstance inst = (expected_m > 0 && expected_m <= 64) ? kInstDecode
                            : (max_m > 128 ? kInstHuge : kInstLarge);
  const InstanceInfo info = instance_info(inst);
  const int64_t bound = (int64_t)num_groups * ceil_div(max_m, info.bm) * ceil_div(n, info.bn);
  return launch(inst, kMasked, p, bound, static_cast<hipStream_t>(stream));
}

}  // namespace

DG_EXPORT dg_status dg_m_grouped_fp8_gemm_nt_masked(
    const void* a, int64_t lda, int64_t a_group_stride,
    const float* sfa, int64_t sfa_sm, int64_t sfa_sk, int64_t sfa_group_stride,
    const void* b, int64_t ldb, int64_t b_group_stride,
    const float* sfb, int64_t sfb_sn, int64_t sfb_sk, int64_t sfb_group_stride,
    void* d, int64_t ldd, int64_t d_group_stride,
    const int32_t* masked_m, int num_groups, int64_t max_m, int64_t n, int64_t k,
    int64_t expected_m, void* stream) {
  return grouped_masked(a, lda, a_group_stride, sfa, sfa_sm, sfa_sk, sfa_group_stride, b, ldb, b_group_stride, sfb,
                        sfb_sn, sfb_sk, sfb_group_stride, d, ldd, d_group_stride, masked_m, num_groups, max_m, n, k,
                        expected_m, stream, false);
}

DG_EXPORT dg_status dg_m_grouped_fp8_gemm_nt_masked_ue8m0(
    const void* a, int64_t lda, int64_t a_group_stride,
    const int32_t* sfa, int64_t sfa_sm, int64_t sfa_sk, int64_t sfa_group_stride,
    const void* b, int64_t ldb, int64_t b_group_stride,
    const int32_t* sfb, int64_t sfb_sn, int64_t sfb_sk, int64_t sfb_group_stride,
    void* d, int64_t ldd, int64_t d_group_stride,
    const int32_t* masked_m, int num_groups, int64_t max_m, int64_t n, int64_t k,
    int64_t expected_m, void* stream) {
  return grouped_masked(a, lda, a_group_stride, sfa, sfa_sm, sfa_sk, sfa_group_stride, b, ldb, b_group_stride, sfb,
                        sfb_sn, sfb_sk, sfb_group_stride, d, ldd, d_group_stride, masked_m, num_groups, max_m, n, k,
                        expected_m, stream, true);
}

namespace {

dg_status cast_checks(const void* x, int64_t ldx, int64_t x_elem, const void* q, int64_t ldq, const float* sf,
                      int64_t s0, int64_t s1, int64_t rows, int64_t k) {
  if (rows < 0 || k < 0 || s0 < 0 || s1 < 0) return DG_ERROR_INVALID_VALUE;
  if (rows == 0 || k == 0) return DG_SUCCESS;
  if (!x || !q || !sf) return DG_ERROR_INVALID_VALUE;
  if (ldx < k || ldq < k) return DG_ERROR_INVALID_VALUE;
  if (!strides_ok({ldx, ldq, s0, s1, rows, k})) return DG_ERROR_NOT_SUPPORTED;
  if (k % 128 != 0) return DG_ERROR_NOT_SUPPORTED;
  if ((ldx * x_elem) % 16 != 0 || ldq % 16 != 0) return DG_ERROR_NOT_SUPPORTED;
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(sf, 4)) return DG_ERROR_NOT_SUPPORTED;
  return DG_SUCCESS;
}

dg_status per_token(const void* x, int64_t ldx, void* q, int64_t ldq, float* sf, int64_t sf_sm, int64_t sf_sk,
                    int64_t m, int64_t k, int ue8m0, bool f32, void* stream) {
  dg_status st = cast_checks(x, ldx, f32 ? 4 : 2, q, ldq, sf, sf_sm, sf_sk, m, k);
  if (st != DG_SUCCESS || m == 0 || k == 0) return st;
  CastParams p{x, ldx, static_cast<uint8_t*>(q), ldq, sf, sf_sm, sf_sk, m, k, ue8m0 ? 1 : 0};
  return launch_per_token_cast(p, f32, device_cus(), static_cast<hipStream_t>(stream)) == hipSuccess
             ? DG_SUCCESS : DG_ERROR_LAUNCH;
}

}  // namespace

DG_EXPORT dg_status dg_per_token_cast_fp8(const void* x, int64_t ldx, void* q, int64_t ldq, float* sf,
                                          int64_t sf_sm, int64_t sf_sk, int64_t m, int64_t k, int ue8m0,
                                          void* stream) {
  return per_token(x, ldx, q, ldq, sf, sf_sm, sf_sk, m, k, ue8m0, false, stream);
}

DG_EXPORT dg_status dg_per_token_cast_fp8_f32(const void* x, int64_t ldx, void* q, int64_t ldq, float* sf,
                                              int64_t sf_sm, int64_t sf_sk, int64_t m, int64_t k, int ue8m0,
                                              void* stream) {
  return per_token(x, ldx, q, ldq, sf, sf_sm, sf_sk, m, k, ue8m0, true, stream);
}

DG_EXPORT dg_status dg_per_block_cast_fp8(const void* x, int64_t ldx, void* q, int64_t ldq, float* sf,
                                          int64_t sf_sn, int64_t sf_sk, int64_t n, int64_t k, int ue8m0,
                                          void* stream) {
  dg_status st = cast_checks(x, ldx, 4, q, ldq, sf, sf_sn, sf_sk, n, k);
  if (st != DG_SUCCESS || n == 0 || k == 0) return st;
  if (ceil_div(n, 128) * (k / 128) > INT_MAX) return DG_ERROR_NOT_SUPPORTED;
  CastParams p{x, ldx, static_cast<uint8_t*>(q), ldq, sf, sf_sn, sf_sk, n, k, ue8m0 ? 1 : 0};
  return launch_per_block_cast(p, static_cast<hipStream_t>(stream)) == hipSuccess ? DG_SUCCESS : DG_ERROR_LAUNCH;
}

DG_EXPORT dg_status dg_pack_ue8m0(const float* sf, int64_t sf_s0, int64_t sf_s1, int32_t* out, int64_t out_s0,
                                  int64_t out_s1, int64_t rows, int64_t kblocks, void* stream) {
  if (rows < 0 || kblocks < 0 || sf_s0 < 0 || sf_s1 < 0 || out_s0 < 0 || out_s1 < 0) return DG_ERROR_INVALID_VALUE;
  if (rows == 0 || kblocks == 0) return DG_SUCCESS;
  if (!sf || !out) return DG_ERROR_INVALID_VALUE;
  if (!strides_ok({sf_s0, sf_s1, out_s0, out_s1, rows, kblocks})) return DG_ERROR_NOT_SUPPORTED;
  if (!aligned(sf, 4) || !aligned(out, 4)) return DG_ERROR_NOT_SUPPORTED;
  PackParams p{sf, sf_s0, sf_s1, out, out_s0, out_s1, rows, kblocks};
  return launch_pack_ue8m0(p, device_cus(), static_cast<hipStream_t>(stream)) == hipSuccess ? DG_SUCCESS
                                                                                            : DG_ERROR_LAUNCH;
}

DG_EXPORT int dg_get_mk_alignment_for_contiguous_layout(void) { return kContiguousAlignment; }

DG_EXPORT dg_status dg_set_num_cus(int num_cus) {
  g_num_cus_override = num_cus > 0 ? num_cus : 0;
  return DG_SUCCESS;
}

DG_EXPORT int dg_get_num_cus(void) { return device_cus(); }

DG_EXPORT dg_status dg_set_contiguous_plan(int plan) {
  if (plan < 0 || plan > 2) return DG_ERROR_INVALID_VALUE;
  g_contig_plan = plan;
  return DG_SUCCESS;
}

