/*
 * libdgfp8 -- FP8 GEMM with fine-grained block scaling for MI355X (gfx950).
 *
 * C ABI.  Plain pointers and sizes only.  Every pointer marked "device" is a
 * device address on the current HIP device; "stream" is a hipStream_t passed
 * as void* (NULL selects the default stream).  All work is enqueued on that
 * stream and the call returns without synchronising.  The caller owns every
 * buffer, including the optional split-K workspace of dg_fp8_gemm_nt_ws; the
 * library allocates no device memory and keeps no device state besides the
 * compute-unit count used for the persistent grid.
 *
 * Errors: every entry point validates its arguments on the host and returns a
 * dg_status.  Nothing aborts and no exception crosses the ABI.  A problem
 * with a zero-sized dimension returns DG_SUCCESS without launching anything.
 * Device-side preconditions that are not checked are stated per function.
 *
 * Method (pages on DeepGEMM): D(bf16) = A . B^T in the NT layout (both
 * operands K-major), with E4M3 A carrying one fp32 scale per row per 128-wide
 * K block and E4M3 B one fp32 scale per 128x128 block; every K block's partial
 * product is scaled and promoted into an fp32 accumulator.  Sources: page
 * "GitHub 推荐：DeepSeek 开源周最大黑马 DeepGEMM…" (问题判断: 128x128 block
 * scaling; 创新之处: per-block scaling through promotion; 解法哲学: the
 * fp8_gemm_nt call with a caller-provided output d); page juejin.cn post on
 * DeepGEMM (section 3: two-level accumulation and M-only grouping; section
 * 4(3): dense, contiguous and masked GEMM types; section 5: API names).
 *
 * Scale-factor contract (all GEMM entry points):
 *   SFA is fp32, logically [rows, K/128]; element (i, kb) lives at
 *       sfa[i * sfa_sm + kb * sfa_sk]  (row-major: sfa_sm = K/128, sfa_sk = 1;
 *       MN-major / "transposed": sfa_sm = 1, sfa_sk = rows).
 *   SFB is fp32, logically [ceil(N/128), K/128]; element (nb, kb) at
 *       sfb[nb * sfb_sn + kb * sfb_sk]; output column j uses nb = j / 128.
 *   E4M3 is the OCP "FN" flavour (largest finite 448, no infinities).
 *   Strides are in elements and must be >= 0.
 *   Scale values (fp32 entry points): finite fp32, negative ones flipping the
 *   sign of their block's contribution.  A zero scale makes its block
 *   contribute nothing, as the definition says.  Subnormal scales are applied
 *   exactly as long as the product sfa * sfb of a row's block is at least
 *   2^-189; smaller products contribute nothing.  A product of 2^65 or more,
 *   or an infinite or NaN scale, gives NaN in every output it weights.  (The
 *   casts produce scales between fp32(1e-4)/448 and 2^121.)
 *
 * Alignment contract: K % 128 == 0; lda, ldb and the A/B base addresses are
 * multiples of 16 bytes; N % 8 == 0, ldd % 8 == 0 and D is 16-byte aligned.
 * Violations return DG_ERROR_NOT_SUPPORTED.
 *
 * Accuracy (measured on gfx950 and pinned by tests): within one 128-wide K
 * block the matrix unit keeps each product only within a 14-bit window below
 * the block's largest product, cutting each toward zero.  Every block's
 * partial is then promoted into an fp32 accumulator.  The promotion rounds the
 * partial's excess bits to nearest even, and truncates toward minus infinity
 * the accumulator bits that a larger partial pushes below the fp32 grid.  The
 * bf16 output is rounded to nearest even once.  Results are deterministic and
 * do not depend on the persistent grid width.  A K split changes only the
 * last bits: its partial tiles are added in split order.
 *
 * Size contract: one group's A rows and B rows are addressed with 32-bit byte
 * offsets (rows x leading dimension < 2^32), and no size, leading dimension,
 * scale stride or group stride may exceed 2^40; larger values return
 * DG_ERROR_NOT_SUPPORTED before anything is launched (the casts and the
 * scale packing apply the 2^40 bound too).
 */
#ifndef DGFP8_H_
#define DGFP8_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dg_status {
  DG_SUCCESS = 0,
  DG_ERROR_INVALID_VALUE = 1,     /* null pointer, negative size, bad stride, bad group count */
  DG_ERROR_NOT_SUPPORTED = 2,     /* K % 128 != 0, misaligned pointer / leading dimension, N % 8 != 0 */
  DG_ERROR_MISALIGNED_LAYOUT = 3, /* contiguous layout: m_total % 128 != 0 */
  DG_ERROR_LAUNCH = 4,            /* HIP reported an error at launch */
  DG_ERROR_SCRATCH_LIMIT = 5      /* dg_fp8_gemm_nt_noalloc: the problem needs more split-K scratch than its static maximum */
} dg_status;

/* Human-readable name of a status; never NULL.  Errors are returned rather
 * than raised, so the caller decides how to report them (page "GitHub 推荐：
 * DeepSeek 开源周最大黑马 DeepGEMM…", 解法哲学 and 可复用的模式与技巧: host-side
 * assertions on every layout field give the caller a clear error). */
const char* dg_status_string(dg_status status);

/*
 * Dense GEMM: D[m, n] = sum_kb sfa[m, kb] * sfb[n/128, kb] * sum_{k in kb} A[m, k] * B[n, k],
 * rounded to bf16 (round to nearest even).
 *   a   device, E4M3 [m, k], row stride lda (bytes = elements)
 *   sfa device, fp32, see the scale-factor contract (rows = m)
 *   b   device, E4M3 [n, k], row stride ldb
 *   sfb device, fp32 [ceil(n/128), k/128] with strides sfb_sn, sfb_sk
 *   d   device, bf16 [m, n], row stride ldd (elements); fully overwritten
 * Never splits the K range (see dg_fp8_gemm_nt_ws); equivalent to
 * dg_fp8_gemm_nt_ws with no workspace.
 * Page "GitHub 推荐…DeepGEMM…", 解法哲学 (fp8_gemm_nt with output d);
 * page juejin.cn, section 4(3) (dense GEMM type).
 */
dg_status dg_fp8_gemm_nt(const void* a, int64_t lda,
                         const float* sfa, int64_t sfa_sm, int64_t sfa_sk,
                         const void* b, int64_t ldb,
                         const float* sfb, int64_t sfb_sn, int64_t sfb_sk,
                         void* d, int64_t ldd,
                         int64_t m, int64_t n, int64_t k,
                         void* stream);

/*
 * Dense GEMM as dg_fp8_gemm_nt, with a caller-provided workspace that lets a
 * small-m problem (too few output tiles to occupy the device) split its K
 * blocks over several workgroups per output tile.  Each split unit sums its
 * K blocks in order into an fp32 partial tile; the last unit to finish adds
 * the partials in split order and writes D.  Results are deterministic and
 * independent of dg_set_num_cus, but may differ from the unsplit sum in the
 * last fp32 bits (both within the method's tolerance).
 *   ws        device, 16-byte aligned, ws_bytes long, or NULL (no split).
 *             Its first 256 KiB hold arrival counters: they must be zero
 *             before the workspace is first used, and every completed call
 *             leaves them zero, so a workspace can be reused by any later call
 *             on the same stream.  Calls that may run concurrently need
 *             distinct workspaces.  The rest holds fp32 partial tiles.
 *   ws_bytes  at least dg_fp8_gemm_nt_workspace_size(m, n, k) to enable the
 *             split; a smaller (or NULL) workspace runs the unsplit kernel.
 * Split-K is this library's answer to small m on a 256-CU device; the pages
 * only note that thin shapes (small M, large N and K) run at low efficiency
 * (page discosf.com news post on DeepGEMM, sections 4.3 and 5.4).
 */
dg_status dg_fp8_gemm_nt_ws(const void* a, int64_t lda,
                            const float* sfa, int64_t sfa_sm, int64_t sfa_sk,
                            const void* b, int64_t ldb,
                            const float* sfb, int64_t sfb_sn, int64_t sfb_sk,
                            void* d, int64_t ldd,
                            int64_t m, int64_t n, int64_t k,
                            void* ws, size_t ws_bytes,
                            void* stream);

/*
 * Accumulating dense GEMM: D = RNE_bf16(C + A . B^T), C an fp32 addend of D's
 * shape added to the fp32 result before the single rounding to bf16.  The
 * optional c argument of fp8_gemm_nt (page "GitHub 推荐…DeepGEMM…", 解法哲学);
 * the pages say no more about it, and this reading is the plainest one.
 * Same arguments, workspace rules and results as dg_fp8_gemm_nt_ws, plus
 *   c    device, fp32 [m, n], row stride ldc (elements); read only, must not
 *        overlap d
 * Errors (for m, n > 0): null c or ldc < n -> DG_ERROR_INVALID_VALUE;
 * c not 16-byte aligned or ldc % 4 != 0 -> DG_ERROR_NOT_SUPPORTED.
 */
dg_status dg_fp8_gemm_nt_acc(const void* a, int64_t lda,
                             const float* sfa, int64_t sfa_sm, int64_t sfa_sk,
                             const void* b, int64_t ldb,
                             const float* sfb, int64_t sfb_sn, int64_t sfb_sk,
                             const float* c, int64_t ldc,
                             void* d, int64_t ldd,
                             int64_t m, int64_t n, int64_t k,
                             void* ws, size_t ws_bytes,
                             void* stream);

/*
 * Dense GEMM for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments (without ws, ws_bytes) and results as dg_fp8_gemm_nt_ws given
 * a workspace of dg_fp8_gemm_nt_workspace_size(m, n, k) bytes: the split-K
 * partial tiles and arrival counters live in a static device array of the
 * library instead, 16 MiB of partials plus the 256 KiB counter block
 * (16.25 MiB per device, held from the device's first such call until the
 * process ends).  Nothing is allocated and nothing is freed.
 *   A problem whose split plan needs more than that returns
 *   DG_ERROR_SCRATCH_LIMIT before anything is launched (call
 *   dg_fp8_gemm_nt_ws with a workspace of your own instead).
 *   Every call on one device shares that device's array: calls that may
 *   overlap on one device (other streams, other host threads) race and give
 *   wrong results; calls in order on one stream are safe.  The counters are
 *   zero when the array is first used and every completed call leaves them
 *   zero.
 */
dg_status dg_fp8_gemm_nt_noalloc(const void* a, int64_t lda,
                                 const float* sfa, int64_t sfa_sm, int64_t sfa_sk,
                                 const void* b, int64_t ldb,
                                 const float* sfb, int64_t sfb_sn, int64_t sfb_sk,
                                 void* d, int64_t ldd,
                                 int64_t m, int64_t n, int64_t k,
                                 void* stream);

/* Workspace bytes dg_fp8_gemm_nt_ws needs to split this problem; 0 when the
 * problem runs unsplit (or the sizes are invalid).  Depends only on m, n, k
 * and the device's compute-unit count. */
size_t dg_fp8_gemm_nt_workspace_size(int64_t m, int64_t n, int64_t k);

/* The output tile (block_m x block_n) and K split count dg_fp8_gemm_nt_ws
 * would use for this problem with a workspace of ws_bytes (0: none).  The
 * choice is a pure function of the shape and the device's compute-unit count,
 * made by a cost model rather than by timing candidates (page "GitHub 推荐：
 * DeepSeek 开源周最大黑马 DeepGEMM…", 创新之处 on the analytical heuristics
 * that rank a small, constrained set of block shapes; page "企业官网建设流程
 * 全解析", section 2.1 on per-shape configurations).  For profiling and logs; the
 * choice never changes results beyond the split-K note above.  Errors: null
 * outputs or non-positive sizes -> DG_ERROR_INVALID_VALUE, k % 128 != 0 ->
 * DG_ERROR_NOT_SUPPORTED. */
dg_status dg_fp8_gemm_nt_tile_config(int64_t m, int64_t n, int64_t k, size_t ws_bytes,
                                     int* block_m, int* block_n, int* splits);

/*
 * M-grouped GEMM, contiguous layout (MoE prefill / training forward).
 * The rows of all groups are concatenated along M; each group's segment is
 * padded to a multiple of 128 rows (dg_get_mk_alignment_for_contiguous_layout).
 *   a         device, E4M3 [m_total, k], row stride lda
 *   sfa       device, fp32, rows = m_total (scale-factor contract)
 *   b         device, E4M3 [num_groups, n, k]; group g starts at b + g * b_group_stride,
 *             rows of a group have stride ldb
 *   sfb       device, fp32 [num_groups, ceil(n/128), k/128]; group g at sfb + g * sfb_group_stride
 *   d         device, bf16 [m_total, n], row stride ldd
 *   m_indices device, int32 [m_total]: group of each row, -1 on padding rows
 * Row i with m_indices[i] = g >= 0 gets row i of A times B[g]^T.  Rows with
 * m_indices[i] == -1 are NOT written (their contents are left untouched).
 * Preconditions (not checked on the device): in each aligned 128-row block
 * every row with m_indices >= 0 has the same value, which lies in
 * [0, num_groups).  The group of a block is read from its first row; a block
 * whose first row is -1 is skipped entirely.
 * The work is one or two kernel launches on the same stream, planned from the
 * sizes alone (the host never reads m_indices, so the call can be captured in
 * a graph): when groups average two or more 128-row blocks, pairs of
 * consecutive blocks of one group run as 256-row tiles and the blocks left
 * over as 128-row tiles in a second launch, both tile lists built on the
 * device; otherwise one tile per block, split into two launches when the tiles
 * end in a thinly filled last round.  Every row is computed with the same
 * operations in all of these plans, so the results do not depend on the plan
 * or on dg_set_num_cus.  No K is split (see the _ws variant).
 * Errors: m_total % 128 != 0 -> DG_ERROR_MISALIGNED_LAYOUT.
 * Page juejin.cn, sections 3 and 4(3) (M-only grouping, contiguous layout
 * aligned to the M block); page "GitHub 推荐…", 风险与不足 (128-row padding).
 */
dg_status dg_m_grouped_fp8_gemm_nt_contiguous(const void* a, int64_t lda,
                                              const float* sfa, int64_t sfa_sm, int64_t sfa_sk,
                                              const void* b, int64_t ldb, int64_t b_group_stride,
                                              const float* sfb, int64_t sfb_sn, int64_t sfb_sk,
                                              int64_t sfb_group_stride,
                                              void* d, int64_t ldd,
                                              const int32_t* m_indices, int64_t m_total,
                                              int64_t n, int64_t k, int num_groups,
                                              void* stream);

/*
 * M-grouped GEMM, masked layout (MoE decode; usable under HIP graph capture).
 *   a        device, E4M3 [num_groups, max_m, k]; group g at a + g * a_group_stride, rows lda
 *   sfa      device, fp32 [num_groups, max_m, k/128]; group g at sfa + g * sfa_group_stride,
 *            then the scale-factor contract with rows = max_m
 *   b, sfb   as in the contiguous variant
 *   d        device, bf16 [num_groups, max_m, n]; group g at d + g * d_group_stride, rows ldd
 *   masked_m device, int32 [num_groups]: valid rows of each group, read on the
 *            device at run time (never by the host), clamped to [0, max_m]
 *   expected_m  hint of the typical masked_m (it picks the tile height: at most
 *            64 selects 64-row tiles, made for decode); never changes results
 * For group g, rows i < masked_m[g] get A[g, i] times B[g]^T; rows at or beyond
 * masked_m[g] are left untouched.
 * Page juejin.cn, section 4(3) (masked grouped GEMM for decode with graphs).
 */
dg_status dg_m_grouped_fp8_gemm_nt_masked(const void* a, int64_t lda, int64_t a_group_stride,
                                          const float* sfa, int64_t sfa_sm, int64_t sfa_sk,
                                          int64_t sfa_group_stride,
                                          const void* b, int64_t ldb, int64_t b_group_stride,
                                          const float* sfb, int64_t sfb_sn, int64_t sfb_sk,
                                          int64_t sfb_group_stride,
                                          void* d, int64_t ldd, int64_t d_group_stride,
                                          const int32_t* masked_m, int num_groups,
                                          int64_t max_m, int64_t n, int64_t k,
                                          int64_t expected_m,
                                          void* stream);

/*
 * Per-token FP8 cast (the library's GEMMs take E4M3 inputs; the caller does the
 * cast: page ssnai.com DeepGEMM analysis, the warning that casting is the
 * caller's job).  For each row i and 128-wide block kb of a bf16 [m, k] input:
 *   amax = max |x|;  s = fl32(max(amax, 1e-4) / 448)  (IEEE fp32 division);
 *   if ue8m0 != 0: s = smallest power of two >= s;
 *   q = E4M3 round-to-nearest-even of clamp(fl32(x / s), -448, 448), sign kept.
 *   x   device, bf16 [m, k], row stride ldx (elements), 16-byte aligned rows
 *   q   device, E4M3 [m, k], row stride ldq (bytes), 16-byte aligned rows
 *   sf  device, fp32 [m, k/128]: element (i, kb) at sf[i * sf_sm + kb * sf_sk]
 * Results are bit-exact with the definition above.
 */
dg_status dg_per_token_cast_fp8(const void* x, int64_t ldx,
                                void* q, int64_t ldq,
                                float* sf, int64_t sf_sm, int64_t sf_sk,
                                int64_t m, int64_t k, int ue8m0,
                                void* stream);

/* Same as dg_per_token_cast_fp8 for an fp32 [m, k] input. */
dg_status dg_per_token_cast_fp8_f32(const void* x, int64_t ldx,
                                    void* q, int64_t ldq,
                                    float* sf, int64_t sf_sm, int64_t sf_sk,
                                    int64_t m, int64_t k, int ue8m0,
                                    void* stream);

/*
 * Weight-side cast: fp32 [n, k] -> E4M3 [n, k] with one scale per 128x128 block
 * (rows beyond n in the last block do not exist and do not enter its amax).
 * The weights' block granularity is the method's (page "GitHub 推荐：DeepSeek
 * 开源周最大黑马 DeepGEMM…", 问题判断); the pages tell users to prepare
 * weights and scales with the library's weight conversion tools (page
 * ssnai.com DeepGEMM analysis, the FP8/FP4 pitfall notes and Mega MoE steps).
 * Same scale and code rules as dg_per_token_cast_fp8, amax taken over the block.
 *   sf  device, fp32 [ceil(n/128), k/128]: element (nb, kb) at sf[nb * sf_sn + kb * sf_sk]
 */
dg_status dg_per_block_cast_fp8(const void* x, int64_t ldx,
                                void* q, int64_t ldq,
                                float* sf, int64_t sf_sn, int64_t sf_sk,
                                int64_t n, int64_t k, int ue8m0,
                                void* stream);

/*
 * Packed UE8M0 scales (the exponent-only scale format; page "GitHub 推荐：DeepSeek
 * 开源周最大黑马 DeepGEMM…", 可复用的模式与技巧 "UE8M0 int32 packing" and
 * the SF dual path next to it; page ssnai.com DeepGEMM analysis, on the scale
 * formats of the two GPU generations).
 *
 * Packed contract: a scale word is an int32 holding the 8-bit biased
 * exponents e (value 2^(e-127)) of 4 consecutive K blocks, little-endian:
 * byte j (bits 8j..8j+7) of word w belongs to K block 4w + j.  Bytes past the
 * last K block are ignored.  e = 255 is not a scale (outside the contract).
 *   SFA words: logically [rows, ceil(K/512)]; word (i, w) at sfa[i * sfa_sm + w * sfa_sk]
 *   SFB words: logically [ceil(N/128), ceil(K/512)]; word (nb, w) at sfb[nb * sfb_sn + w * sfb_sk]
 * Strides are in int32 elements.  With such scales each K block's product
 * 2^(ea + eb - 254) * P is exact in the accumulator's exponent range, so these
 * entry points run kernels without any per-block rescaling; with power-of-two
 * fp32 scales the fp32 entry points give bit-identical results.
 */

/* Dense GEMM as dg_fp8_gemm_nt_ws (same workspace rules) with packed UE8M0 scales. */
dg_status dg_fp8_gemm_nt_ue8m0(const void* a, int64_t lda,
                               const int32_t* sfa, int64_t sfa_sm, int64_t sfa_sk,
                               const void* b, int64_t ldb,
                               const int32_t* sfb, int64_t sfb_sn, int64_t sfb_sk,
                               void* d, int64_t ldd,
                               int64_t m, int64_t n, int64_t k,
                               void* ws, size_t ws_bytes,
                               void* stream);

/* Contiguous grouped GEMM as dg_m_grouped_fp8_gemm_nt_contiguous with packed
 * UE8M0 scales (sfb_group_stride in int32 elements). */
dg_status dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0(const void* a, int64_t lda,
                                                    const int32_t* sfa, int64_t sfa_sm, int64_t sfa_sk,
                                                    const void* b, int64_t ldb, int64_t b_group_stride,
                                                    const int32_t* sfb, int64_t sfb_sn, int64_t sfb_sk,
                                                    int64_t sfb_group_stride,
                                                    void* d, int64_t ldd,
                                                    const int32_t* m_indices, int64_t m_total,
                                                    int64_t n, int64_t k, int num_groups,
                                                    void* stream);

/*
 * Contiguous grouped GEMM as dg_m_grouped_fp8_gemm_nt_contiguous, with a
 * split-K workspace (caller-owned, 16-byte aligned, same contract as the dense
 * one: the first 256 KiB are arrival counters, zero before first use and left
 * zero by every completed call; calls that may overlap need distinct
 * workspaces).  When the paired plan runs and ws_bytes is at least
 * dg_m_grouped_fp8_gemm_nt_contiguous_workspace_size(...), the second launch
 * (the blocks no pair covers, typically one per group) splits K over the CUs
 * its few tiles would leave idle: the kernel picks the split from the number
 * of leftover blocks it finds, so the call stays graph-capturable.  Each split
 * sums its K range in order and the last to arrive adds the fp32 partial tiles
 * in split order, so results are deterministic and independent of
 * dg_set_num_cus; rows of leftover blocks may differ from the unsplit call in
 * the last bits, rows of paired blocks do not.  With ws null or too small the
 * call behaves as dg_m_grouped_fp8_gemm_nt_contiguous.
 * Errors: as dg_m_grouped_fp8_gemm_nt_contiguous; ws not 16-byte aligned ->
 * DG_ERROR_NOT_SUPPORTED.
 * Splitting K over workgroups is this library's addition for a 256-CU device
 * (the pages only note low efficiency for thin shapes: page "企业官网建设流程全解析",
 * sections 4.3 and 5.4).
 */
dg_status dg_m_grouped_fp8_gemm_nt_contiguous_ws(const void* a, int64_t lda,
                                                 const float* sfa, int64_t sfa_sm, int64_t sfa_sk,
                                                 const void* b, int64_t ldb, int64_t b_group_stride,
                                                 const float* sfb, int64_t sfb_sn, int64_t sfb_sk,
                                                 int64_t sfb_group_stride,
                                                 void* d, int64_t ldd,
                                                 const int32_t* m_indices, int64_t m_total,
                                                 int64_t n, int64_t k, int num_groups,
                                                 void* ws, size_t ws_bytes, void* stream);

/* As dg_m_grouped_fp8_gemm_nt_contiguous_ws with packed UE8M0 scales. */
dg_status dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0_ws(const void* a, int64_t lda,
                                                       const int32_t* sfa, int64_t sfa_sm, int64_t sfa_sk,
                                                       const void* b, int64_t ldb, int64_t b_group_stride,
                                                       const int32_t* sfb, int64_t sfb_sn, int64_t sfb_sk,
                                                       int64_t sfb_group_stride,
                                                       void* d, int64_t ldd,
                                                       const int32_t* m_indices, int64_t m_total,
                                                       int64_t n, int64_t k, int num_groups,
                                                       void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes the _ws contiguous calls can use for this problem (0: the
 * plan never splits K).  Non-positive sizes, k % 128 != 0, m_total % 128 != 0 or
 * num_groups < 1 give 0. */
size_t dg_m_grouped_fp8_gemm_nt_contiguous_workspace_size(int64_t m_total, int64_t n, int64_t k,
                                                          int num_groups);

/* Masked grouped GEMM as dg_m_grouped_fp8_gemm_nt_masked with packed UE8M0
 * scales (group strides in int32 elements). */
dg_status dg_m_grouped_fp8_gemm_nt_masked_ue8m0(const void* a, int64_t lda, int64_t a_group_stride,
                                                const int32_t* sfa, int64_t sfa_sm, int64_t sfa_sk,
                                                int64_t sfa_group_stride,
                                                const void* b, int64_t ldb, int64_t b_group_stride,
                                                const int32_t* sfb, int64_t sfb_sn, int64_t sfb_sk,
                                                int64_t sfb_group_stride,
                                                void* d, int64_t ldd, int64_t d_group_stride,
                                                const int32_t* masked_m, int num_groups,
                                                int64_t max_m, int64_t n, int64_t k,
                                                int64_t expected_m,
                                                void* stream);

/*
 * Scale transform fp32 -> packed UE8M0: for every row i and K block kb,
 * e = biased exponent of sf(i, kb), plus 1 when any mantissa bit is set (the
 * smallest power of two >= the scale, as the casts' ue8m0 mode), stored in
 * byte kb % 4 of word (i, kb / 4); bytes past the last K block are 0.  Exact for
 * power-of-two scales, which is what the casts produce with ue8m0 != 0.  Inputs
 * must be positive normal fp32 no larger than 2^127 (other values are outside
 * the contract).
 *   sf   device, fp32 [rows, kblocks]: element (i, kb) at sf[i * sf_s0 + kb * sf_s1]
 *   out  device, int32 [rows, ceil(kblocks/4)]: word (i, w) at out[i * out_s0 + w * out_s1]
 * Errors: negative sizes/strides or null pointers -> DG_ERROR_INVALID_VALUE;
 * pointers not 4-byte aligned -> DG_ERROR_NOT_SUPPORTED.
 */
dg_status dg_pack_ue8m0(const float* sf, int64_t sf_s0, int64_t sf_s1,
                        int32_t* out, int64_t out_s0, int64_t out_s1,
                        int64_t rows, int64_t kblocks,
                        void* stream);

/*
 * Plan of the contiguous grouped GEMM: 0 (default) picks by the cost model;
 * 1 forces the paired plan (256-row tiles on pairs of consecutive 128-row
 * blocks of one group, found on the device from m_indices, and 128-row tiles on
 * the blocks no pair covers: two launches); 2 forces one tile per 128-row
 * block.  Layouts of more than 2048 blocks always take plan 2.  Every plan
 * computes each output row with the same operations, so the choice never
 * changes a bit of the result; it is a tuning and testing knob, process-wide.
 * Errors: plan outside 0..2 -> DG_ERROR_INVALID_VALUE.
 */
dg_status dg_set_contiguous_plan(int plan);

/*
 * Plan of the dense GEMM (dg_fp8_gemm_nt and its variants): instance < 0
 * (default) picks the kernel instance and K split by the cost model; otherwise
 * every following dense call in the process uses this instance, with `splits`
 * K splits when the call has a workspace that holds them (else 1).  The
 * workspace-size and tile-config queries report the forced plan.  Instances:
 *   0 128x256, 1 128x128, 2 256x256, 3 128x64, 4 64x64  (LDS stages shared by
 *     the workgroup's waves)
 *   6 192x256
 * A tuning and testing knob (the split changes the fp32 summation order, so
 * results may differ in the last bits between plans).
 * Errors: instance > 6 or splits < 1 -> DG_ERROR_INVALID_VALUE; instance 5
 * (masked groups only), or splits > 1 with instance 2 or 6 (no split-K
 * variant), or splits > 65536 -> DG_ERROR_NOT_SUPPORTED.
 */
dg_status dg_set_dense_plan(int instance, int splits);

/* Row alignment of each group's segment in the contiguous layout: 128.
 * (Page ssnai.com DeepGEMM analysis: the alignment query for contiguous MoE.) */
int dg_get_mk_alignment_for_contiguous_layout(void);

/*
 * Width of the persistent GEMM grid in compute units (default: all CUs of the
 * current device).  Results never depend on it.  num_cus <= 0 restores the
 * default.  (Analog of set_num_sms: page ssnai.com DeepGEMM analysis.)
 */
dg_status dg_set_num_cus(int num_cus);
int dg_get_num_cus(void);

#ifdef __cplusplus
}
#endif

#endif /* DGFP8_H_ */
