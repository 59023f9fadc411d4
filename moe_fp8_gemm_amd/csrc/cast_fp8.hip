// FP8 (E4M3) quantizers: per-token 1x128 blocks (bf16 or fp32 input) and
// per-weight 128x128 blocks (fp32 input).  Bandwidth-bound streaming kernels.
//
// The GEMMs take E4M3 operands with block scales; the cast is the caller's job
// (page ssnai.com DeepGEMM analysis: no automatic FP8 casting).  Scale and code
// rules, bit-exact:
//   amax = max |x| over the block;  s = fl32(max(amax, 1e-4) / 448)  (IEEE division);
//   UE8M0 mode: s rounded up to a power of two (exponent-only scales, page
//   ssnai.com analysis, the SM100 scale-format notes);
//   q = E4M3 RNE of clamp(fl32(x / s), +-448), sign of zero kept.
// Block scaling and the E4M3 format: page "GitHub 推荐…DeepGEMM…", 问题判断;
// page "企业官网建设流程全解析", section 2.3.
//
// Per-token layout: 16 lanes own one 128-element block (8 elements each), so a
// wave covers 4 blocks and the block amax is a 16-lane butterfly reduction.
#include "dgfp8_internal.h"

namespace dgfp8 {
namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kE4M3Max = 448.0f;
constexpr float kAmaxFloor = 1e-4f;

__device__ __forceinline__ float block_scale(float amax, int ue8m0) {
  float s = fmaxf(amax, kAmaxFloor) / kE4M3Max;   // correctly rounded fp32 division
  if (ue8m0) {
    uint32_t u = __float_as_uint(s);
    if (u & 0x007FFFFFu) u = (u & 0x7F800000u) + 0x00800000u;
    s = __uint_as_float(u);
  }
  return s;
}

// Correctly rounded fl32(|x| / s) from y = RN(1/s) (Markstein): q = RN(|x|*y)
// is within one ulp of the quotient, the remainder |x| - q*s is exact in one
// FMA, and RN(q + rem*y) is the correctly rounded quotient.  Three VALU ops
// per element instead of a full division.  s is normal and positive and every
// quotient that can reach a non-zero E4M3 code is a normal fp32 number, as the
// method requires.  The clamped magnitude gets x's sign back (so -0 stays -0).
struct BlockDivisor {
  float s, y;
};
__device__ __forceinline__ BlockDivisor make_divisor(float s) {
  return {s, 1.0f / s};   // correctly rounded fp32 division, once per block
}
__device__ __forceinline__ float scaled(float x, BlockDivisor d) {
#pragma clang fp contract(off)
  const float a = fabsf(x);
  const float q = a * d.y;
  const float rem = __builtin_fmaf(-q, d.s, a);
  const float t = fminf(__builtin_fmaf(rem, d.y, q), kE4M3Max);
  return __builtin_copysignf(t, x);
}

// Four E4M3 codes, byte i from x_i.  The hardware conversion rounds to nearest
// even with E4M3 subnormals; it equals a bit-level RNE encoder on every fp32
// value of magnitude <= 448 (checked exhaustively on gfx950), so the codes are
// the method's.
__device__ __forceinline__ uint32_t quant4(float x0, float x1, float x2, float x3, BlockDivisor d) {
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(scaled(x0, d), scaled(x1, d), 0, false);
  v = __builtin_amdgcn_cvt_pk_fp8_f32(scaled(x2, d), scaled(x3, d), v, true);
  return (uint32_t)v;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Per-token mapping: a wave owns whole rows (grid-stride over rows); its four
// 16-lane groups walk the row's 128-element blocks with a stride of 4, so one
// pass reads 4 adjacent blocks (1 KB of bf16) per wave, and kUnroll passes are
// loaded before any is used to keep several 16-byte loads in flight per lane.
// No division in the index math.
constexpr int kUnroll = 4;

template <bool kF32>
__device__ __forceinline__ void load8(const void* src_row, int col, float (&x)[8]) {
  if constexpr (kF32) {
    const float* src = (const float*)src_row + col;
    const f32x4 v0 = *(const f32x4*)src;
    const f32x4 v1 = *(const f32x4*)(src + 4);
    x[0] = v0.x; x[1] = v0.y; x[2] = v0.z; x[3] = v0.w;
    x[4] = v1.x; x[5] = v1.y; x[6] = v1.z; x[7] = v1.w;
  } else {
    const u32x4 v = *(const u32x4*)((const uint16_t*)src_row + col);
    x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x); x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
    x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z); x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
  }
}

template <bool kF32>
__global__ void __launch_bounds__(256) per_token_cast_kernel(CastParams p) {
  const int lane16 = threadIdx.x & 15;
  const int grp = (threadIdx.x >> 4) & 3;
  const int kbs = (int)(p.k / 128);
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  for (int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); row < p.rows; row += nwaves) {
    const void* xrow = kF32 ? (const void*)((const float*)p.x + row * p.ldx)
                            : (const void*)((const uint16_t*)p.x + row * p.ldx);
    uint8_t* qrow = p.q + row * p.ldq;
    float* srow = p.sf + row * p.sf_s0;
    for (int kb0 = grp; kb0 < kbs; kb0 += 4 * kUnroll) {
      // every value below is uniform over the 16 lanes of a block
      float x[kUnroll][8];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        if (kb0 + 4 * u < kbs) load8<kF32>(xrow, (kb0 + 4 * u) * 128 + lane16 * 8, x[u]);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int kb = kb0 + 4 * u;
        if (kb >= kbs) break;
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[u][i]));
#pragma unroll
        for (int off = 8; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 16));
        const BlockDivisor d = make_divisor(block_scale(amax, p.ue8m0));
        u32x2 out;
        out.x = quant4(x[u][0], x[u][1], x[u][2], x[u][3], d);
        out.y = quant4(x[u][4], x[u][5], x[u][6], x[u][7], d);
        *(u32x2*)(qrow + kb * 128 + lane16 * 8) = out;
        if (lane16 == 0) srow[kb * p.sf_s1] = d.s;
      }
    }
  }
}

// One workgroup per 128x128 block: 16 lanes per row, 16 rows per pass, 8 passes.
__global__ void __launch_bounds__(256) per_block_cast_kernel(CastParams p) {
  const int64_t kbs = p.k / 128;
  const int64_t nb = blockIdx.x / kbs;
  const int64_t kb = blockIdx.x - nb * kbs;
  const int lane16 = threadIdx.x & 15;
  const int rsub = threadIdx.x >> 4;               // 0..15
  const int64_t col = kb * 128 + lane16 * 8;
  float x[8][8];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t row = nb * 128 + i * 16 + rsub;
    if (row < p.rows) {
      const float* src = (const float*)p.x + row * p.ldx + col;
      const f32x4 v0 = *(const f32x4*)src;
      const f32x4 v1 = *(const f32x4*)(src + 4);
      x[i][0] = v0.x; x[i][1] = v0.y; x[i][2] = v0.z; x[i][3] = v0.w;
      x[i][4] = v1.x; x[i][5] = v1.y; x[i][6] = v1.z; x[i][7] = v1.w;
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[i][j] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(x[i][j]));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  __shared__ float wave_max[4];
  if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wave_max[0], wave_max[1]), fmaxf(wave_max[2], wave_max[3]));
  const BlockDivisor d = make_divisor(block_scale(amax, p.ue8m0));
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t row = nb * 128 + i * 16 + rsub;
    if (row < p.rows) {
      u32x2 out;
      out.x = quant4(x[i][0], x[i][1], x[i][2], x[i][3], d);
      out.y = quant4(x[i][4], x[i][5], x[i][6], x[i][7], d);
      *(u32x2*)(p.q + row * p.ldq + col) = out;
    }
  }
  if (threadIdx.x == 0) p.sf[nb * p.sf_s0 + kb * p.sf_s1] = d.s;
}

// Packing of power-of-two scales into UE8M0 words: byte j of word (i, w) is
// the biased fp32 exponent of scale (i, 4w + j) rounded up to a power of two
// (the exponent plus one when any mantissa bit is set), 0 past the last K
// block.  One thread per word; a scale that already is a power of two keeps
// its exact value.  (Page "GitHub 推荐…DeepGEMM…", 可复用的模式与技巧: four
// UE8M0 exponents per int32, little-endian.)
__global__ void __launch_bounds__(256) pack_ue8m0_kernel(PackParams p) {
  const int64_t words = (p.kblocks + 3) / 4;
  const int64_t total = p.rows * words;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / words, w = i - r * words;
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t kb = 4 * w + j;
      if (kb < p.kblocks) {
        const uint32_t bits = __builtin_bit_cast(uint32_t, p.sf[r * p.sf_s0 + kb * p.sf_s1]);
        const uint32_t e = ((bits >> 23) & 0xFFu) + ((bits & 0x7FFFFFu) != 0u ? 1u : 0u);
        word |= (e & 0xFFu) << (8 * j);
      }
    }
    p.out[r * p.out_s0 + w * p.out_s1] = (int32_t)word;
  }
}

}  // namespace

hipError_t launch_pack_ue8m0(const PackParams& p, int num_cus, hipStream_t stream) {
  const int64_t total = p.rows * ((p.kblocks + 3) / 4);
  int64_t grid = (total + 255) / 256;
  const int64_t cap = (int64_t)num_cus * 16;
  if (grid > cap) grid = cap;
  hipLaunchKernelGGL(pack_ue8m0_kernel, dim3((unsigned)grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_per_token_cast(const CastParams& p, bool input_fp32, int num_cus, hipStream_t stream) {
  int64_t grid = (p.rows + 3) / 4;               // one row per wave
  const int64_t cap = (int64_t)num_cus * 32;    // grid-stride beyond 32 workgroups per CU
  if (grid > cap) grid = cap;
  if (input_fp32)
    hipLaunchKernelGGL(per_token_cast_kernel<true>, dim3((unsigned)grid), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(per_token_cast_kernel<false>, dim3((unsigned)grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_per_block_cast(const CastParams& p, hipStream_t stream) {
  const int64_t blocks = ((p.rows + 127) / 128) * (p.k / 128);
  hipLaunchKernelGGL(per_block_cast_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace dgfp8
