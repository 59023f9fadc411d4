// Device helpers shared by the GEMM kernels: vector types, direct-to-LDS
// loads, the LDS row swizzle and fragment reads, LDS-only barriers, bf16
// packing, and the split of a scale into the MFMA's E8M0 exponent and a
// mantissa applied to the accumulator.
#pragma once

#include <utility>

#include "dgfp8_internal.h"

namespace dgfp8 {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define DG_GAS __attribute__((address_space(1)))
#define DG_LAS __attribute__((address_space(3)))

constexpr int kKBlock = 128;      // width of a scale block along K == K of one MFMA

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// s_waitcnt immediate (gfx9 encoding): vmcnt <= VM, lgkmcnt == 0, expcnt unconstrained.
template <int VM>
struct WaitVmLgkm0 {
  static constexpr int value = (VM & 0xF) | ((VM >> 4) << 14) | (0x7 << 4) | (0x0 << 8);
};

// 16-byte slot permutation of an LDS row.  Depends on the row's low 4 bits only,
// so every 16-row fragment sees the same per-lane pattern (reads use immediate
// offsets) and its 16 reads of one logical slot hit 16 distinct (bank-half, slot)
// pairs: conflict-free whether the LDS serves 8 or 16 lanes per cycle.
__device__ __forceinline__ int swz16(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// Direct-to-LDS loads.  Issued as inline asm so that the compiler's wait-count
// pass does not track them (it merges DMA histories conservatively at loop
// headers and would wait for every DMA before each LDS read); the kernel waits
// for them explicitly with s_waitcnt vmcnt.  No register is written by these
// instructions: the data goes to LDS at M0 + 16 * lane (resp. 4 * lane).  M0
// is an input operand of the asm, so the compiler sets it and knows its value.
__device__ __forceinline__ uint32_t lds_addr(const DG_LAS void* p) {
  return (uint32_t)(uintptr_t)p;
}
// Wave-uniform value the compiler may not prove uniform (it is carried across
// tiles in a loop): read it from the first active lane into scalar registers.
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const uint8_t*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ void dma16(const uint8_t* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(uniform_ptr(sbase)), "{m0}"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
}
__device__ __forceinline__ void dma4(const float* vaddr, uint32_t lds) {
  asm volatile("global_load_lds_dword %0, off"
               :: "v"(vaddr), "{m0}"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
}

// Workgroup barrier that orders LDS accesses only (lgkmcnt), leaving DMA and
// other vector-memory counters alone.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Two 16-byte LDS reads of a fragment (offsets of this lane's two slots).
__device__ __forceinline__ i32x8 read_frag(DG_LAS uint8_t* base, uint32_t off0, uint32_t off1) {
  const i32x4 lo = *(DG_LAS i32x4*)(base + off0);
  const i32x4 hi = *(DG_LAS i32x4*)(base + off1);
  return (i32x8){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
}

constexpr int kBRowScaleE8M0 = 127 - 63;   // 2^-63 on the B-row port (fp32-scale kernels)

// Raw buffer descriptors (word 3 of the resource: 32-bit data, no swizzle) and
// the cache-policy operand of buffer accesses that are coherent device-wide.
constexpr int kRawBufferFlags = 0x00020000;
constexpr int kScopeDevice = 16;   // sc1

__device__ __forceinline__ int scale_exponent(float s) {
  return (int)((__builtin_bit_cast(uint32_t, s) >> 23) & 0xFFu);
}
__device__ __forceinline__ float scale_mantissa(float s) {
  return __builtin_bit_cast(float, (__builtin_bit_cast(uint32_t, s) & 0x807FFFFFu) | 0x3F800000u);
}

// acc *= s, component by component: a splat of s would let the optimizer
// widen the scalar load of s into a vector load over its neighbours, which
// pins the ratio array in scratch memory.
__device__ __forceinline__ void rescale(f32x4& a, float s) {
  a.x *= s;
  a.y *= s;
  a.z *= s;
  a.w *= s;
}

// Compile-time loop: f(std::integral_constant<int, I>) for I = I0 .. N-1.
template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

}  // namespace dgfp8
