// Dense GEMM that allocates nothing: the split-K scratch (fp32 partial tiles
// and per-tile arrival counters) lives in a static device array of the library
// instead of a caller-provided workspace.  For callers that cannot call
// hipMalloc (code under HIP graph capture, tight serving loops, harnesses that
// forbid allocation).  The GEMM itself is dg_fp8_gemm_nt_ws: same plans, same
// kernels, same bits.
#include <mutex>

#include "dgfp8_internal.h"

#define DG_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

// 256 KiB of arrival counters (the workspace layout of dg_fp8_gemm_nt_ws)
// followed by 16 MiB of partial tiles.  Zero-initialised when the code object
// is loaded; every completed split-K call leaves the counters zero again.
constexpr size_t kCounterBytes = 256u << 10;
constexpr size_t kScratchBytes = kCounterBytes + (16u << 20);
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch_ptr[kMaxDevices] = {nullptr};

__global__ void __launch_bounds__(256) clear_words(uint32_t* p, int64_t words) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < words; i += (int64_t)gridDim.x * 256) p[i] = 0u;
}

// Device address of the current device's array.  The array's name is only a
// host-side handle: the address comes from hipGetSymbolAddress, called once
// per device with that device current, and is kept.  The counter block is
// cleared once, on the caller's stream, before the device's first use (a
// kernel rather than a memset, so the clear may also be captured in a graph).
dg_status scratch_for_current_device(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DG_ERROR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DG_ERROR_LAUNCH;
    hipLaunchKernelGGL(clear_words, dim3(64), dim3(256), 0, stream, static_cast<uint32_t*>(p),
                       (int64_t)(kCounterBytes / 4));
    if (hipGetLastError() != hipSuccess) return DG_ERROR_LAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DG_SUCCESS;
}

}  // namespace

DG_EXPORT dg_status dg_fp8_gemm_nt_noalloc(const void* a, int64_t lda, const float* sfa, int64_t sfa_sm,
                                           int64_t sfa_sk, const void* b, int64_t ldb, const float* sfb,
                                           int64_t sfb_sn, int64_t sfb_sk, void* d, int64_t ldd, int64_t m,
                                           int64_t n, int64_t k, void* stream) {
  // The plan the workspace entry point would run with a large enough
  // workspace; 0 when it does not split (or the sizes are invalid, which
  // dg_fp8_gemm_nt_ws then reports).
  const size_t need = dg_fp8_gemm_nt_workspace_size(m, n, k);
  if (need > kScratchBytes) return DG_ERROR_SCRATCH_LIMIT;
  void* ws = nullptr;
  if (need > 0) {
    const dg_status st = scratch_for_current_device(static_cast<hipStream_t>(stream), &ws);
    if (st != DG_SUCCESS) return st;
  }
  return dg_fp8_gemm_nt_ws(a, lda, sfa, sfa_sm, sfa_sk, b, ldb, sfb, sfb_sn, sfb_sk, d, ldd, m, n, k, ws,
                           need > 0 ? kScratchBytes : 0, stream);
}
