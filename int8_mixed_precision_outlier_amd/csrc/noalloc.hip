// int8_mixed_matmul_noalloc: the decomposed matmul for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving
// loops).  Its workspace is a file-scope device array of fixed size that
// every GPU the library runs on holds until the process ends; the kernels
// are int8_mixed_matmul's, on the same workspace layout.
//
// The array's host-side name is only a stand-in for the symbol, never a
// device address: the address is taken once per device with
// hipGetSymbolAddress (each GPU holds its own copy at its own address) and
// only that address is handed to the kernels.
#include "../../include/int8mm.h"
#include "api_internal.hpp"

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

namespace {

constexpr size_t kScratchBytes = INT8MM_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The device address of `scratch` on the current device (looked up on the
// first call on that device, with it current).
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

extern "C" int int8_mixed_matmul_noalloc(const void* X_f16, int64_t M, int64_t K,
                                         const int8_t* W_i8, const float* w_absmax,
                                         const void* W_f16, int64_t N, float alpha,
                                         const void* bias_f16, void* Y_f16, int64_t n_cap,
                                         hipStream_t stream) {
  const size_t need = int8_mixed_matmul_workspace_size(M, K, N, n_cap, nullptr);
  if (need == 0) return INT8MM_EINVAL;  // shape or capacity out of range
  if (need > kScratchBytes) return INT8MM_ESCRATCH;
  if (!W_f16 && K > 0 && M > 0 && N > 0) return INT8MM_EINVAL;
  if (M == 0 || N == 0) return INT8MM_OK;
  void* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return i8mm::hip_error_status(e);
  return i8mm::run_mixed(X_f16, M, K, W_i8, w_absmax, W_f16, nullptr, N, alpha, bias_f16, Y_f16,
                         ws, kScratchBytes, n_cap, stream);
}
