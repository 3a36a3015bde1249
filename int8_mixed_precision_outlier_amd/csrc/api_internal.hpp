// Host-side pieces of the C-ABI layer shared between its source files.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace i8mm {

// The whole decomposed matmul on a caller-given workspace: argument checks,
// then detection, quantization + gather and the GEMM (or decode) kernel,
// all enqueued on `stream`.  Exactly one of W_f16 and cache is non-null
// (unless the call is a no-op).  Returns an int8mm_status.
int run_mixed(const void* X_f16, int64_t M, int64_t K, const int8_t* W_i8,
              const float* w_absmax, const void* W_f16, const void* cache, int64_t N,
              float alpha, const void* bias_f16, void* Y_f16, void* workspace,
              size_t workspace_bytes, int64_t n_cap, hipStream_t stream);

// INT8MM_OK for hipSuccess; otherwise records the error for
// int8mm_last_hip_error and returns INT8MM_EHIP.
int hip_error_status(hipError_t e);

}  // namespace i8mm
