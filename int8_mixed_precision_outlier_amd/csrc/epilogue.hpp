// Fused epilogue of one 32x32 output block, shared by the tiled prefill GEMM
// and the decode kernel.
//
// The int8 MFMA runs with the weight tile as the "A" operand (MFMA rows = n,
// output features) and the activation tile as "B" (MFMA columns = m,
// tokens), i.e. it produces Y^T blocks.  Lane l then owns token m = mb + l%32
// and, per group of four registers, four consecutive output features, so the
// fp16 result leaves as 8-byte stores along the rows of Y.
//
// Per element (developer.aliyun.com "LLM.int8()" 图2, Jason's Study 方法 1/2):
//   y = fp32(Out_i32) * (x_absmax[m]/127) * (w_absmax[n]/127)   dequantize
//   y += sum_t X_out[m][t] * W_out[t][n]     fp16 MFMA, fp32 accumulation
//   Y[m][n] = fp16_rne(y)
#pragma once

#include "common.hpp"
#include "launch.hpp"

namespace i8mm {

// Store an int32 accumulator block (the Out_i32 export).
__device__ __forceinline__ void store_block_i32(const v16i& acc, int nb, int mb, int M, int N,
                                                int32_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int m = mb + (lane & 31);
  if (m >= M) return;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int n = nb + g * 8 + (lane >> 5) * 4;
    if (n < N) {
      int4 v = make_int4(acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]);
      *reinterpret_cast<int4*>(out + (size_t)m * N + n) = v;
    }
  }
}

// Dequantize, add the outlier product and store fp16.  Must be called by all
// 64 lanes of the wavefront (the MFMA is wave-wide); n16 is wave-uniform.
__device__ __forceinline__ void store_block_f16(const v16i& acc, int nb, int mb, int M, int N,
                                                int n16, const Epilogue& e) {
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5;
  const int m = mb + (lane & 31);
  const float rx = (m < M) ? e.xabs[m] / 127.0f : 0.0f;
  v16f y;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int n = nb + g * 8 + h * 4;
    float4 w = make_float4(0.f, 0.f, 0.f, 0.f);
    if (n < N) w = *reinterpret_cast<const float4*>(e.wabs + n);
    y[4 * g + 0] = (float)acc[4 * g + 0] * rx * (w.x / 127.0f);
    y[4 * g + 1] = (float)acc[4 * g + 1] * rx * (w.y / 127.0f);
    y[4 * g + 2] = (float)acc[4 * g + 2] * rx * (w.z / 127.0f);
    y[4 * g + 3] = (float)acc[4 * g + 3] * rx * (w.w / 127.0f);
  }
  if (n16 > 0) {
    const int nr = nb + (lane & 31);
    const bool nok = nr < N, mok = m < M;
    const uint16_t* wrow = e.WoutT + (size_t)nr * n16 + h * 8;
    const uint16_t* xrow = e.Xout + (size_t)m * n16 + h * 8;
    for (int t0 = 0; t0 < n16; t0 += 16) {
      v8h a = {}, b = {};
      if (nok) a = *reinterpret_cast<const v8h*>(wrow + t0);
      if (mok) b = *reinterpret_cast<const v8h*>(xrow + t0);
      y = mfma_f16(a, b, y);
    }
  }
  if (m < M) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int n = nb + g * 8 + h * 4;
      if (n < N) {
        const uint32_t lo = (uint32_t)f2h(y[4 * g]) | ((uint32_t)f2h(y[4 * g + 1]) << 16);
        const uint32_t hi = (uint32_t)f2h(y[4 * g + 2]) | ((uint32_t)f2h(y[4 * g + 3]) << 16);
        *reinterpret_cast<uint2*>(e.Y + (size_t)m * N + n) = make_uint2(lo, hi);
      }
    }
  }
  // keep the scheduler from hoisting the next block's loads above this one
  // (with 256 accumulator registers live that would spill)
  __builtin_amdgcn_sched_barrier(0);
}

}  // namespace i8mm
