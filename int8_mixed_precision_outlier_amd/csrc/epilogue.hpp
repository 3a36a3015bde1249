// Fused epilogue pieces of the tiled prefill GEMM for one 32x32 output
// block: dequantization, fp16 store and int32 store (the operands are
// staged in LDS by the GEMM itself).
//
// The int8 MFMA runs with the weight tile as the "A" operand (MFMA rows = n,
// output features) and the activation tile as "B" (MFMA columns = m,
// tokens), i.e. it produces Y^T blocks.  Lane l then owns token m = mb + l%32
// and, per group of four registers, four consecutive output features, so the
// fp16 result leaves as 8-byte stores along the rows of Y.
//
// Per element (developer.aliyun.com "LLM.int8()" 图2, Jason's Study 方法 1/2):
//   y = fp32(Out_i32) * (x_absmax[m]/127) * (w_absmax[n]/127)   dequantize
//   y += bias[n]                              when the layer has a bias
//   y += sum_t X_out[m][t] * W_out[t][n]     fp16 MFMA, fp32 accumulation
//   Y[m][n] = fp16_rne(y)
//
// X_out and W_out^T are fp16 matrices in the packed layout of pack.hpp over
// bytes (an fp16 row of n_cap values is a 2*n_cap-byte packed row), so a
// 64-byte block holds 32 outlier columns and a 16-byte chunk 8 of them.
#pragma once

#include "common.hpp"
#include "launch.hpp"
#include "pack.hpp"

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

// y = fp32(acc) * rx * (w/127) (+ bias when the layer has one)
__device__ __forceinline__ v16f dequant(const v16i& acc, float rx, const float4 (&w)[4],
                                        const uint2 (&b)[4], bool has_bias) {
  v16f y;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    y[4 * g + 0] = (float)acc[4 * g + 0] * rx * (w[g].x / 127.0f);
    y[4 * g + 1] = (float)acc[4 * g + 1] * rx * (w[g].y / 127.0f);
    y[4 * g + 2] = (float)acc[4 * g + 2] * rx * (w[g].z / 127.0f);
    y[4 * g + 3] = (float)acc[4 * g + 3] * rx * (w[g].w / 127.0f);
    if (has_bias) {
      y[4 * g + 0] += h2f((uint16_t)(b[g].x & 0xffffu));
      y[4 * g + 1] += h2f((uint16_t)(b[g].x >> 16));
      y[4 * g + 2] += h2f((uint16_t)(b[g].y & 0xffffu));
      y[4 * g + 3] += h2f((uint16_t)(b[g].y >> 16));
    }
  }
  return y;
}

__device__ __forceinline__ void store_f16(const v16f& y, int nb, int mb, int M, int N,
                                          uint16_t* __restrict__ Y) {
  const int lane = threadIdx.x & 63;
  const int m = mb + (lane & 31);
  if (m >= M) return;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int n = nb + g * 8 + (lane >> 5) * 4;
    if (n < N) {
      const uint32_t lo = (uint32_t)f2h(y[4 * g]) | ((uint32_t)f2h(y[4 * g + 1]) << 16);
      const uint32_t hi = (uint32_t)f2h(y[4 * g + 2]) | ((uint32_t)f2h(y[4 * g + 3]) << 16);
      *reinterpret_cast<uint2*>(Y + (size_t)m * N + n) = make_uint2(lo, hi);
    }
  }
}

}  // namespace i8mm
