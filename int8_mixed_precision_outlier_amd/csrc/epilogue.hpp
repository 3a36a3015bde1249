// Fused epilogue pieces of the tiled prefill GEMM for one 16x16 output
// block: dequantization, fp16 store and int32 store (the operands are
// staged in LDS by the GEMM itself).
//
// The int8 MFMA runs with the weight tile as the "A" operand (MFMA rows = n,
// output features) and the activation tile as "B" (MFMA columns = m,
// tokens), i.e. it produces Y^T blocks.  Register e of lane l then holds
// feature nb + 4*(l/16) + e of token mb + l%16, so the fp16 result leaves
// as 8-byte stores along the rows of Y.
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

// Store an int32 accumulator block (the Out_i32 export).  N % 16 == 0, so
// a lane's four features are all in range or all out.
__device__ __forceinline__ void store16_i32(const v4i& acc, int nb, int mb, int M, int N,
                                            int32_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int m = mb + (lane & 15), n = nb + 4 * (lane >> 4);
  if (m < M && n < N) *reinterpret_cast<v4i*>(out + (size_t)m * N + n) = acc;
}

// y = fp32(acc) * rx * (w/127) (+ bias when the layer has one), for the
// lane's four features (w, b) of token rx
__device__ __forceinline__ v4f dequant16(const v4i& acc, float rx, const float4& w, const uint2& b,
                                         bool has_bias) {
  v4f y;
  y[0] = (float)acc[0] * rx * (w.x / 127.0f);
  y[1] = (float)acc[1] * rx * (w.y / 127.0f);
  y[2] = (float)acc[2] * rx * (w.z / 127.0f);
  y[3] = (float)acc[3] * rx * (w.w / 127.0f);
  if (has_bias) {
    y[0] += h2f((uint16_t)(b.x & 0xffffu));
    y[1] += h2f((uint16_t)(b.x >> 16));
    y[2] += h2f((uint16_t)(b.y & 0xffffu));
    y[3] += h2f((uint16_t)(b.y >> 16));
  }
  return y;
}

__device__ __forceinline__ void store16_f16(const v4f& y, int nb, int mb, int M, int N,
                                            uint16_t* __restrict__ Y) {
  const int lane = threadIdx.x & 63;
  const int m = mb + (lane & 15), n = nb + 4 * (lane >> 4);
  if (m < M && n < N) {
    const uint32_t lo = (uint32_t)f2h(y[0]) | ((uint32_t)f2h(y[1]) << 16);
    const uint32_t hi = (uint32_t)f2h(y[2]) | ((uint32_t)f2h(y[3]) << 16);
    *reinterpret_cast<uint2*>(Y + (size_t)m * N + n) = make_uint2(lo, hi);
  }
}

}  // namespace i8mm
