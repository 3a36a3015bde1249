// Fused epilogue pieces of the tiled prefill GEMM for one 16x16 output
// block: dequantization, fp16 store and int32 store (the operands are
// staged in LDS by the GEMM itself).
//
// The int8 MFMA runs with the weight tile as the "A" operand (MFMA rows = n,
// output features) and the activation tile as "B" (MFMA columns = m,
// tokens), i.e. it produces Y^T blocks.  Register e of lane l then holds
// feature nb + 4*(l/16) + e of token mb + l%16; two blocks of adjacent
// features leave together as 16-byte stores along the rows of Y.
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

// y = fp32(acc) * (rx * sw) + b for the lane's four features: rx =
// x_absmax/127 of its token, sw = w_absmax/127 and b the bias of the
// features (zeros when the layer has none).  One product and one fma per
// element; the scales are taken as a product with 1/127 rather than a
// quotient (a few fp32 ulps, far inside the output's fp16 rounding).
__device__ __forceinline__ v4f dequant16(const v4i& acc, float rx, const float4& sw,
                                         const float4& b) {
  v4f y;
  y[0] = fmaf((float)acc[0], rx * sw.x, b.x);
  y[1] = fmaf((float)acc[1], rx * sw.y, b.y);
  y[2] = fmaf((float)acc[2], rx * sw.z, b.z);
  y[3] = fmaf((float)acc[3], rx * sw.w, b.w);
  return y;
}

// Two fp32 values as packed fp16, round to nearest even (one
// v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const h2 h = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, h);
}

// Two 16x16 blocks of adjacent features (nb .. nb+15 in ya, nb+16 .. +31
// in yb) for the same 16 tokens, as one 16-byte store per lane.  In a
// block, lanes 16q .. 16q+15 (row q of the wavefront) hold features
// 4q .. 4q+3 of tokens 0-15.  v_permlane16_swap exchanges rows 1 and 3 of
// its first operand with rows 0 and 2 of its second, so with ya first
// and yb second, row q of the lanes then holds 8 consecutive features of
// one token: 0-7 (q = 0) and 8-15 (q = 2) of ya, 0-7 (q = 1) and 8-15
// (q = 3) of yb.  Each token's 64 bytes go out in one instruction as four
// 16-byte pieces, against 32-byte pieces from two instructions.  N % 16
// == 0, so a lane's 8 features are all in range or all out.
__device__ __forceinline__ void store32_f16(const v4f& ya, const v4f& yb, int nb, int mb, int M,
                                            int N, uint16_t* __restrict__ Y) {
  const int lane = threadIdx.x & 63, q = lane >> 4;
  const auto lo = __builtin_amdgcn_permlane16_swap(pack_f16x2(ya[0], ya[1]),
                                                   pack_f16x2(yb[0], yb[1]), false, false);
  const auto hi = __builtin_amdgcn_permlane16_swap(pack_f16x2(ya[2], ya[3]),
                                                   pack_f16x2(yb[2], yb[3]), false, false);
  const int m = mb + (lane & 15), n = nb + 8 * (q >> 1) + 16 * (q & 1);
  if (m < M && n < N)
    *reinterpret_cast<uint4*>(Y + (size_t)m * N + n) = make_uint4(lo[0], hi[0], lo[1], hi[1]);
}

// One 16x16 block alone (a tile whose wavefront holds an odd number of
// feature blocks): each lane stores its four features of one token as 8
// bytes.  N % 16 == 0, so the four are all in range or all out.
__device__ __forceinline__ void store16_f16(const v4f& y, int nb, int mb, int M, int N,
                                            uint16_t* __restrict__ Y) {
  const int lane = threadIdx.x & 63;
  const int m = mb + (lane & 15), n = nb + 4 * (lane >> 4);
  if (m < M && n < N)
    *reinterpret_cast<uint2*>(Y + (size_t)m * N + n) =
        make_uint2(pack_f16x2(y[0], y[1]), pack_f16x2(y[2], y[3]));
}

}  // namespace i8mm
