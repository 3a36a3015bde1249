// Peak probes (include/int8mm_probes.h): an MFMA-only loop and a streaming
// read, for the measured ceilings the matmul kernels are compared with.
// Not part of the matmul; built into its own library.
#include "../../include/int8mm_probes.h"
#include "common.hpp"

namespace i8mm {

// Eight MFMAs per iteration on four accumulator chains.  RANDOM: the lane's
// eight A and eight B fragments are distinct, consecutive MFMAs use
// different ones; otherwise all use fragment 0.
template <bool RANDOM>
__global__ __launch_bounds__(256) void k_probe_mfma(const int8_t* __restrict__ ops, int64_t iters,
                                                    int32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  v4i a[8], b[8];
#pragma unroll
  for (int f = 0; f < 8; ++f) {
    const int g = RANDOM ? f : 0;
    a[f] = *reinterpret_cast<const v4i*>(ops + g * 1024 + lane * 16);
    b[f] = *reinterpret_cast<const v4i*>(ops + ((g + 3) & 7) * 1024 + lane * 16);
  }
  v4i acc[4] = {v4i{}, v4i{}, v4i{}, v4i{}};
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u & 3] = mfma16_i8(a[u], b[(u * 3) & 7], acc[u & 3]);
  }
  int32_t s = 0;
#pragma unroll
  for (int c = 0; c < 4; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  sink[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// The fp16 counterpart: v_mfma_f32_16x16x32_f16 (the outlier product's
// instruction), same loop shape; the operand buffer holds 8 KB of fp16
// values (the driver fills it with random halves of moderate magnitude).
template <bool RANDOM>
__global__ __launch_bounds__(256) void k_probe_mfma_f16(const int8_t* __restrict__ ops,
                                                        int64_t iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  v8h a[8], b[8];
#pragma unroll
  for (int f = 0; f < 8; ++f) {
    const int g = RANDOM ? f : 0;
    a[f] = *reinterpret_cast<const v8h*>(ops + g * 1024 + lane * 16);
    b[f] = *reinterpret_cast<const v8h*>(ops + ((g + 3) & 7) * 1024 + lane * 16);
  }
  v4f acc[4] = {v4f{}, v4f{}, v4f{}, v4f{}};
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u & 3] = mfma16_f16(a[u], b[(u * 3) & 7], acc[u & 3]);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < 4; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  sink[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

template <bool NT>
__global__ __launch_bounds__(256) void k_probe_read(const v4i* __restrict__ buf, int64_t n16,
                                                    uint32_t* __restrict__ sink) {
  __shared__ uint32_t red[4];
  const int64_t stride = (int64_t)gridDim.x * 256;
  uint32_t x = 0;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    v4i v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      v[u] = NT ? __builtin_nontemporal_load(buf + i + u * stride) : buf[i + u * stride];
#pragma unroll
    for (int u = 0; u < 4; ++u) x ^= (uint32_t)(v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3]);
  }
  for (; i < n16; i += stride) {
    const v4i v = buf[i];
    x ^= (uint32_t)(v[0] ^ v[1] ^ v[2] ^ v[3]);
  }
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o, kWave);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

}  // namespace i8mm

extern "C" int int8mm_probe_mfma_i8(const int8_t* operands, int random, int64_t blocks,
                                    int64_t iters, int32_t* sink, hipStream_t stream) {
  if (!operands || !sink || blocks <= 0 || blocks > (1 << 20) || iters < 0)
    return (int)hipErrorInvalidValue;
  if (random)
    i8mm::k_probe_mfma<true><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(operands, iters, sink);
  else
    i8mm::k_probe_mfma<false><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(operands, iters, sink);
  return (int)hipGetLastError();
}

extern "C" int int8mm_probe_mfma_f16(const void* operands, int random, int64_t blocks,
                                     int64_t iters, float* sink, hipStream_t stream) {
  if (!operands || !sink || blocks <= 0 || blocks > (1 << 20) || iters < 0)
    return (int)hipErrorInvalidValue;
  const int8_t* ops = static_cast<const int8_t*>(operands);
  if (random)
    i8mm::k_probe_mfma_f16<true><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(ops, iters, sink);
  else
    i8mm::k_probe_mfma_f16<false><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(ops, iters, sink);
  return (int)hipGetLastError();
}

extern "C" int int8mm_probe_read(const void* buf, size_t bytes, int nontemporal, int64_t blocks,
                                 uint32_t* sink, hipStream_t stream) {
  if (!buf || !sink || bytes % 16 != 0 || blocks <= 0 || blocks > (1 << 20))
    return (int)hipErrorInvalidValue;
  const int64_t n16 = (int64_t)(bytes / 16);
  const i8mm::v4i* p = static_cast<const i8mm::v4i*>(buf);
  if (nontemporal)
    i8mm::k_probe_read<true><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(p, n16, sink);
  else
    i8mm::k_probe_read<false><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(p, n16, sink);
  return (int)hipGetLastError();
}
