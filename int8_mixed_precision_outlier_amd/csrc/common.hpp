// Device-side helpers shared by the gfx950 kernels of the int8 mixed-precision
// outlier matmul.  Everything here is CDNA4-specific: 64-lane wavefronts and
// the gfx950 MFMA shapes 16x16x64 int8 -> int32 and 16x16x32 fp16 -> fp32.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace i8mm {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// fp16 bits -> fp32 (exact).
__device__ __forceinline__ float h2f(uint16_t b) {
  return __half2float(__ushort_as_half(b));
}

// fp32 -> fp16 bits, round to nearest even.
__device__ __forceinline__ uint16_t f2h(float f) {
  return __half_as_ushort(__float2half_rn(f));
}

// Quantization scale s = RN(127 / absmax), 0 for an all-zero vector.  Plain
// '/' is the correctly rounded IEEE division (no fast-math anywhere in this
// library).
__device__ __forceinline__ float qscale(float absmax) {
  return absmax > 0.0f ? 127.0f / absmax : 0.0f;
}

// q = clamp(round-half-even(RN(x * s)), -127, 127).  rintf is v_rndne_f32.
__device__ __forceinline__ int quant1(float x, float s) {
  float p = x * s;
  float r = __builtin_rintf(p);
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return (int)r;
}

// The sixteen fp16 values of a 16-column chunk (two uint4) quantized with
// scale s into sixteen int8 (one uint4); columns whose bit is set in mb
// (outliers) are zero.  q = RNE(RN32(x * s)) is read as the low byte of the
// fp32 sum RN32(RN32(x * s) + 1.5 * 2^23): a sum in [2^23, 2^24) has unit
// spacing, so its rounding is the round-half-to-even of the product, and
// the low mantissa bits hold 2^22 + q, whose low byte is q in two's
// complement.  That needs |RN32(x * s)| < 2^22, and no clamp is needed: a
// non-outlier column has |x| <= absmax, so |x * s| <= 127 (1 + 2^-22) and
// q stays in [-127, 127] (s = 0 gives 0); an outlier column can exceed
// it and is masked.  Four instructions per value against ten for quant1.
__device__ __forceinline__ uint4 quant_chunk16(const uint4& a, const uint4& b, float s,
                                               uint32_t mb) {
#pragma clang fp contract(off)
  const uint32_t d[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t o[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint16_t h = (uint16_t)(d[2 * k + (e >> 1)] >> (16 * (e & 1)));
      const float p = h2f(h) * s;  // RN32(x * s), not fused with the sum below
      y[e] = __builtin_bit_cast(uint32_t, p + 12582912.0f);
    }
    o[k] = (y[0] & 0xffu) | ((y[1] & 0xffu) << 8) | ((y[2] & 0xffu) << 16) | (y[3] << 24);
  }
  if (mb) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t b4 = (mb >> (4 * k)) & 0xfu;  // bit e -> byte e
      o[k] &= ~(((b4 * 0x00204081u) & 0x01010101u) * 0xffu);
    }
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// Largest fp16 magnitude (as bits) among a 16-column chunk's columns whose
// bit in mb is clear, two columns per packed max.
__device__ __forceinline__ uint32_t absmax_chunk16(const uint4& a, const uint4& b, uint32_t mb) {
  const uint32_t d[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  u16x2 m = (u16x2)(0);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t b2 = (mb >> (2 * k)) & 3u;
    const uint32_t keep = ~((b2 & 1u) * 0xffffu | (b2 & 2u) * 0x7fff8000u);
    m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, d[k] & 0x7fff7fffu & keep));
  }
  return m.x > m.y ? (uint32_t)m.x : (uint32_t)m.y;
}

// 16x16x64 int8 MFMA: C[16][16] += A[16 rows][64 k] . B[16 cols][64 k]^T.
// Lane l supplies row/col (l % 16) and 16 consecutive k bytes of quarter
// (l / 16).  A and B use the same (lane, byte) -> k assignment, so any
// consistent permutation of k gives the same exact integer sum.  Register
// i of lane l holds C[row = 4*(l/16) + i][col = l%16].
__device__ __forceinline__ v4i mfma16_i8(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// 16x16x32 fp16 MFMA with fp32 accumulation; same lane convention, 8 fp16
// of k per lane.
__device__ __forceinline__ v4f mfma16_f16(v8h a, v8h b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int popc(uint32_t x) { return __builtin_popcount(x); }

// s_waitcnt immediate (gfx9 encoding) waiting only on vmcnt <= n (0..63);
// expcnt and lgkmcnt are left at their maxima.
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Workgroup barrier for kernels whose global->LDS DMA stays in flight across
// it: wait until at most `vm` of this wavefront's vector-memory operations
// are outstanding and its LDS operations are done, then s_barrier.
// (A __syncthreads() would wait for every DMA, because its release fence
// counts them as pending LDS writes.)  The empty asm statements keep the
// compiler from moving memory accesses across the barrier.
// LGKM: LDS operations that may stay outstanding (the last ones issued,
// which must not read anything the barrier is meant to release).
template <int VM, int LGKM = 0>
__device__ __forceinline__ void barrier_vm() {
  static_assert(VM >= 0 && VM < 64 && LGKM >= 0 && LGKM < 16, "waitcnt fields");
  constexpr int imm = (VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (LGKM << 8);
  __builtin_amdgcn_s_waitcnt(imm);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Direct global->LDS load of 16 bytes per lane through a buffer descriptor:
// lane i's bytes (from voff + soff, soff wave-uniform) land at lds + 16 * i
// (lds must be wave-uniform).  A descriptor with a record count of 0 makes
// every lane out of range, which writes zeros.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           voff, soff, 0, 0);
}

// The same with 4 bytes per lane (lane i's dword lands at lds + 4 * i);
// out-of-range dwords read as zero one by one.
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, void* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4,
                                           voff, soff, 0, 0);
}

// Workgroups are dispatched to the 8 XCDs round-robin (workgroup b runs on
// XCD b % 8).  This bijection on [0, T) gives each XCD one contiguous range
// of logical indices, so neighbouring tiles/rows share an L2.
__device__ __forceinline__ int xcd_remap(int b, int T) {
  const int q = T >> 3, r = T & 7, x = b & 7;
  return x * q + (x < r ? x : r) + (b >> 3);
}

// Block-wide max of a uint32 over blockDim.x threads (multiple of 64).
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* sm) {
  for (int o = 32; o > 0; o >>= 1) {
    uint32_t w = __shfl_xor(v, o, kWave);
    v = v > w ? v : w;
  }
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) sm[wv] = v;
  __syncthreads();
  uint32_t r = 0;
  const int nw = blockDim.x >> 6;
  for (int i = 0; i < nw; ++i) r = r > sm[i] ? r : sm[i];
  return r;
}

}  // namespace i8mm
