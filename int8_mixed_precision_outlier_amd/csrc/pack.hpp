// Packed int8 layout shared by the quantizers (producers) and the GEMM and
// decode kernels (consumers).
//
// An R x K int8 matrix is stored in blocks of 16 rows x 64 k-bytes (1 KB),
// K zero-padded to a multiple of 64.  Blocks are ordered row-block major:
// block (rb, kb) starts at byte (rb * KB + kb) * 1024, KB = K_pad / 64.
// Inside a block the four 16-byte k-chunks are stored chunk-major: byte
// (r, k) of the block sits at ((k / 16) * 16 + r) * 16 + k % 16.
//
// Why: one 1 KB block is exactly one 64-lane x 16-byte load, so a
// global->LDS DMA instruction reads contiguous whole cache lines, and it is
// exactly one operand of a 16x16x64 int8 MFMA (lane l takes row l % 16 and
// k-chunk l / 16), read as 1 KB of contiguous LDS or global bytes:
// conflict-free without any swizzle.  Decode streams each 16-row block as
// one contiguous run along K.
#pragma once

#include <stdint.h>

namespace i8mm {

constexpr int kPackRows = 16;   // rows per block
constexpr int kPackK = 64;      // k-bytes per block
constexpr int kPackBlock = 1024;

__host__ __device__ __forceinline__ int64_t pack_kpad(int64_t K) { return (K + 63) / 64 * 64; }
__host__ __device__ __forceinline__ int64_t pack_rpad(int64_t R) { return (R + 15) / 16 * 16; }

// byte offset of element (row, k); KB = K_pad / 64
__host__ __device__ __forceinline__ int64_t pack_offset(int64_t row, int64_t k, int64_t KB) {
  return ((row >> 4) * KB + (k >> 6)) * kPackBlock + (((k >> 4) & 3) * 16 + (row & 15)) * 16 +
         (k & 15);
}

}  // namespace i8mm
