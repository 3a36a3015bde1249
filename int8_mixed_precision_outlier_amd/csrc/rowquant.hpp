// Device helpers of the activation quantization and the outlier gather
// used by the decode kernel (decode.hip): the outlier mask's per-word
// prefix counts and rank lookup, block reductions, the packed fp16 outlier
// layout, and the outlier weight source.
//
// Method: "LLM.int8() — 大模型激活值里藏着几个超大异常通道" (方法 1: one
// scale per row of X, 127 / absmax; 方法 2: the outlier columns leave for
// the fp16 path and are zero in the int8 row); developer.aliyun.com
// "LLM.int8()" 图2 (the outlier columns of X and rows of W gathered dense).
#pragma once

#include "common.hpp"
#include "launch.hpp"
#include "pack.hpp"

namespace i8mm {

// Exclusive prefix of the per-word outlier counts over the block: sm_pref[w]
// = outliers in words 0 .. w-1.  Each thread owns `per` consecutive words
// (already in sm_mask).  Returns the total.
template <int NT>
__device__ __forceinline__ int block_word_prefix(const uint32_t* sm_mask, int* sm_pref, int nwords,
                                                 int* sm_tmp) {
  constexpr int NW = NT / 64;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int per = (nwords + NT - 1) / NT;
  const int w0 = t * per;
  int local = 0;
  for (int i = 0; i < per; ++i)
    if (w0 + i < nwords) local += popc(sm_mask[w0 + i]);
  int x = local;
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  if (lane == 63) sm_tmp[wv] = x;
  __syncthreads();
  int before = 0, total = 0;
  for (int i = 0; i < NW; ++i) {
    if (i < wv) before += sm_tmp[i];
    total += sm_tmp[i];
  }
  int run = before + x - local;
  for (int i = 0; i < per; ++i) {
    if (w0 + i < nwords) {
      sm_pref[w0 + i] = run;
      run += popc(sm_mask[w0 + i]);
    }
  }
  __syncthreads();
  return total;
}

// Column of the outlier of rank r (0 <= r < total): the first word whose
// inclusive count exceeds r, then the (r - pref)-th set bit of that word.
__device__ __forceinline__ int select_rank(const uint32_t* sm_mask, const int* sm_pref, int nwords,
                                           int r) {
  int lo = 0, hi = nwords - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (sm_pref[mid] + popc(sm_mask[mid]) > r) hi = mid;
    else lo = mid + 1;
  }
  uint32_t m = sm_mask[lo];
  for (int j = r - sm_pref[lo]; j > 0; --j) m &= m - 1u;
  return lo * 32 + __builtin_ctz(m);
}

// Block-wide max of a uint32 over NT threads.
template <int NT>
__device__ __forceinline__ uint32_t block_max_nt(uint32_t v, uint32_t* sm) {
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t y = __shfl_xor(v, o, kWave);
    v = v > y ? v : y;
  }
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t r = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) r = r > sm[i] ? r : sm[i];
  return r;
}

// fp16 value e (0-15, not a compile-time constant) of a 16-value chunk held
// as two uint4: a select over the eight dwords, so the chunk stays in
// registers (indexing a local array with a run-time index would place it in
// scratch memory).
__device__ __forceinline__ uint16_t pick16(const uint4& a, const uint4& b, int e) {
  const uint32_t dw[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t d = dw[0];
#pragma unroll
  for (int u = 1; u < 8; ++u) d = (e >> 1) == u ? dw[u] : d;
  return (uint16_t)(d >> ((e & 1) * 16));
}

__device__ __forceinline__ uint16_t* out_elem16(uint16_t* P, int row, int t, int KBo) {
  return reinterpret_cast<uint16_t*>(reinterpret_cast<int8_t*>(P) + pack_offset(row, 2 * t, KBo));
}

// fp16 bits of outlier weight W[k][j] from the outlier source (the cache
// row when cached and valid, else the int8 weight dequantized).
__device__ __forceinline__ uint16_t out_weight(const OutlierSource& src, bool cache_ok, int n_dims,
                                               int k, int j, int N, int KB) {
  if (src.W) return src.W[(size_t)k * N + j];
  int sl = cache_ok ? src.slot[k] : -1;
  if (sl >= n_dims) sl = -1;
  if (sl >= 0) return src.rows[(size_t)sl * N + j];
  return f2h((float)src.Wi8[pack_offset(j, k, KB)] * (src.wabs[j] / 127.0f));
}

}  // namespace i8mm
