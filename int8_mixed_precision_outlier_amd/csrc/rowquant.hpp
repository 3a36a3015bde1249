// Device helpers of the activation quantization and the outlier gather,
// shared by the small-M row quantizer (prologue.hip) and the decode kernel
// (decode.hip): the outlier mask's per-word prefix counts and rank lookup,
// block reductions, the packed fp16 outlier layout, the outlier weight
// source, and the quantization of one row by one workgroup.
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

// The row quantization of the decomposition for one row held by a
// workgroup of NT threads: row absmax over the non-outlier columns (mask and
// its prefix counts in LDS), int8 row with the outlier columns zeroed, and
// the row's outlier values at their ranks.  Chunks of 16 columns; a thread
// keeps up to CPT chunks in registers (loaded by row_load) between the
// absmax and the quantization (a longer row is read twice).  The int8 row
// goes to
// q_out(c, uint4) for every chunk c < 4*KB (zeros past the data), the
// outliers to o_out(rank, column, fp16 bits) for ranks < n.  Returns the
// row absmax.
// The chunks a thread keeps in registers (row_load, issued early so their
// latency overlaps the mask setup), then the quantization proper.
template <int NT, int CPT>
__device__ __forceinline__ void row_load(const uint16_t* __restrict__ xr, int K, uint4 (&v)[CPT][2]) {
  const int t = threadIdx.x, nchunks = K >> 4;
  if (nchunks > NT * CPT) return;  // too long to keep: quantize_row reads it twice
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int c = t + j * NT;
    v[j][0] = v[j][1] = make_uint4(0, 0, 0, 0);
    if (c < nchunks) {
      v[j][0] = *reinterpret_cast<const uint4*>(xr + 16 * c);
      v[j][1] = *reinterpret_cast<const uint4*>(xr + 16 * c + 8);
    }
  }
}

template <int NT, int CPT, class QOut, class OOut>
__device__ __forceinline__ float quantize_row(const uint16_t* __restrict__ xr, int K, int KB,
                                              const uint4 (&v)[CPT][2], const uint32_t* sm_mask,
                                              const int* sm_pref, int n, uint32_t* sm_red,
                                              QOut q_out, OOut o_out) {
  const int t = threadIdx.x;
  const int nchunks = K >> 4, pchunks = KB * 4;
  const bool cached = nchunks <= NT * CPT;
  auto chunk_max = [&](const uint4& d0, const uint4& d1, int c, uint32_t amax) {
    // an outlier column's magnitude is masked to 0
    const uint32_t mb = (sm_mask[c >> 1] >> ((c & 1) * 16)) & 0xffffu;
    return max(amax, absmax_chunk16(d0, d1, mb));
  };
  uint32_t amax = 0;
  if (cached) {
#pragma unroll
    for (int j = 0; j < CPT; ++j)
      if (t + j * NT < nchunks) amax = chunk_max(v[j][0], v[j][1], t + j * NT, amax);
  } else {
    for (int c = t; c < nchunks; c += NT)
      amax = chunk_max(*reinterpret_cast<const uint4*>(xr + 16 * c),
                       *reinterpret_cast<const uint4*>(xr + 16 * c + 8), c, amax);
  }
  amax = block_max_nt<NT>(amax, sm_red);
  const float ax = h2f((uint16_t)amax);
  const float s = qscale(ax);
  auto chunk_quant = [&](const uint4& d0, const uint4& d1, int c) {
    uint4 qv = make_uint4(0u, 0u, 0u, 0u);
    if (c < nchunks) {
      const uint32_t word = sm_mask[c >> 1];
      const uint32_t mb = (word >> ((c & 1) * 16)) & 0xffffu;
      // every element quantized, outlier columns then masked to 0
      qv = quant_chunk16(d0, d1, s, mb);
      // the chunk's outlier columns (almost always none), each to its rank
      for (uint32_t bits = mb; bits; bits &= bits - 1u) {
        const int e = __builtin_ctz(bits);
        const int r = sm_pref[c >> 1] + popc(word & ((1u << ((c & 1) * 16 + e)) - 1u));
        if (r < n) o_out(r, 16 * c + e, pick16(d0, d1, e));
      }
    }
    q_out(c, qv);
  };
  const uint4 z = make_uint4(0, 0, 0, 0);
  if (cached) {
#pragma unroll
    for (int j = 0; j < CPT; ++j)
      if (t + j * NT < pchunks) chunk_quant(v[j][0], v[j][1], t + j * NT);
    for (int c = t + CPT * NT; c < pchunks; c += NT) chunk_quant(z, z, c);  // padding only
  } else {
    for (int c = t; c < pchunks; c += NT) {
      if (c < nchunks)
        chunk_quant(*reinterpret_cast<const uint4*>(xr + 16 * c),
                    *reinterpret_cast<const uint4*>(xr + 16 * c + 8), c);
      else
        chunk_quant(z, z, c);
    }
  }
  return ax;
}

}  // namespace i8mm
