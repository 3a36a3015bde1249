// Prologue kernels of the int8 mixed-precision outlier matmul (gfx950):
//   K0  weight quantization (offline): column absmax + quantize/transpose.
//   K1  outlier detection: column absmax of X, ballot into a bit mask (two
//       passes for large X).
//   K2  activation quantization: row absmax over non-outlier columns,
//       int8 rows with the outlier columns zeroed, and the dense fp16
//       outlier pair X_out / W_out^T (packed) gathered in ascending column
//       order, the weight rows from the fp16 W or from an outlier-row cache.
// Method: "LLM.int8() — 大模型激活值里藏着几个超大异常通道" (方法 1, 方法 2,
// 观察 2); developer.aliyun.com "LLM.int8()" §2.2 图2; brain.gartu.xyz
// "LLM.int8()" "Seuil de détection α" and "Vector-wise INT8 Quantization".
#include "common.hpp"
#include "launch.hpp"
#include "pack.hpp"
#include "rowquant.hpp"

#include <stdlib.h>

namespace i8mm {

// ---------------------------------------------------------------- K0
// Column absmax of W[K][N] (fp16).  One workgroup per 64-column strip;
// 256 threads = 32 row lanes x 8 column lanes of 8 fp16 (16 bytes).
__global__ __launch_bounds__(256) void k_weight_absmax(
    const uint16_t* __restrict__ W, int K, int N, float* __restrict__ aw) {
  __shared__ uint16_t red[32][64];
  const int t = threadIdx.x;
  const int cl = t & 7, rl = t >> 3;
  const int col = blockIdx.x * 64 + cl * 8;
  u16x2 m[4] = {0, 0, 0, 0};
  if (col < N) {
    const u16x2 msk = (u16x2)(0x7fff);
    for (int r = rl; r < K; r += 32) {
      uint4 v = *reinterpret_cast<const uint4*>(W + (size_t)r * N + col);
      m[0] = __builtin_elementwise_max(m[0], __builtin_bit_cast(u16x2, v.x) & msk);
      m[1] = __builtin_elementwise_max(m[1], __builtin_bit_cast(u16x2, v.y) & msk);
      m[2] = __builtin_elementwise_max(m[2], __builtin_bit_cast(u16x2, v.z) & msk);
      m[3] = __builtin_elementwise_max(m[3], __builtin_bit_cast(u16x2, v.w) & msk);
    }
  }
  for (int e = 0; e < 4; ++e) {
    red[rl][cl * 8 + 2 * e] = m[e].x;
    red[rl][cl * 8 + 2 * e + 1] = m[e].y;
  }
  __syncthreads();
  if (t < 64) {
    uint16_t mx = 0;
    for (int r = 0; r < 32; ++r) mx = red[r][t] > mx ? red[r][t] : mx;
    const int c = blockIdx.x * 64 + t;
    if (c < N) aw[c] = h2f(mx);
  }
}

// Quantize + transpose a 64(k) x 64(n) tile: W_i8[n][k] = q(W[k][n], s[n]),
// written in the packed layout (pack.hpp): the tile is one k-block of four
// 16-row blocks.  k past K (padding up to a multiple of 64) quantizes 0.
__global__ __launch_bounds__(256) void k_weight_quant(
    const uint16_t* __restrict__ W, int K, int N, const float* __restrict__ aw,
    int8_t* __restrict__ Wq, int KB) {
  __shared__ __align__(16) int8_t tile[64][64 + 16];
  __shared__ float sc[64];
  const int t = threadIdx.x;
  const int k0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  if (t < 64) sc[t] = (n0 + t < N) ? qscale(aw[n0 + t]) : 0.0f;
  __syncthreads();
  // load: 64 rows x 8 chunks of 8 fp16
  for (int q = t; q < 512; q += 256) {
    const int r = q >> 3, c = (q & 7) * 8;
    const int k = k0 + r, n = n0 + c;
    uint16_t h[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (k < K && n < N) {
      uint4 v = *reinterpret_cast<const uint4*>(W + (size_t)k * N + n);
      __builtin_memcpy(h, &v, 16);
    }
    for (int e = 0; e < 8; ++e) tile[c + e][r] = (int8_t)quant1(h2f(h[e]), sc[c + e]);
  }
  __syncthreads();
  // store: thread t -> row block t/64, k-chunk (t/16)%4, row t%16 (16 bytes)
  const int rbl = t >> 6, c = (t >> 4) & 3, r = t & 15;
  const int n = n0 + rbl * 16 + r;
  if (n < N) {
    uint4 v;
    __builtin_memcpy(&v, &tile[rbl * 16 + r][c * 16], 16);
    *reinterpret_cast<uint4*>(Wq + ((((size_t)(n0 >> 4) + rbl) * KB + blockIdx.y) * 4 + c) * 256 +
                              r * 16) = v;
  }
}

// Pack a row-major int8 matrix [R][K] into the packed layout, zero-filling
// the row and k padding.  One thread per 16-byte chunk of the destination.
__global__ __launch_bounds__(256) void k_pack_rows(const int8_t* __restrict__ src, int R, int K,
                                                   int8_t* __restrict__ dst, int KB, int64_t nchunks) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= nchunks) return;
  // destination chunk q = ((rb * KB + kb) * 4 + c) * 16 + r
  const int r = (int)(q & 15), c = (int)((q >> 4) & 3);
  const int64_t blk = q >> 6;
  const int kb = (int)(blk % KB);
  const int64_t rb = blk / KB;
  const int64_t row = rb * 16 + r;
  const int k = kb * 64 + c * 16;
  uint4 v = make_uint4(0, 0, 0, 0);
  if (row < R && k < K) v = *reinterpret_cast<const uint4*>(src + row * K + k);
  *reinterpret_cast<uint4*>(dst + q * 16) = v;
}

// ---------------------------------------------------------------- K1
// Column absmax of X[M][K] and the outlier bit mask.  One workgroup per
// strip of 32 columns (64 bytes of a row); NT threads = NT/4 row lanes x 4
// column lanes of 8 fp16, eight rows in flight per lane (four left the
// 13B-scale shapes latency-bound: 1 us slower).  The row lanes'
// maxima are combined by wavefront shuffles and then across wavefronts in
// LDS; the final compare runs on one wavefront whose ballot yields the
// 32-bit mask word of the strip directly.
template <int NT>
__global__ __launch_bounds__(NT) void k_detect(
    const uint16_t* __restrict__ X, int M, int K, float alpha,
    float* __restrict__ colmax, uint32_t* __restrict__ mask) {
  constexpr int RL = NT / 4;  // row lanes
  constexpr int NW = NT / 64;  // wavefronts
  __shared__ uint32_t red[NW][16];
  const int t = threadIdx.x;
  const int cl = t & 3, rl = t >> 2;
  // the two 64-byte halves of a 128-byte line go to one XCD's L2
  const int strip = xcd_remap(blockIdx.x, gridDim.x);
  const int col = strip * 32 + cl * 8;
  const u16x2 msk = (u16x2)(0x7fff);
  u16x2 m[4] = {0, 0, 0, 0};
  if (col < K) {
    const uint16_t* p = X + (size_t)rl * K + col;
    const size_t step = (size_t)RL * K;
    int r = rl;
    for (; r + 7 * RL < M; r += 8 * RL, p += 8 * step) {
      uint4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const uint4*>(p + u * step);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        m[0] = __builtin_elementwise_max(m[0], __builtin_bit_cast(u16x2, v[u].x) & msk);
        m[1] = __builtin_elementwise_max(m[1], __builtin_bit_cast(u16x2, v[u].y) & msk);
        m[2] = __builtin_elementwise_max(m[2], __builtin_bit_cast(u16x2, v[u].z) & msk);
        m[3] = __builtin_elementwise_max(m[3], __builtin_bit_cast(u16x2, v[u].w) & msk);
      }
    }
    for (; r < M; r += RL, p += step) {
      uint4 v = *reinterpret_cast<const uint4*>(p);
      m[0] = __builtin_elementwise_max(m[0], __builtin_bit_cast(u16x2, v.x) & msk);
      m[1] = __builtin_elementwise_max(m[1], __builtin_bit_cast(u16x2, v.y) & msk);
      m[2] = __builtin_elementwise_max(m[2], __builtin_bit_cast(u16x2, v.z) & msk);
      m[3] = __builtin_elementwise_max(m[3], __builtin_bit_cast(u16x2, v.w) & msk);
    }
  }
  // reduce over the 16 row lanes of each wavefront (lane bits 2..5), then
  // over the wavefronts through LDS
#pragma unroll
  for (int o = 4; o < 64; o <<= 1) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t y = __shfl_xor(__builtin_bit_cast(uint32_t, m[e]), o, kWave);
      m[e] = __builtin_elementwise_max(m[e], __builtin_bit_cast(u16x2, y));
    }
  }
  const int lane = t & 63;
  if (lane < 4) {
#pragma unroll
    for (int e = 0; e < 4; ++e) red[t >> 6][lane * 4 + e] = __builtin_bit_cast(uint32_t, m[e]);
  }
  __syncthreads();
  if (t < 64) {  // wavefront 0 finishes the strip
    const int c = strip * 32 + t;
    bool out = false;
    if (t < 32) {
      // column t of the strip: lane t/8, pair (t%8)/2, half t%2
      uint16_t mx = 0;
      for (int q = 0; q < NW; ++q) {
        const uint32_t pr = red[q][(t >> 3) * 4 + ((t & 7) >> 1)];
        const uint16_t v16 = (uint16_t)((t & 1) ? (pr >> 16) : (pr & 0xffffu));
        mx = v16 > mx ? v16 : mx;
      }
      const float v = h2f(mx);
      if (c < K) {
        colmax[c] = v;
        out = v > alpha;  // strict: a magnitude equal to alpha stays int8
      }
    }
    const unsigned long long b = __ballot(out);
    if (t == 0) mask[strip] = (uint32_t)b;
  }
}

// Few rows (M <= 32, the decode calls): one wavefront per strip of 32
// columns, lane l taking row l/2 and 16 columns (32 bytes); the column
// maxima are reduced over the rows by shuffles alone (no LDS, no barrier),
// then lanes 0 and 1 compare their 16 columns and form the mask word.  With
// the mask of its strip known, the wavefront also takes each row's absmax
// over the strip's non-outlier columns and writes it (fp16 magnitude bits)
// to rowpart[row][strip] (row stride pstride), when rowpart is given: the
// quantizer then reduces these instead of reading whole rows.
__global__ __launch_bounds__(64) void k_detect_small(
    const uint16_t* __restrict__ X, int M, int K, float alpha, float* __restrict__ colmax,
    uint32_t* __restrict__ mask, uint16_t* __restrict__ rowpart, int pstride) {
  const int lane = threadIdx.x;
  const int r = lane >> 1, h = lane & 1;
  const int c0 = 32 * blockIdx.x + 16 * h;  // K % 16 == 0: a half is all in range or out
  const u16x2 msk = (u16x2)(0x7fff);
  u16x2 m[8], own[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) m[j] = (u16x2)(0);
  if (r < M && c0 < K) {
    const uint4 a = *reinterpret_cast<const uint4*>(X + (size_t)r * K + c0);
    const uint4 b = *reinterpret_cast<const uint4*>(X + (size_t)r * K + c0 + 8);
    const uint32_t d[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) m[j] = __builtin_bit_cast(u16x2, d[j]) & msk;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) own[j] = m[j];
#pragma unroll
  for (int o = 2; o < 64; o <<= 1) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t y = __shfl_xor(__builtin_bit_cast(uint32_t, m[j]), o, kWave);
      m[j] = __builtin_elementwise_max(m[j], __builtin_bit_cast(u16x2, y));
    }
  }
  uint32_t bits = 0;
  if (lane < 2 && c0 < K) {
    float v[16];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      v[2 * j] = h2f(m[j].x);
      v[2 * j + 1] = h2f(m[j].y);
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) bits |= (v[e] > alpha ? 1u : 0u) << e;  // strict
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<float4*>(colmax + c0 + 4 * q) =
          make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
  }
  const uint32_t word = __shfl(bits, 0, kWave) | (__shfl(bits, 1, kWave) << 16);
  if (lane == 0) mask[blockIdx.x] = word;
  if (rowpart) {
    const uint32_t mb = (word >> (16 * h)) & 0xffffu;  // this lane's 16 columns
    uint32_t pm = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t lo = own[j].x & (((mb >> (2 * j)) & 1u) - 1u);
      const uint32_t hv = own[j].y & (((mb >> (2 * j + 1)) & 1u) - 1u);
      pm = max(pm, max(lo, hv));
    }
    pm = max(pm, (uint32_t)__shfl_xor(pm, 1, kWave));
    if (h == 0 && r < M) rowpart[(size_t)r * pstride + blockIdx.x] = (uint16_t)pm;
  }
}

// Large X: the column absmax in two passes.  Pass 1 (k_colmax_part): each
// workgroup reads kPartRows whole rows x 2048 columns (4 KB per row,
// coalesced) and writes their column magnitude maxima, as fp16 bit
// patterns, to one row of a partial matrix [ceil(M/kPartRows)][K].  Pass 2
// is k_detect on that matrix: its column absmax is the column absmax of X.
constexpr int kPartRows = 32;

__global__ __launch_bounds__(256) void k_colmax_part(const uint16_t* __restrict__ X, int M, int K,
                                                     uint16_t* __restrict__ part) {
  const int c = (blockIdx.y * 256 + threadIdx.x) * 8;  // first of 8 columns
  if (c >= K) return;
  const int r0 = blockIdx.x * kPartRows;
  const int rows = min(kPartRows, M - r0);
  const u16x2 msk = (u16x2)(0x7fff);
  u16x2 m[4] = {0, 0, 0, 0};
  const uint16_t* p = X + (size_t)r0 * K + c;
  int r = 0;
  for (; r + 8 <= rows; r += 8, p += (size_t)8 * K) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const uint4*>(p + (size_t)u * K);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      m[0] = __builtin_elementwise_max(m[0], __builtin_bit_cast(u16x2, v[u].x) & msk);
      m[1] = __builtin_elementwise_max(m[1], __builtin_bit_cast(u16x2, v[u].y) & msk);
      m[2] = __builtin_elementwise_max(m[2], __builtin_bit_cast(u16x2, v[u].z) & msk);
      m[3] = __builtin_elementwise_max(m[3], __builtin_bit_cast(u16x2, v[u].w) & msk);
    }
  }
  for (; r < rows; ++r, p += K) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    m[0] = __builtin_elementwise_max(m[0], __builtin_bit_cast(u16x2, v.x) & msk);
    m[1] = __builtin_elementwise_max(m[1], __builtin_bit_cast(u16x2, v.y) & msk);
    m[2] = __builtin_elementwise_max(m[2], __builtin_bit_cast(u16x2, v.z) & msk);
    m[3] = __builtin_elementwise_max(m[3], __builtin_bit_cast(u16x2, v.w) & msk);
  }
  *reinterpret_cast<uint4*>(part + (size_t)blockIdx.x * K + c) =
      make_uint4(__builtin_bit_cast(uint32_t, m[0]), __builtin_bit_cast(uint32_t, m[1]),
                 __builtin_bit_cast(uint32_t, m[2]), __builtin_bit_cast(uint32_t, m[3]));
}

// ---------------------------------------------------------------- K2
// Shared part: load the outlier mask into LDS and build, per mask word, the
// number of outlier columns before it (exclusive prefix).  The rank of
// outlier column k is then pref[k/32] + popcount(mask[k/32] below bit k%32),
// which places it in the ascending list without materializing the list.
// Returns the total count.
__device__ __forceinline__ int load_mask_prefix(const uint32_t* __restrict__ mask_g, int nwords,
                                                uint32_t* sm_mask, int* sm_pref, int* sm_tmp) {
  const int t = threadIdx.x;
  const int per = (nwords + 255) / 256;  // words per thread (<= 8 for K <= 65536)
  const int w0 = t * per;
  int local = 0;
  for (int i = 0; i < per; ++i) {
    const int w = w0 + i;
    if (w < nwords) {
      const uint32_t b = mask_g[w];
      sm_mask[w] = b;
      local += popc(b);
    }
  }
  // inclusive scan of `local` across the block: wavefront scan + LDS
  const int lane = t & 63, wv = t >> 6;
  int x = local;
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  if (lane == 63) sm_tmp[wv] = x;
  __syncthreads();
  int before = 0;
  for (int i = 0; i < wv; ++i) before += sm_tmp[i];
  int total = 0;
  for (int i = 0; i < 4; ++i) total += sm_tmp[i];
  int run = before + x - local;  // exclusive prefix of this thread
  for (int i = 0; i < per; ++i) {
    const int w = w0 + i;
    if (w < nwords) {
      sm_pref[w] = run;
      run += popc(sm_mask[w]);
    }
  }
  __syncthreads();
  return total;
}

constexpr int kGatherRanks = 1024;  // outlier ranks per gather workgroup (multiple of 16)

// fp16 element (row, t) of a packed outlier matrix with KBo blocks per row
__device__ __forceinline__ uint16_t* out_elem(uint16_t* P, int row, int t, int KBo) {
  return reinterpret_cast<uint16_t*>(reinterpret_cast<int8_t*>(P) + pack_offset(row, 2 * t, KBo));
}

// One row of X quantized by WPR wavefronts (one or two), for rows of at
// most WPR * 64 * CPL 16-column chunks: lane l of part h holds chunks
// h * 64 * CPL + l + 64 j in registers.  The row absmax over the
// non-outlier columns and the outliers' ranks come from wavefront
// reductions and scans, and the mask words straight from global memory
// (L2); with two parts per row their absmax and outlier counts meet in LDS
// at one workgroup barrier (sm_x: two words per wavefront), which every
// wavefront reaches (valid = false: a wavefront past the last row only
// takes part in the barrier).  Writes the packed int8 row (zeros past K up
// to the padded row), x_absmax, the row's X_out values (zero from n up to
// roundup(n, 16)); row 0 also the outlier list and the header.
template <int CPL, int WPR>
__device__ __forceinline__ void quant_row_wave(const uint16_t* __restrict__ X, int K,
                                               const uint32_t* __restrict__ mask_g, int n_cap,
                                               int8_t* __restrict__ Xi8, int KB,
                                               float* __restrict__ xabs, uint16_t* __restrict__ Xout,
                                               int32_t* __restrict__ hdr, int32_t* __restrict__ idx,
                                               const OutlierSource& src, int N, int KBo, int i,
                                               bool valid, uint32_t* sm_x) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int h = wv % WPR;            // part of the row
  const int c0 = h * 64 * CPL;       // its first chunk
  const int nwords = (K + 31) >> 5, nchunks = valid ? K >> 4 : 0, pchunks = valid ? KB * 4 : 0;
  const uint16_t* xr = X + (size_t)(valid ? i : 0) * K;
  // 1. the part's chunks and their mask bits, all loads in flight together
  uint4 d[CPL][2];
  uint32_t mb[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = c0 + lane + 64 * j;
    d[j][0] = d[j][1] = make_uint4(0u, 0u, 0u, 0u);
    uint32_t wd = 0;
    if (c < nchunks) {
      d[j][0] = *reinterpret_cast<const uint4*>(xr + 16 * c);
      d[j][1] = *reinterpret_cast<const uint4*>(xr + 16 * c + 8);
      wd = mask_g[c >> 1];
    }
    mb[j] = (wd >> ((c & 1) * 16)) & 0xffffu;
  }
  // 2. absmax over the non-outlier columns (an outlier's magnitude masked to 0)
  uint32_t amax = 0;
#pragma unroll
  for (int j = 0; j < CPL; ++j) amax = max(amax, absmax_chunk16(d[j][0], d[j][1], mb[j]));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = max(amax, (uint32_t)__shfl_xor(amax, o, kWave));
  // 3. rank of each chunk's first outlier within the part: the outliers of
  // all chunks of earlier passes, then an exclusive scan over the lanes
  // (skipped for a pass without outliers, the common case)
  int base[CPL];
  int run = 0;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int cnt = popc(mb[j]);
    base[j] = run;
    if (__ballot(cnt != 0) != 0) {
      int x = cnt;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, kWave);
        if (lane >= o) x += y;
      }
      base[j] = run + x - cnt;
      run += __shfl(x, 63, kWave);
    }
  }
  if constexpr (WPR > 1) {
    // the parts of one row: the row absmax, and the outliers before this part
    if (lane == 0) {
      sm_x[2 * wv] = amax;
      sm_x[2 * wv + 1] = (uint32_t)run;
    }
    __syncthreads();
    const int w0 = wv - h;
    int before = 0, total = 0;
#pragma unroll
    for (int q = 0; q < WPR; ++q) {
      amax = max(amax, sm_x[2 * (w0 + q)]);
      const int cq = (int)sm_x[2 * (w0 + q) + 1];
      total += cq;
      before += q < h ? cq : 0;
    }
#pragma unroll
    for (int j = 0; j < CPL; ++j) base[j] += before;
    run = total;
  }
  if (!valid) return;
  const float ax = h2f((uint16_t)amax);
  const float s = qscale(ax);
  const int n_all = run;
  const int n = n_all < n_cap ? n_all : n_cap;
  const int npad = (n + 15) & ~15;
  // 4. quantize, store the packed int8 chunks, scatter the outliers
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = c0 + lane + 64 * j;
    if (c < pchunks) {
      uint4 qv = make_uint4(0u, 0u, 0u, 0u);
      if (c < nchunks) {
        qv = quant_chunk16(d[j][0], d[j][1], s, mb[j]);
        const int r0 = base[j];
        if (mb[j] == 0xffffu && (r0 & 7) == 0 && r0 + 16 <= n) {
          // a chunk of 16 outlier columns with aligned ranks: two 16-byte stores
          *reinterpret_cast<uint4*>(out_elem16(Xout, i, r0, KBo)) = d[j][0];
          *reinterpret_cast<uint4*>(out_elem16(Xout, i, r0 + 8, KBo)) = d[j][1];
          if (i == 0) {
#pragma unroll
            for (int e = 0; e < 16; ++e) idx[r0 + e] = 16 * c + e;
          }
        } else {
          for (uint32_t bb = mb[j]; bb; bb &= bb - 1u) {
            const int e = __builtin_ctz(bb);
            const int r = r0 + popc(mb[j] & ((1u << e) - 1u));
            if (r < n) {
              *out_elem16(Xout, i, r, KBo) = pick16(d[j][0], d[j][1], e);
              if (i == 0) idx[r] = 16 * c + e;
            }
          }
        }
      }
      *reinterpret_cast<uint4*>(Xi8 + pack_offset(i, 16 * c, KB)) = qv;
    }
  }
  if (h != 0) return;
  for (int r = n + lane; r < npad; r += 64) *out_elem16(Xout, i, r, KBo) = 0;
  if (lane == 0) xabs[i] = ax;
  if (i == 0) {
    // outlier dims missing from an outlier-row cache (or no valid cache)
    const bool cached = !src.W && src.cache;
    int missed = 0, bad = 0;
    if (cached) {
      const int4 ch = *reinterpret_cast<const int4*>(src.cache);
      const bool ok = ch.x == kCacheMagic && ch.y == K && ch.z == N && ch.w >= 0 && ch.w <= K;
      bad = ok ? 0 : 1;
      if (!ok) {
        missed = n_all > 0;
      } else {
        for (int wd = lane; wd < nwords; wd += 64)
          for (uint32_t bb = mask_g[wd]; bb; bb &= bb - 1u) {
            const int sl = src.slot[wd * 32 + __builtin_ctz(bb)];
            if (sl < 0 || sl >= ch.w) missed = 1;
          }
      }
    }
    missed = __any(missed) ? 1 : 0;
    if (lane == 0) {
      hdr[0] = (n_all > n_cap ? 1 : 0) | (missed ? 2 : 0) | (bad ? 4 : 0);
      hdr[1] = n;
      hdr[2] = n_all;
      hdr[3] = 0;
    }
  }
}

// Row role: blockIdx.x < M, one workgroup per row (WPR = 1 or 2: blockIdx.x
// < ceil(M / (4 / WPR)), WPR wavefronts per row, quant_row_wave).  Gather
// role: the remaining blocks each take 256 columns j of W and one group of
// outlier ranks, and write that part of rows j of W_out^T.  CPT = 16-column
// chunks per thread (WPR > 0: per lane of each part; the row lives in
// registers between the absmax and the quantize); the int8 row is written
// in the packed layout, padding chunks as zeros.
// X_out and W_out^T are packed fp16 (KBo blocks of 32 outlier columns per
// row), zero from n up to npad = roundup(n, 16), the end of the last
// 16-column k-step the GEMM reads.
template <int CPT, int WPR>
__global__ __launch_bounds__(256) void k_quant_act(
    const uint16_t* __restrict__ X, int M, int K, const uint32_t* __restrict__ mask,
    int n_cap, int8_t* __restrict__ Xi8, int KB, float* __restrict__ xabs,
    uint16_t* __restrict__ Xout, int32_t* __restrict__ hdr, int32_t* __restrict__ idx,
    OutlierSource src, int N, uint16_t* __restrict__ WoutT, int KBo) {
  // the mask and its prefix counts; the gather role reuses these 16 KB as
  // its transpose tile once its outlier list is built
  __shared__ __align__(16) uint32_t sm_buf[2 * INT8MM_MAX_K_WORDS];
  uint32_t* sm_mask = sm_buf;
  int* sm_pref = reinterpret_cast<int*>(sm_buf + INT8MM_MAX_K_WORDS);
  __shared__ int sm_tmp[8];
  __shared__ uint32_t sm_red[8];
  __shared__ int sm_list[kGatherRanks];
  __shared__ int sm_slot[kGatherRanks];
  const int t = threadIdx.x;
  const int nwords = (K + 31) >> 5;
  const int nchunks = K >> 4;   // 16-column chunks holding data
  constexpr int RPW = WPR > 0 ? 4 / WPR : 1;  // rows per workgroup
  const int row_wgs = WPR > 0 ? (M + RPW - 1) / RPW : M;
  if constexpr (WPR > 0) {
    if ((int)blockIdx.x < row_wgs) {
      // RPW rows per workgroup, WPR wavefronts each; the workgroups of one
      // 16-row packed block go to one XCD, so its L2 merges their 16-byte
      // pieces of each packed line before write-back
      const int i = xcd_remap(blockIdx.x, row_wgs) * RPW + (t >> 6) / WPR;
      if (WPR == 1 && i >= M) return;  // no barrier in the one-wavefront form
      quant_row_wave<CPT, WPR>(X, K, mask, n_cap, Xi8, KB, xabs, Xout, hdr, idx, src, N, KBo, i,
                               i < M, sm_red);
      return;
    }
  }
  // the row's loads go out first so their latency overlaps the mask setup
  uint4 v[WPR > 0 ? 1 : CPT][2];
  const bool row_role = WPR == 0 && (int)blockIdx.x < M;
  // rows of one 16-row packed block go to one XCD, so its L2 merges their
  // 16-byte pieces of each packed line before write-back
  const int i = row_role ? xcd_remap(blockIdx.x, M) : 0;
  if (row_role) {
    const uint16_t* xr = X + (size_t)i * K;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int c = t + j * 256;
      v[j][0] = v[j][1] = make_uint4(0, 0, 0, 0);
      if (c < nchunks) {
        v[j][0] = *reinterpret_cast<const uint4*>(xr + 16 * c);
        v[j][1] = *reinterpret_cast<const uint4*>(xr + 16 * c + 8);
      }
    }
  }
  const int n_all = load_mask_prefix(mask, nwords, sm_mask, sm_pref, sm_tmp);
  const int n = n_all < n_cap ? n_all : n_cap;
  const int npad = (n + 15) & ~15;
  // outlier-row cache: its header must name this K and N, else no slot is
  // read and every outlier row takes the dequantized stand-in
  const bool cached = !src.W && src.cache;
  bool cache_ok = false;
  int n_dims = 0;
  if (cached) {
    const int4 ch = *reinterpret_cast<const int4*>(src.cache);
    cache_ok = ch.x == kCacheMagic && ch.y == K && ch.z == N && ch.w >= 0 && ch.w <= K;
    n_dims = cache_ok ? ch.w : 0;
  }
  // cache row of outlier dim k, or -1 (not cached, or no valid cache)
  auto slot_of = [&](int k) {
    const int sl = cache_ok ? src.slot[k] : -1;
    return sl >= 0 && sl < n_dims ? sl : -1;
  };

  if (row_role) {
    const int pchunks = KB * 4;   // chunks up to the padded K
    uint32_t amax = 0;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int c = t + j * 256;
      if (c < nchunks) {
        // an outlier column's magnitude is masked to 0
        const uint32_t mb = (sm_mask[c >> 1] >> ((c & 1) * 16)) & 0xffffu;
        amax = max(amax, absmax_chunk16(v[j][0], v[j][1], mb));
      }
    }
    amax = block_max_u32(amax, sm_red);
    const float ax = h2f((uint16_t)amax);
    const float s = qscale(ax);
    if (t == 0) xabs[i] = ax;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int c = t + j * 256;
      if (c < pchunks) {
        uint4 qv = make_uint4(0u, 0u, 0u, 0u);
        if (c < nchunks) {
          const uint32_t word = sm_mask[c >> 1];
          const uint32_t mb = (word >> ((c & 1) * 16)) & 0xffffu;
          // every element quantized, outlier columns then masked to 0
          qv = quant_chunk16(v[j][0], v[j][1], s, mb);
          const int base = sm_pref[c >> 1];
          const int r0 = base + ((c & 1) ? popc(word & 0xffffu) : 0);  // rank of the chunk's first outlier
          if (mb == 0xffffu && (r0 & 7) == 0 && r0 + 16 <= n) {
            // a chunk of 16 outlier columns with aligned ranks: two 16-byte stores
            *reinterpret_cast<uint4*>(out_elem(Xout, i, r0, KBo)) = v[j][0];
            *reinterpret_cast<uint4*>(out_elem(Xout, i, r0 + 8, KBo)) = v[j][1];
            if (i == 0) {
#pragma unroll
              for (int e = 0; e < 16; ++e) idx[r0 + e] = 16 * c + e;
            }
          } else {
            // outlier columns in this chunk (almost always none): scatter
            // each to its rank.  A loop over the set bits, not an unrolled
            // test of all 16, keeps the common path short: the wavefront
            // runs as many iterations as its busiest lane needs.
            const uint32_t dw[8] = {v[j][0].x, v[j][0].y, v[j][0].z, v[j][0].w,
                                    v[j][1].x, v[j][1].y, v[j][1].z, v[j][1].w};
            for (uint32_t bits = mb; bits; bits &= bits - 1u) {
              const int e = __builtin_ctz(bits);
              const int bit = (c & 1) * 16 + e;
              const int r = base + popc(word & ((1u << bit) - 1u));
              if (r < n) {
                uint32_t d = dw[0];
#pragma unroll
                for (int u = 1; u < 8; ++u) d = (e >> 1) == u ? dw[u] : d;
                *out_elem(Xout, i, r, KBo) = (uint16_t)(d >> ((e & 1) * 16));
                if (i == 0) idx[r] = 16 * c + e;
              }
            }
          }
        }
        *reinterpret_cast<uint4*>(Xi8 + pack_offset(i, 16 * c, KB)) = qv;
      }
    }
    for (int r = n + t; r < npad; r += 256) *out_elem(Xout, i, r, KBo) = 0;
    // row 0 also reports outlier dims missing from an outlier-row cache
    int missed = 0;
    if (i == 0 && cached) {
      const int per = (nwords + 255) / 256;
      for (int u = 0; u < per; ++u) {
        const int w = t * per + u;
        if (w < nwords) {
          for (uint32_t b = sm_mask[w]; b; b &= b - 1u)
            if (slot_of(w * 32 + __builtin_ctz(b)) < 0) missed = 1;
        }
      }
    }
    if (i == 0) missed = __syncthreads_or(missed);
    if (i == 0 && t == 0) {
      hdr[0] = (n_all > n_cap ? 1 : 0) | (missed ? 2 : 0) | (cached && !cache_ok ? 4 : 0);
      hdr[1] = n;
      hdr[2] = n_all;
      hdr[3] = 0;
    }
  } else {
    // gather role: workgroup (column block cb, rank group g) writes ranks
    // [g*kGatherRanks, (g+1)*kGatherRanks) of 256 columns j of W_out^T, so
    // a large outlier count (alpha -> 0) spreads over many workgroups.  The
    // ascending outlier list of its ranks is built in LDS.  Then, 32 ranks
    // at a time, the workgroup reads those 32 rows of its 256 columns with
    // 16-byte loads (the next 32 in flight during the rest of the step),
    // transposes them through LDS and writes each column j as four 16-byte
    // chunks (one 64-byte block) of W_out^T row j.
    const int gi = (int)blockIdx.x - row_wgs;
    const int nbn = (N + 255) >> 8;
    const int jb = (gi % nbn) * 256;
    const int base = (gi / nbn) * kGatherRanks;
    if (base >= npad) return;  // uniform: nothing of this rank group is used
    const int top = min(n, base + kGatherRanks);
    const int per = (nwords + 255) / 256;
    for (int u = 0; u < per; ++u) {
      const int w = t * per + u;
      if (w < nwords) {
        uint32_t b = sm_mask[w];
        int r = sm_pref[w];
        if (r < top && r + popc(b) > base) {
          while (b && r < top) {
            if (r >= base) {
              const int k = w * 32 + __builtin_ctz(b);
              sm_list[r - base] = k;
              sm_slot[r - base] = src.W ? 0 : slot_of(k);
            }
            ++r;
            b &= b - 1u;
          }
        }
      }
    }
    __syncthreads();  // the list is complete; sm_buf becomes the tile
    uint16_t* tile = reinterpret_cast<uint16_t*>(sm_buf);  // [32 ranks][256 columns]
    static_assert(32 * 256 * 2 <= (int)sizeof(sm_buf) && kGatherRanks % 32 == 0, "tile");
    const int lim = min(npad, base + kGatherRanks);  // a multiple of 16
    const int er = t >> 5;             // rank within a group of 8
    const int jl = (t & 31) * 8;       // first of the thread's 8 columns
    const int jc = jb + jl;            // N % 16 == 0: all 8 in range or none
    // ranks r0 + er + 8p, p < 4, columns jc .. jc+7 (zeros past n)
    auto load = [&](int r0, uint4(&v)[4]) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int r = r0 + er + 8 * p;
        v[p] = make_uint4(0, 0, 0, 0);
        if (r < n && jc < N) {
          const int k = sm_list[r - base];
          if (src.W) {
            v[p] = *reinterpret_cast<const uint4*>(src.W + (size_t)k * N + jc);
          } else {
            const int sl = sm_slot[r - base];
            if (sl >= 0) {
              v[p] = *reinterpret_cast<const uint4*>(src.rows + (size_t)sl * N + jc);
            } else {  // a dim missing from the cache: dequantized int8 row
              uint16_t h[8];
#pragma unroll
              for (int e = 0; e < 8; ++e)
                h[e] = f2h((float)src.Wi8[pack_offset(jc + e, k, KB)] * (src.wabs[jc + e] / 127.0f));
              __builtin_memcpy(&v[p], h, 16);
            }
          }
        }
      }
    };
    const int j = jb + t;
    uint4 v[4];
    load(base, v);
    for (int r0 = base; r0 < lim; r0 += 32) {
#pragma unroll
      for (int p = 0; p < 4; ++p) *reinterpret_cast<uint4*>(tile + (er + 8 * p) * 256 + jl) = v[p];
      __syncthreads();
      if (r0 + 32 < lim) load(r0 + 32, v);
      if (j < N) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (r0 + 8 * q < lim) {
            uint16_t h[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) h[e] = tile[(8 * q + e) * 256 + t];
            uint4 o;
            __builtin_memcpy(&o, h, 16);
            *reinterpret_cast<uint4*>(out_elem(WoutT, j, r0 + 8 * q, KBo)) = o;
          }
        }
      }
      __syncthreads();  // the tile is read before the next step overwrites it
    }
  }
}

// The row quantizer of the decode calls (M <= 32, after k_detect_small
// with rowpart): one wavefront per (row, 1024 columns), so a row's work is
// spread over ceil(K/1024) compute units and no workgroup barrier is
// needed.  Lane l takes one 16-column chunk.  Everything it needs is loaded
// at once: its chunk of X, its mask word, the row's strip maxima (the row
// absmax is their max) and the mask words for the outlier counts before the
// wavefront's columns and in all of K.  Then it quantizes its chunk, stores
// 16 packed bytes, and scatters its outliers to their ranks; the wavefront
// of columns 0-1023 also writes x_absmax and the zeros of X_out past n, and
// that of row 0 the header (with the outlier-row cache check).
// kWordLoads x 64 lanes x 4 mask words cover K up to kWordLoads * 8192,
// kPartLoads x 64 lanes x 8 strip maxima K up to kPartLoads * 16384.
template <int kWordLoads, int kPartLoads>
__global__ __launch_bounds__(64) void k_quant_strips(
    const uint16_t* __restrict__ X, int M, int K, const uint32_t* __restrict__ mask_g,
    const uint16_t* __restrict__ rowpart, int pstride, int n_cap, int8_t* __restrict__ Xi8, int KB,
    float* __restrict__ xabs, uint16_t* __restrict__ Xout, int32_t* __restrict__ hdr,
    int32_t* __restrict__ idx, OutlierSource src, int N, int KBo) {
  const int lane = threadIdx.x;
  const int g = blockIdx.x, i = blockIdx.y;
  const int nwords = (K + 31) >> 5;
  const int nstrips = nwords;
  const int nchunks = K >> 4, pchunks = KB * 4;
  const int c = g * 64 + lane;
  // 1. every load of the wavefront in flight together (indices clamped, not
  // predicated, so they issue back to back)
  uint4 d0 = make_uint4(0u, 0u, 0u, 0u), d1 = d0;
  uint32_t myword = 0;
  if (c < nchunks) {
    d0 = *reinterpret_cast<const uint4*>(X + (size_t)i * K + 16 * c);
    d1 = *reinterpret_cast<const uint4*>(X + (size_t)i * K + 16 * c + 8);
    myword = mask_g[c >> 1];
  }
  const uint16_t* rp = rowpart + (size_t)i * pstride;
  uint4 pv[kPartLoads];
#pragma unroll
  for (int j = 0; j < kPartLoads; ++j) {
    const int s0 = 8 * (lane + 64 * j);
    pv[j] = *reinterpret_cast<const uint4*>(rp + min(s0, pstride - 8));
  }
  uint4 wv[kWordLoads];
#pragma unroll
  for (int j = 0; j < kWordLoads; ++j) {
    const int w0 = 4 * (lane + 64 * j);
    wv[j] = *reinterpret_cast<const uint4*>(mask_g + min(w0, ((nwords + 3) & ~3) - 4));
  }
  // 2. row absmax (strips past nstrips are not counted) and outlier counts
  uint32_t pm = 0;
#pragma unroll
  for (int j = 0; j < kPartLoads; ++j) {
    const int s0 = 8 * (lane + 64 * j);
    const uint32_t dw[4] = {pv[j].x, pv[j].y, pv[j].z, pv[j].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t v = (dw[e >> 1] >> ((e & 1) * 16)) & 0xffffu;
      if (s0 + e < nstrips) pm = max(pm, v);
    }
  }
  const int wbefore = g * 32;  // mask words left of this wavefront's columns
  int before = 0, total = 0;
#pragma unroll
  for (int j = 0; j < kWordLoads; ++j) {
    const int w0 = 4 * (lane + 64 * j);
    const uint32_t ww[4] = {wv[j].x, wv[j].y, wv[j].z, wv[j].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int pc = w0 + e < nwords ? popc(ww[e]) : 0;
      total += pc;
      before += w0 + e < wbefore ? pc : 0;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    pm = max(pm, (uint32_t)__shfl_xor(pm, o, kWave));
    total += __shfl_xor(total, o, kWave);
    before += __shfl_xor(before, o, kWave);
  }
  const int n_all = total;
  const int n = n_all < n_cap ? n_all : n_cap;
  // ranks within the wavefront: exclusive scan of the chunks' outlier counts
  const uint32_t mb = (myword >> ((c & 1) * 16)) & 0xffffu;
  int x = popc(mb);
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  const int r0 = before + x - popc(mb);
  // 3. quantize the chunk (zeros past K up to the padded row)
  const float ax = h2f((uint16_t)pm);
  const float s = qscale(ax);
  if (c < pchunks) {
    uint4 qv = make_uint4(0u, 0u, 0u, 0u);
    if (c < nchunks) {
      qv = quant_chunk16(d0, d1, s, mb);
      for (uint32_t bb = mb; bb; bb &= bb - 1u) {
        const int e = __builtin_ctz(bb);
        const int r = r0 + popc(mb & ((1u << e) - 1u));
        if (r < n) {
          *out_elem16(Xout, i, r, KBo) = pick16(d0, d1, e);
          if (i == 0) idx[r] = 16 * c + e;
        }
      }
    }
    *reinterpret_cast<uint4*>(Xi8 + pack_offset(i, 16 * c, KB)) = qv;
  }
  if (g == 0) {
    const int npad = (n + 15) & ~15;
    for (int r = n + lane; r < npad; r += 64) *out_elem16(Xout, i, r, KBo) = 0;
    if (lane == 0) xabs[i] = ax;
    if (i == 0) {
      // outlier dims missing from an outlier-row cache (or no valid cache)
      const bool cached = !src.W && src.cache;
      int missed = 0, bad = 0;
      if (cached) {
        const int4 ch = *reinterpret_cast<const int4*>(src.cache);
        const bool ok = ch.x == kCacheMagic && ch.y == K && ch.z == N && ch.w >= 0 && ch.w <= K;
        bad = ok ? 0 : 1;
        if (!ok) {
          missed = n_all > 0;
        } else {
          for (int wd = lane; wd < nwords; wd += 64)
            for (uint32_t bb = mask_g[wd]; bb; bb &= bb - 1u) {
              const int sl = src.slot[wd * 32 + __builtin_ctz(bb)];
              if (sl < 0 || sl >= ch.w) missed = 1;
            }
        }
      }
      missed = __any(missed) ? 1 : 0;
      if (lane == 0) {
        hdr[0] = (n_all > n_cap ? 1 : 0) | (missed ? 2 : 0) | (bad ? 4 : 0);
        hdr[1] = n;
        hdr[2] = n_all;
        hdr[3] = 0;
      }
    }
  }
}

// The row quantizer of the decode calls (M <= 32): one workgroup of NT
// threads per row, no W_out^T gather (the decode kernel gathers the
// outlier rows of its own features).  Writes x_absmax, the packed int8 row,
// the row's X_out values (zero from n to roundup(n, 16)); row 0 also the
// outlier list and the header.
template <int NT>
__global__ __launch_bounds__(NT) void k_quant_rows(
    const uint16_t* __restrict__ X, int M, int K, const uint32_t* __restrict__ mask_g, int n_cap,
    int8_t* __restrict__ Xi8, int KB, float* __restrict__ xabs, uint16_t* __restrict__ Xout,
    int32_t* __restrict__ hdr, int32_t* __restrict__ idx, OutlierSource src, int N, int KBo) {
  __shared__ uint32_t sm_mask[INT8MM_MAX_K_WORDS];
  __shared__ int sm_pref[INT8MM_MAX_K_WORDS];
  __shared__ uint32_t sm_red[NT / 64];
  __shared__ int sm_tmp[NT / 64];
  const int t = threadIdx.x, i = blockIdx.x;
  const int nwords = (K + 31) >> 5;
  // the row's loads go out first so their latency overlaps the mask setup
  uint4 v[8][2];
  row_load<NT, 8>(X + (size_t)i * K, K, v);
  for (int wd = t; wd < nwords; wd += NT) sm_mask[wd] = mask_g[wd];
  __syncthreads();
  const int n_all = block_word_prefix<NT>(sm_mask, sm_pref, nwords, sm_tmp);
  const int n = n_all < n_cap ? n_all : n_cap;
  const int npad = (n + 15) & ~15;
  const float ax = quantize_row<NT, 8>(
      X + (size_t)i * K, K, KB, v, sm_mask, sm_pref, n, sm_red,
      [&](int c, uint4 qv) { *reinterpret_cast<uint4*>(Xi8 + pack_offset(i, 16 * c, KB)) = qv; },
      [&](int r, int k, uint16_t hv) {
        *out_elem16(Xout, i, r, KBo) = hv;
        if (i == 0) idx[r] = k;
      });
  for (int r = n + t; r < npad; r += NT) *out_elem16(Xout, i, r, KBo) = 0;
  if (t == 0) xabs[i] = ax;
  if (i == 0) {
    // outlier dims missing from an outlier-row cache (or no valid cache)
    const bool cached = !src.W && src.cache;
    int missed = 0, bad = 0;
    if (cached) {
      const int4 ch = *reinterpret_cast<const int4*>(src.cache);
      const bool ok = ch.x == kCacheMagic && ch.y == K && ch.z == N && ch.w >= 0 && ch.w <= K;
      bad = ok ? 0 : 1;
      if (!ok) {
        missed = n_all > 0;
      } else {
        for (int wd = t; wd < nwords; wd += NT)
          for (uint32_t bb = sm_mask[wd]; bb; bb &= bb - 1u) {
            const int sl = src.slot[wd * 32 + __builtin_ctz(bb)];
            if (sl < 0 || sl >= ch.w) missed = 1;
          }
      }
    }
    missed = __syncthreads_or(missed);
    if (t == 0) {
      hdr[0] = (n_all > n_cap ? 1 : 0) | (missed ? 2 : 0) | (bad ? 4 : 0);
      hdr[1] = n;
      hdr[2] = n_all;
      hdr[3] = 0;
    }
  }
}

// The detector's stage export: the ascending outlier list and the header
// from the mask alone (in the fused call the quantizer's row 0 writes them).
__global__ __launch_bounds__(256) void k_mask_index(const uint32_t* __restrict__ mask_g,
                                                    int nwords, int n_cap,
                                                    int32_t* __restrict__ idx,
                                                    int32_t* __restrict__ hdr) {
  __shared__ uint32_t sm_mask[INT8MM_MAX_K_WORDS];
  __shared__ int sm_pref[INT8MM_MAX_K_WORDS];
  __shared__ int sm_tmp[8];
  const int n_all = load_mask_prefix(mask_g, nwords, sm_mask, sm_pref, sm_tmp);
  const int t = threadIdx.x;
  for (int w = t; w < nwords; w += 256) {
    int r = sm_pref[w];
    for (uint32_t b = sm_mask[w]; b && r < n_cap; b &= b - 1u, ++r) idx[r] = w * 32 + __builtin_ctz(b);
  }
  if (t == 0) {
    hdr[0] = n_all > n_cap ? 1 : 0;
    hdr[1] = n_all < n_cap ? n_all : n_cap;
    hdr[2] = n_all;
    hdr[3] = 0;
  }
}

// ------------------------------------------------------------ launchers

hipError_t launch_quantize_weight(const uint16_t* W, int K, int N, int8_t* Wq, float* aw,
                                  hipStream_t st) {
  if (N == 0) return hipSuccess;
  const int KB = (int)(pack_kpad(K) / 64);
  k_weight_absmax<<<dim3((N + 63) / 64), dim3(256), 0, st>>>(W, K, N, aw);
  if (KB > 0) k_weight_quant<<<dim3((N + 63) / 64, KB), dim3(256), 0, st>>>(W, K, N, aw, Wq, KB);
  return hipGetLastError();
}

hipError_t launch_pack_rows(const int8_t* src, int R, int K, int8_t* dst, hipStream_t st) {
  const int KB = (int)(pack_kpad(K) / 64);
  const int64_t nchunks = pack_rpad(R) * KB * 64 / 16;
  if (nchunks == 0) return hipSuccess;
  k_pack_rows<<<dim3((unsigned)((nchunks + 255) / 256)), dim3(256), 0, st>>>(src, R, K, dst, KB,
                                                                            nchunks);
  return hipGetLastError();
}

hipError_t launch_detect(const uint16_t* X, int M, int K, float alpha, float* colmax,
                         uint32_t* mask, uint16_t* scratch, hipStream_t st, uint16_t* rowpart) {
  if (K == 0) return hipSuccess;
  if (M > kDetectTwoPassM && (int64_t)M * K >= kDetectTwoPassElems && scratch) {
    const int P = (M + kPartRows - 1) / kPartRows;
    k_colmax_part<<<dim3(P, (K + 2047) / 2048), dim3(256), 0, st>>>(X, M, K, scratch);
    k_detect<256><<<dim3((K + 31) / 32), dim3(256), 0, st>>>(scratch, P, K, alpha, colmax, mask);
  } else if (M <= kDecodeMaxM) {
    k_detect_small<<<dim3((K + 31) / 32), dim3(64), 0, st>>>(X, M, K, alpha, colmax, mask,
                                                             rowpart, rowpart_stride(K));
  } else {
    k_detect<256><<<dim3((K + 31) / 32), dim3(256), 0, st>>>(X, M, K, alpha, colmax, mask);
  }
  return hipGetLastError();
}

hipError_t launch_mask_index(const uint32_t* mask, int K, int n_cap, int32_t* idx, int32_t* hdr,
                             hipStream_t st) {
  k_mask_index<<<dim3(1), dim3(256), 0, st>>>(mask, (K + 31) / 32, n_cap, idx, hdr);
  return hipGetLastError();
}

hipError_t launch_quant_act(const uint16_t* X, int M, int K, uint32_t* mask, int n_cap,
                            int8_t* Xi8, float* xabs, uint16_t* Xout, int32_t* hdr, int32_t* idx,
                            const OutlierSource& src, int N, uint16_t* WoutT, int KBo, bool gather,
                            hipStream_t st) {
  static const bool wave_ok = [] {
    const char* s = getenv("I8MM_QUANT_WAVE");
    return !(s && atoi(s) == 0);
  }();
  const int KB = (int)(pack_kpad(K) / 64);
  const int cpt = (KB * 4 + 255) / 256;
  const int cpl = (KB * 4 + 63) / 64;
  // rank groups of the gather role: enough for n_cap outliers
  const int groups = n_cap > 0 ? (n_cap + kGatherRanks - 1) / kGatherRanks : 1;
  const int64_t gwg = gather ? (int64_t)((N + 255) / 256) * groups : 0;
  const dim3 block(256);
  if (wave_ok && cpl <= 6) {
    // rows of up to 6144 columns: one wavefront per row (a whole-call
    // prologue 3-4 us shorter on the 2048-row 13B-scale shapes; at 8192
    // columns the row takes 192 registers per lane and the kernel was 2 us
    // slower than the workgroup-per-row form)
    const dim3 grid((unsigned)((M + 3) / 4 + gwg));
#define I8MM_QW(C)                                                                       \
  k_quant_act<C, 1><<<grid, block, 0, st>>>(X, M, K, mask, n_cap, Xi8, KB, xabs, Xout, hdr, \
                                            idx, src, N, WoutT, KBo)
    if (cpl <= 2) I8MM_QW(2);
    else if (cpl <= 4) I8MM_QW(4);
    else if (cpl <= 5) I8MM_QW(5);
    else I8MM_QW(6);
#undef I8MM_QW
    return hipGetLastError();
  }
  if (wave_ok && cpl <= 12) {
    // rows of up to 12288 columns: two wavefronts per row, 6 chunks per lane
    const dim3 grid((unsigned)((M + 1) / 2 + gwg));
#define I8MM_QW2(C)                                                                      \
  k_quant_act<C, 2><<<grid, block, 0, st>>>(X, M, K, mask, n_cap, Xi8, KB, xabs, Xout, hdr, \
                                            idx, src, N, WoutT, KBo)
    if (cpl <= 8) I8MM_QW2(4);
    else if (cpl <= 10) I8MM_QW2(5);
    else I8MM_QW2(6);
#undef I8MM_QW2
    return hipGetLastError();
  }
  const dim3 grid((unsigned)(M + gwg));
#define I8MM_QA(C)                                                                       \
  k_quant_act<C, 0><<<grid, block, 0, st>>>(X, M, K, mask, n_cap, Xi8, KB, xabs, Xout, hdr, \
                                            idx, src, N, WoutT, KBo)
  if (cpt <= 1) I8MM_QA(1);
  else if (cpt <= 2) I8MM_QA(2);
  else if (cpt <= 4) I8MM_QA(4);
  else if (cpt <= 8) I8MM_QA(8);
  else I8MM_QA(16);
#undef I8MM_QA
  return hipGetLastError();
}

hipError_t launch_quant_strips(const uint16_t* X, int M, int K, const uint32_t* mask,
                               const uint16_t* rowpart, int n_cap, int8_t* Xi8, float* xabs,
                               uint16_t* Xout, int32_t* hdr, int32_t* idx,
                               const OutlierSource& src, int N, int KBo, hipStream_t st) {
  const int KB = (int)(pack_kpad(K) / 64);
  const dim3 grid((unsigned)((KB * 4 + 63) / 64), (unsigned)M);
  // only the loads the row's mask words and strip maxima need
#define I8MM_QS(WL, PL)                                                                       \
  k_quant_strips<WL, PL><<<grid, dim3(64), 0, st>>>(X, M, K, mask, rowpart, rowpart_stride(K), \
                                                    n_cap, Xi8, KB, xabs, Xout, hdr, idx, src, N, \
                                                    KBo)
  if (K <= 8192) I8MM_QS(1, 1);
  else if (K <= 16384) I8MM_QS(2, 1);
  else if (K <= 32768) I8MM_QS(4, 2);
  else I8MM_QS(8, 4);
#undef I8MM_QS
  return hipGetLastError();
}

hipError_t launch_quant_rows(const uint16_t* X, int M, int K, uint32_t* mask, int n_cap,
                             int8_t* Xi8, float* xabs, uint16_t* Xout, int32_t* hdr, int32_t* idx,
                             const OutlierSource& src, int N, int KBo, hipStream_t st) {
  const int KB = (int)(pack_kpad(K) / 64);
  k_quant_rows<512><<<dim3(M), dim3(512), 0, st>>>(X, M, K, mask, n_cap, Xi8, KB, xabs, Xout, hdr,
                                                   idx, src, N, KBo);
  return hipGetLastError();
}

// Outlier-row cache: rows[s][j] = W[dims[s]][j] (once, at load).
__global__ __launch_bounds__(256) void k_cache_rows(const uint16_t* __restrict__ W, int N,
                                                    const int32_t* __restrict__ dims,
                                                    uint16_t* __restrict__ rows, int nbn) {
  const int s = blockIdx.x / nbn;
  const int j = (blockIdx.x % nbn) * 256 + threadIdx.x;
  if (j < N) rows[(size_t)s * N + j] = W[(size_t)dims[s] * N + j];
}

hipError_t launch_cache_rows(const uint16_t* W, int N, const int32_t* dims, int n_dims,
                             uint16_t* rows, hipStream_t st) {
  if (n_dims == 0 || N == 0) return hipSuccess;
  const int nbn = (N + 255) / 256;
  k_cache_rows<<<dim3((unsigned)((int64_t)nbn * n_dims)), dim3(256), 0, st>>>(W, N, dims, rows,
                                                                              nbn);
  return hipGetLastError();
}

}  // namespace i8mm
