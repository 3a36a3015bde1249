// Decode kernel (M <= 32, and 33-64 tokens where use_decode says so): the
// int8 weight W_i8 (packed layout, pack.hpp) is streamed from HBM exactly
// once, every byte feeding a 16x16x64 int8 MFMA whose 16 columns are
// tokens (one MFMA per weight fragment and token block of 16, up to four).
// Bandwidth-bound: at M = 64 the product does 128 ops per weight byte, far
// below the chip's ops/byte ridge.
//
// A workgroup owns one 16-row block of W_i8 (16 output features) over all
// of K, so no cross-workgroup reduction is needed, and the work splits into
// N/16 equal workgroups: at the 175B-scale shapes (N = 36864, 49152) that is
// exactly 9 or 12 per compute unit, where 32-feature workgroups left half
// the units with one more than the rest.  Its KS wavefronts split the K
// blocks evenly and combine their int32 partial sums through LDS at the end
// (exact, order-independent).  One 64-byte K block of the row block is one
// contiguous 1 KB piece of W_i8, which the 64 lanes read with one 16-byte
// load each (lane l: row l%16, k-chunk l/16), exactly the MFMA's operand
// layout.  The weight loads are nontemporal (the stream is never re-read);
// the activations (X_i8, same layout, one to four row blocks) stay resident
// in L2.  U K blocks per iteration, the next iteration's loads issued before
// the current MFMAs.
//
// The epilogue takes the steps of the prefill GEMM's (epilogue.hpp):
// dequantize (+ bias), fp16-MFMA outlier product, fp16 store; its operands
// are loaded from global memory before the cross-wavefront reduction, so
// their latency overlaps it.
#include <hip/hip_ext.h>

#include "common.hpp"
#include "launch.hpp"
#include "pack.hpp"
#include "rowquant.hpp"

#include <stdlib.h>

#include <atomic>

namespace i8mm {

// Outlier-product operand of a 16-row MFMA: lane l takes row `row` of a
// packed fp16 matrix, outlier columns 32*blk + 8*(l/16) .. +7 (16-byte chunk
// l/16 of block blk); zeros at or past npad = roundup(n, 16), where the
// matrices are not zero-filled.
__device__ __forceinline__ v8h load_out16(const uint16_t* __restrict__ P, int row, int KBo,
                                          int blk, int npad) {
  const int c = (threadIdx.x & 63) >> 4;
  if (32 * blk + 8 * c >= npad) return v8h{};
  return *reinterpret_cast<const v8h*>(reinterpret_cast<const int8_t*>(P) +
                                       pack_offset(row, 64 * blk + 16 * c, KBo));
}

// The K loop alone, with int32 output (the int8_gemm_i32 export where the
// matmul takes the decode kernel): R row blocks (16 features each) per
// workgroup; KS wavefronts split K; U K blocks per iteration; T token
// blocks of 16 (T = ceil(M / 16)).  X_i8 is a packed operand in global
// memory.
template <int R, int KS, int U, int T>
__global__ __launch_bounds__(KS * 64) void k_decode_i32(
    const int8_t* __restrict__ Xi8, const int8_t* __restrict__ Wi8, int M, int N, int KB,
    int32_t* __restrict__ acc_out) {
  __shared__ v4i red[KS > 1 ? KS - 1 : 1][R][T][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n0 = blockIdx.x * 16 * R;
  const int per = (KB + KS - 1) / KS;
  const int kb0 = min(KB, w * per);
  const int kb1 = min(KB, kb0 + per);
  const size_t rbytes = (size_t)KB * 1024;  // one packed 16-row block over K
  const int8_t* wp = Wi8 + (size_t)blockIdx.x * R * rbytes + lane * 16;
  const int8_t* xp = Xi8 + lane * 16;

  v4i acc[R][T];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int t = 0; t < T; ++t) acc[r][t] = v4i{};

  v4i wa[R][U], xa[T][U], wb[R][U], xb[T][U];
  auto load = [&](int kb, v4i(&wv)[R][U], v4i(&xv)[T][U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t o = (size_t)(kb + u) * 1024;
#pragma unroll
      for (int r = 0; r < R; ++r)
        wv[r][u] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(wp + r * rbytes + o));
#pragma unroll
      for (int t = 0; t < T; ++t) xv[t][u] = *reinterpret_cast<const v4i*>(xp + t * rbytes + o);
    }
  };
  auto compute = [&](const v4i(&wv)[R][U], const v4i(&xv)[T][U]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int t = 0; t < T; ++t) acc[r][t] = mfma16_i8(wv[r][u], xv[t][u], acc[r][t]);
  };

  const int nit = (kb1 - kb0) / U;  // full iterations
  const int kbe = kb0 + nit * U;
  if (nit > 0) load(kb0, wa, xa);
  for (int it = 0; it < nit; it += 2) {
    const int kb = kb0 + it * U;
    if (it + 1 < nit) load(kb + U, wb, xb);
    compute(wa, xa);
    if (it + 1 < nit) {
      if (it + 2 < nit) load(kb + 2 * U, wa, xa);
      compute(wb, xb);
    }
  }
  for (int kb = kbe; kb < kb1; ++kb) {  // remaining blocks, one at a time
    const size_t o = (size_t)kb * 1024;
    v4i x1[T];
#pragma unroll
    for (int t = 0; t < T; ++t) x1[t] = *reinterpret_cast<const v4i*>(xp + t * rbytes + o);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const v4i w1 = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(wp + r * rbytes + o));
#pragma unroll
      for (int t = 0; t < T; ++t) acc[r][t] = mfma16_i8(w1, x1[t], acc[r][t]);
    }
  }

  if constexpr (KS > 1) {
    if (w > 0) {
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int t = 0; t < T; ++t) red[w - 1][r][t][lane] = acc[r][t];
    }
    __syncthreads();
    if (w > 0) return;
#pragma unroll
    for (int s = 0; s < KS - 1; ++s)
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int t = 0; t < T; ++t) acc[r][t] += red[s][r][t][lane];
  }
  // lane l holds features n0 + 16r + 4*(l/16) .. +3 of token 16t + l%16
  const int fq = 4 * (lane >> 4), tl = lane & 15;
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int m = 16 * t + tl;
    if (m < M) {
#pragma unroll
      for (int r = 0; r < R; ++r)
        *reinterpret_cast<v4i*>(acc_out + (size_t)m * N + n0 + 16 * r + fq) = acc[r][t];
    }
  }
}

// ---------------------------------------------------------------------------
// The decode call's GEMM (M <= 64), with the outlier weights gathered by the
// kernel itself.
//
// Every workgroup first issues the loads of its first two K iterations, so
// the weight stream is under way while it sets up.  Its 16*R output features
// need the outlier rows of W only for those features: the workgroup gathers
// them straight from the fp16 W (or the outlier-row cache) for its own
// columns, while its K loop runs, and writes that slice of W_out^T to the
// workspace.  So no separate gather pass precedes the kernel.
//   * M >= 2: the detector and the row quantizer ran before in the same call
//     and left X_i8, x_absmax, X_out, the outlier list and the header in the
//     workspace.
//   * M == 1: there is no detector or quantizer launch.  Every workgroup
//     derives the outlier mask and the row absmax from the one row itself
//     (its column absmax is |x|), quantizes the row into its own LDS and
//     reads its int8 operand from there; workgroup 0 writes the
//     intermediates (column absmax, mask, list, header, x_absmax, X_i8,
//     X_out) to the workspace as the two other kernels would have.
struct DecodeInputs {
  const uint16_t* X;   // [M][K] fp16 activations (read only when M == 1)
  float alpha;         // M == 1: the threshold
  float* colmax;       // M == 1: the detector's column-absmax field (written)
  uint32_t* mask_out;  // M == 1: the detector's mask field (written)
  int8_t* Xi8;         // workspace X_i8 (packed)
  float* xabs;         // workspace x_absmax
  uint16_t* Xout;      // workspace X_out (packed fp16)
  uint16_t* WoutT;     // workspace W_out^T (packed fp16): each workgroup its features
  int32_t* idx;        // workspace outlier list
  int32_t* hdr;        // workspace header
  OutlierSource src;   // outlier weight rows: fp16 W, or a cache
  int K;
};

template <int R, int KS, int U, int T, bool ONE>
__global__ __launch_bounds__(KS * 64) void k_decode_mm(
    const int8_t* __restrict__ Wi8, int M, int N, int KB, Epilogue epi, DecodeInputs in) {
  constexpr int NT = KS * 64;
  __shared__ v4i red[KS > 1 ? KS - 1 : 1][R][T][64];
  __shared__ uint32_t sm_red[NT / 64];
  __shared__ int sm_tmp[NT / 64];
  extern __shared__ __align__(16) int8_t dsm[];
  const int K = in.K;
  const int nwords = (K + 31) >> 5;
  const int nwp = (nwords + 3) & ~3;
  // M == 1: mask words, their prefix counts and the int8 row (KB*64 bytes)
  uint32_t* sm_mask = reinterpret_cast<uint32_t*>(dsm);
  int* sm_pref = reinterpret_cast<int*>(dsm + 4 * nwp);
  int8_t* sm_x = dsm + 8 * nwp;

  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int b = blockIdx.x;
  const int n0 = b * 16 * R;
  // wavefront 0 also issues the epilogue's operand loads and gathers (ahead
  // of its K loop; at 12 row blocks after it, while the others finish
  // theirs), so it takes 1/16 fewer K blocks than the others (the
  // 175B-scale QKV decode: its K loop otherwise ended ~5 us after wavefront
  // 1's; with the deficit the kernel ran ~1.3 us faster)
  const int per = (KB + KS - 1) / KS;
  const int per0 = per - per / 16;
  const int per1 = (KB - per0 + KS - 2) / (KS - 1);
  const int kb0 = w == 0 ? 0 : min(KB, per0 + (w - 1) * per1);
  const int kb1 = w == 0 ? min(KB, per0) : min(KB, kb0 + per1);
  const size_t rbytes = (size_t)KB * 1024;  // one packed 16-row block over K
  const int8_t* wp = Wi8 + (size_t)b * R * rbytes + lane * 16;
  const int8_t* xp = in.Xi8 + lane * 16;
  const int tl = lane & 15, q4 = lane >> 4;

  // 1. the first two iterations' loads.  Loads are never conditional inside
  // the K loop: a block index past the last iteration is clamped to it (a
  // few redundant loads at the end), so the in-order load counters let the
  // next iteration's loads stay in flight under the current MFMAs.
  const int nit = (kb1 - kb0) / U;
  const int klast = kb0 + (nit > 0 ? (nit - 1) * U : 0);
  v4i wa[R][U], wb[R][U], xa[T][U], xb[T][U];
  auto load_w = [&](int kb, v4i(&wv)[R][U]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < R; ++r)
        wv[r][u] = __builtin_nontemporal_load(
            reinterpret_cast<const v4i*>(wp + r * rbytes + (size_t)(kb + u) * 1024));
  };
  auto load_x = [&](int kb, v4i(&xv)[T][U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (ONE) {
        xv[0][u] = tl == 0 ? *reinterpret_cast<const v4i*>(sm_x + (kb + u) * 64 + 16 * q4) : v4i{};
      } else {
#pragma unroll
        for (int tt = 0; tt < T; ++tt)
          xv[tt][u] = *reinterpret_cast<const v4i*>(xp + tt * rbytes + (size_t)(kb + u) * 1024);
      }
    }
  };
  if (nit > 0) {
    load_w(kb0, wa);
    if constexpr (!ONE) load_x(kb0, xa);
    load_w(min(kb0 + U, klast), wb);
    if constexpr (!ONE) load_x(min(kb0 + U, klast), xb);
  }

  // 2. the outlier count (and, M == 1, the whole activation quantization)
  int n_all, n;
  float ax1 = 0.0f;
  bool cache_ok = false;
  int n_dims = 0;
  const bool cached = !in.src.W && in.src.cache;
  if (cached) {  // the outlier-row cache must name this K and N
    const int4 ch = *reinterpret_cast<const int4*>(in.src.cache);
    cache_ok = ch.x == kCacheMagic && ch.y == K && ch.z == N && ch.w >= 0 && ch.w <= K;
    n_dims = cache_ok ? ch.w : 0;
  }
  if constexpr (ONE) {
    // column j is an outlier iff |x_j| > alpha (the detector's fp32 compare)
    const uint16_t* xr = in.X;
    uint32_t amax = 0;
    for (int wd = t; wd < nwords; wd += NT) {
      uint32_t word = 0;
      for (int half = 0; half < 2; ++half) {
        const int c0 = 32 * wd + 16 * half;
        if (c0 < K) {
          uint16_t h[16];
          const uint4 a0 = *reinterpret_cast<const uint4*>(xr + c0);
          const uint4 a1 = *reinterpret_cast<const uint4*>(xr + c0 + 8);
          __builtin_memcpy(h, &a0, 16);
          __builtin_memcpy(h + 8, &a1, 16);
          float cm[16];
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            cm[e] = h2f((uint16_t)(h[e] & 0x7fffu));
            const bool o = cm[e] > in.alpha;
            word |= (o ? 1u : 0u) << (16 * half + e);
            const uint32_t a = o ? 0u : (uint32_t)(h[e] & 0x7fffu);
            amax = a > amax ? a : amax;
          }
          if (b == 0) {
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4)
              *reinterpret_cast<float4*>(in.colmax + c0 + 4 * e4) =
                  make_float4(cm[4 * e4], cm[4 * e4 + 1], cm[4 * e4 + 2], cm[4 * e4 + 3]);
          }
        }
      }
      sm_mask[wd] = word;
      if (b == 0) in.mask_out[wd] = word;
    }
    amax = block_max_nt<NT>(amax, sm_red);
    ax1 = h2f((uint16_t)amax);
    n_all = block_word_prefix<NT>(sm_mask, sm_pref, nwords, sm_tmp);
    n = min(n_all, epi.n_cap);
    const int npad1 = (n + 15) & ~15;
    // the int8 row into LDS (every workgroup); workgroup 0 also writes it,
    // the list and the outlier values to the workspace
    const float s1 = qscale(ax1);
    const int nchunks = K >> 4;
    for (int c = t; c < KB * 4; c += NT) {
      uint4 qv = make_uint4(0u, 0u, 0u, 0u);
      if (c < nchunks) {
        const uint32_t word = sm_mask[c >> 1];
        const uint32_t mb = (word >> ((c & 1) * 16)) & 0xffffu;
        const uint4 a0 = *reinterpret_cast<const uint4*>(in.X + 16 * c);
        const uint4 a1 = *reinterpret_cast<const uint4*>(in.X + 16 * c + 8);
        qv = quant_chunk16(a0, a1, s1, mb);
        if (b == 0) {
          for (uint32_t bits = mb; bits; bits &= bits - 1u) {
            const int e = __builtin_ctz(bits);
            const int r = sm_pref[c >> 1] + popc(word & ((1u << ((c & 1) * 16 + e)) - 1u));
            if (r < n) {
              *out_elem16(in.Xout, 0, r, epi.KBo) = pick16(a0, a1, e);
              in.idx[r] = 16 * c + e;
            }
          }
        }
      }
      *reinterpret_cast<uint4*>(sm_x + 16 * c) = qv;
      if (b == 0) *reinterpret_cast<uint4*>(in.Xi8 + pack_offset(0, 16 * c, KB)) = qv;
    }
    if (b == 0) {
      for (int r = n + t; r < npad1; r += NT) *out_elem16(in.Xout, 0, r, epi.KBo) = 0;
      int missed = 0;
      if (cached && cache_ok) {
        for (int wd = t; wd < nwords; wd += NT)
          for (uint32_t bb = sm_mask[wd]; bb; bb &= bb - 1u) {
            const int sl = in.src.slot[wd * 32 + __builtin_ctz(bb)];
            if (sl < 0 || sl >= n_dims) missed = 1;
          }
      } else if (cached && n_all > 0) {
        missed = 1;
      }
      missed = __syncthreads_or(missed);
      if (t == 0) {
        in.xabs[0] = ax1;
        in.hdr[0] = (n_all > epi.n_cap ? 1 : 0) | (missed ? 2 : 0) | (cached && !cache_ok ? 4 : 0);
        in.hdr[1] = n;
        in.hdr[2] = n_all;
        in.hdr[3] = 0;
      }
    }
    __syncthreads();  // the int8 row is in LDS
    if (nit > 0) {
      load_x(kb0, xa);
      load_x(min(kb0 + U, klast), xb);
    }
  } else {
    // clamped to the capacity the buffers were sized for
    n = min(max(__builtin_amdgcn_readfirstlane(in.hdr[1]), 0), epi.n_cap);
    n_all = (__builtin_amdgcn_readfirstlane(in.hdr[0]) & 1) ? epi.n_cap + 1 : n;
  }
  const int npad = (n + 15) & ~15;

  // 3. the epilogue's operands, issued now so they land during the K loop
  // (only wavefront 0 runs the epilogue): dequantization constants, bias,
  // and the first block of 32 outlier columns: lane (feature 16r + tl,
  // outliers 8*q4 .. +7) of W_out, and of X_out (token 16tt + tl)
  auto outlier_col = [&](int rk) {  // column of outlier rank rk < n
    if constexpr (ONE) return select_rank(sm_mask, sm_pref, nwords, rk);
    else return min(max(in.idx[rk], 0), K - 1);  // (clamped: never a read outside W)
  };
  auto gather_w = [&](int blk, v8h(&ow)[R]) {
    const int rk = 32 * blk + (lane & 31);
    const int kcol = rk < n ? outlier_col(rk) : 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      uint16_t h[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int tt = 8 * q4 + e;
        const int k = __shfl(kcol, tt, kWave);
        h[e] = 32 * blk + tt < n ? out_weight(in.src, cache_ok, n_dims, k, n0 + 16 * r + tl, N, KB)
                                 : (uint16_t)0;
      }
      __builtin_memcpy(&ow[r], h, 16);
    }
  };
  auto gather_x = [&](int blk, v8h(&ox)[T]) {
    if constexpr (ONE) {  // the one row's outlier values
      const int rk = 32 * blk + (lane & 31);
      const int kcol = rk < n ? outlier_col(rk) : 0;
      uint16_t h[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int tt = 8 * q4 + e;
        const int k = __shfl(kcol, tt, kWave);
        h[e] = (tl == 0 && 32 * blk + tt < n) ? in.X[k] : (uint16_t)0;
      }
      __builtin_memcpy(&ox[0], h, 16);
    } else {
#pragma unroll
      for (int tt = 0; tt < T; ++tt) ox[tt] = load_out16(in.Xout, 16 * tt + tl, epi.KBo, blk, npad);
    }
  };
  const int fq = 4 * q4;
  float rx[T];
  float4 wv4[R];
  uint2 bv[R];
  v8h ow[R], ox[T];
  auto epilogue_loads = [&]() {
#pragma unroll
    for (int tt = 0; tt < T; ++tt) {
      const int m = 16 * tt + tl;
      if constexpr (ONE) rx[tt] = m == 0 ? ax1 / 127.0f : 0.0f;
      else rx[tt] = m < M ? in.xabs[m] / 127.0f : 0.0f;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int nn = n0 + 16 * r;
      wv4[r] = *reinterpret_cast<const float4*>(epi.wabs + nn + fq);
      bv[r] = epi.bias ? *reinterpret_cast<const uint2*>(epi.bias + nn + fq) : make_uint2(0u, 0u);
    }
    if (n > 0) {
      gather_w(0, ow);
      gather_x(0, ox);
    }
  };
  // issued before the K loop, so their latency hides under it; except at
  // 12 row blocks, where holding them through the loop spilled registers
  // (the 175B-scale FFN expansion decode, N = 49152: 99.0 against 107.5 us
  // of kernel with them issued after it)
  constexpr bool kEarlyEpilogue = R < 12;
  if (kEarlyEpilogue && w == 0) epilogue_loads();

  // 4. the K loop
  v4i acc[R][T];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int tt = 0; tt < T; ++tt) acc[r][tt] = v4i{};
  auto compute = [&](const v4i(&wv)[R][U], const v4i(&xv)[T][U]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int tt = 0; tt < T; ++tt) acc[r][tt] = mfma16_i8(wv[r][u], xv[tt][u], acc[r][tt]);
  };
  int it = 0;
  if (nit > 0) {
    for (; it + 1 < nit; it += 2) {
      const int kb = kb0 + it * U;
      compute(wa, xa);
      const int k2 = min(kb + 2 * U, klast);
      load_w(k2, wa);
      load_x(k2, xa);
      compute(wb, xb);
      const int k3 = min(kb + 3 * U, klast);
      load_w(k3, wb);
      load_x(k3, xb);
    }
    if (it < nit) compute(wa, xa);  // odd iteration count: the last one
  }
  if constexpr (U == 2) {
    for (int kb = kb0 + nit * U; kb < kb1; ++kb) {  // the one remaining block
      v4i w1[R], x1[T];
#pragma unroll
      for (int r = 0; r < R; ++r)
        w1[r] = __builtin_nontemporal_load(
            reinterpret_cast<const v4i*>(wp + r * rbytes + (size_t)kb * 1024));
      if constexpr (ONE) {
        x1[0] = tl == 0 ? *reinterpret_cast<const v4i*>(sm_x + kb * 64 + 16 * q4) : v4i{};
      } else {
#pragma unroll
        for (int tt = 0; tt < T; ++tt)
          x1[tt] = *reinterpret_cast<const v4i*>(xp + tt * rbytes + (size_t)kb * 1024);
      }
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int tt = 0; tt < T; ++tt) acc[r][tt] = mfma16_i8(w1[r], x1[tt], acc[r][tt]);
    }
  } else if (kb1 > kb0 + nit * U) {
    // the remaining kb1 - kr < U blocks: their loads issued together
    // (clamped to the last block, as in the loop), then the MFMAs of those
    // that exist
    const int kr = kb0 + nit * U;
    v4i w1[R][U - 1], x1[T][U - 1];
#pragma unroll
    for (int u = 0; u < U - 1; ++u) {
      const int kb = min(kr + u, kb1 - 1);
#pragma unroll
      for (int r = 0; r < R; ++r)
        w1[r][u] = __builtin_nontemporal_load(
            reinterpret_cast<const v4i*>(wp + r * rbytes + (size_t)kb * 1024));
      if constexpr (ONE) {
        x1[0][u] = tl == 0 ? *reinterpret_cast<const v4i*>(sm_x + kb * 64 + 16 * q4) : v4i{};
      } else {
#pragma unroll
        for (int tt = 0; tt < T; ++tt)
          x1[tt][u] = *reinterpret_cast<const v4i*>(xp + tt * rbytes + (size_t)kb * 1024);
      }
    }
#pragma unroll
    for (int u = 0; u < U - 1; ++u) {
      if (kr + u < kb1) {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int tt = 0; tt < T; ++tt) acc[r][tt] = mfma16_i8(w1[r][u], x1[tt][u], acc[r][tt]);
      }
    }
  }

  if (!kEarlyEpilogue && w == 0) epilogue_loads();

  // 5. the K-splitting wavefronts' partial sums, combined in LDS
  if constexpr (KS > 1) {
    if (w > 0) {
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int tt = 0; tt < T; ++tt) red[w - 1][r][tt][lane] = acc[r][tt];
    }
    __syncthreads();
    if (w > 0) return;
#pragma unroll
    for (int s2 = 0; s2 < KS - 1; ++s2)
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int tt = 0; tt < T; ++tt) acc[r][tt] += red[s2][r][tt][lane];
  }

  // 6. dequantize (+ bias), outlier product, fp16 store
  const bool has_bias = epi.bias != nullptr;
  v4f y[R][T];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float wq[4] = {wv4[r].x / 127.0f, wv4[r].y / 127.0f, wv4[r].z / 127.0f,
                         wv4[r].w / 127.0f};
    const float bq[4] = {h2f((uint16_t)(bv[r].x & 0xffffu)), h2f((uint16_t)(bv[r].x >> 16)),
                         h2f((uint16_t)(bv[r].y & 0xffffu)), h2f((uint16_t)(bv[r].y >> 16))};
#pragma unroll
    for (int tt = 0; tt < T; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        y[r][tt][i] = (float)acc[r][tt][i] * rx[tt] * wq[i];
        if (has_bias) y[r][tt][i] += bq[i];
      }
  }
  const int nblk = (n + 31) >> 5;
  for (int blk = 0; blk < nblk; ++blk) {
    // this workgroup's slice of W_out^T (and, M == 1, the one X_out row)
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (32 * blk + 8 * q4 < npad)
        *reinterpret_cast<v8h*>(out_elem16(in.WoutT, n0 + 16 * r + tl, 32 * blk + 8 * q4, epi.KBo)) = ow[r];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int tt = 0; tt < T; ++tt) y[r][tt] = mfma16_f16(ow[r], ox[tt], y[r][tt]);
    if (blk + 1 < nblk) {
      gather_w(blk + 1, ow);
      gather_x(blk + 1, ox);
    }
  }
  // more outlier columns than n_cap: not the method's result, so it leaves
  // as NaN rather than as a plausible wrong value
  if (n_all > epi.n_cap) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int tt = 0; tt < T; ++tt)
        y[r][tt] = v4f{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
  }
#pragma unroll
  for (int tt = 0; tt < T; ++tt) {
    const int m = 16 * tt + tl;
    if (m < M) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint32_t lo = (uint32_t)f2h(y[r][tt][0]) | ((uint32_t)f2h(y[r][tt][1]) << 16);
        const uint32_t hi = (uint32_t)f2h(y[r][tt][2]) | ((uint32_t)f2h(y[r][tt][3]) << 16);
        *reinterpret_cast<uint2*>(epi.Y + (size_t)m * N + n0 + 16 * r + fq) = make_uint2(lo, hi);
      }
    }
  }
}

template <int R, int KS>
static hipError_t run_decode_i32(const int8_t* Xi8, const int8_t* Wi8, int M, int N, int K,
                                 int32_t* acc, hipStream_t st) {
  constexpr int U = 2;
  const int KB = (int)(pack_kpad(K) / 64);
  const dim3 grid(N / (16 * R)), block(KS * 64);
  if constexpr (KS == 2) {  // 33-64 tokens: two wavefronts (as in the matmul)
    if (M > 48) {
      k_decode_i32<R, KS, U, 4><<<grid, block, 0, st>>>(Xi8, Wi8, M, N, KB, acc);
      return hipGetLastError();
    }
    if (M > 32) {
      k_decode_i32<R, KS, U, 3><<<grid, block, 0, st>>>(Xi8, Wi8, M, N, KB, acc);
      return hipGetLastError();
    }
  }
  if (M > 16)
    k_decode_i32<R, KS, U, 2><<<grid, block, 0, st>>>(Xi8, Wi8, M, N, KB, acc);
  else
    k_decode_i32<R, KS, U, 1><<<grid, block, 0, st>>>(Xi8, Wi8, M, N, KB, acc);
  return hipGetLastError();
}

template <int R>
static hipError_t run_decode_i32_ks(int ks, const int8_t* Xi8, const int8_t* Wi8, int M, int N,
                                    int K, int32_t* acc, hipStream_t st) {
  if constexpr (R != 3) {  // decode_config never gives R = 3 eight wavefronts
    if (ks >= 8 && M <= kDecodeMaxM) return run_decode_i32<R, 8>(Xi8, Wi8, M, N, K, acc, st);
  }
  return run_decode_i32<R, 2>(Xi8, Wi8, M, N, K, acc, st);
}

// Row blocks per workgroup R in {1,2,3,4} (dividing N/16) and K-splitting
// wavefronts KS in {2,8}.  Every weight fragment meets T activation
// fragments, so the activation reads from L2 are T/R of the weight bytes:
// R >= 3 streams fastest.  The workgroups all run at once, so the busiest
// compute unit sets the time: score(R) = speed(R) * (workgroups per unit
// on average / on the busiest unit), with speed 0.7, 0.88, 1.0, 1.0 for
// R = 1..4 (balanced 175B-scale shapes, M = 32).  At N = 36864 that picks
// R = 3 (768 workgroups, 3 per unit: 80 us against 90 us for R = 4 or
// R = 2 at 4.5 per unit); at N = 49152 R = 4.  KS is 2 unless the
// workgroups fill at most two thirds of the units, where 8 wavefronts per
// workgroup hold more loads in flight on the busy ones.  With weights
// streaming from HBM and M = 32, two wavefronts ran the 175B-scale output
// projection (N = 12288, R = 3, 256 workgroups) in 36.7 against 38.35 us
// per call with eight, and the 13B-scale QKV (N = 15360, R = 4, 240
// workgroups) in 24.4 against 25.6 us (3 paired runs each); at 160
// workgroups (13B-scale output projection, R = 2) eight were 0.4 us
// faster.  R = 3 is never picked with 8 (R = 1 or 2 wins wherever its
// workgroups are that few).  I8MM_DECODE_CFG = 10*R + KS forces a
// configuration for tuning sweeps (within the instantiated set).
void decode_config(int N, int* R_out, int* ks_out, bool wide) {
  static const int cfg = [] {
    const char* s = getenv("I8MM_DECODE_CFG");
    return s ? atoi(s) : 0;
  }();
  const int nrb = N / 16;
  const int cus = device_cu_count();
  // Wide workgroups: when the row blocks split into exactly one workgroup
  // per compute unit of R in {5, 6, 8, 9, 12} row blocks, two wavefronts
  // each streaming R blocks per K step.  The activation fragments are then
  // re-read from the L2 2/R times per weight byte instead of 2/3: on the
  // 175B-scale QKV decode (R = 9) the kernel ran 73.3 us against 75.2 us
  // with R = 3 and four wavefronts per unit (four or eight wavefronts per
  // wide workgroup were slower).
  if (wide && cfg == 0 && nrb % cus == 0) {
    const int r = nrb / cus;
    if (r == 5 || r == 6 || r == 8 || r == 9 || r == 12) {
      *R_out = r;
      *ks_out = 2;
      return;
    }
  }
  int R = 1;
  double best = -1.0;
  static const double speed[5] = {0.0, 0.70, 0.88, 1.0, 1.0};
  for (int r = 4; r >= 1; --r) {
    if (nrb % r) continue;
    const double wgs = (double)(nrb / r), rounds = (double)((nrb / r + cus - 1) / cus);
    const double score = speed[r] * (wgs / cus) / rounds;
    if (score > best + 1e-9) {
      best = score;
      R = r;
    }
  }
  int ks = 3 * (nrb / R) <= 2 * cus ? 8 : 2;
  if (cfg > 0 && cfg / 10 >= 1 && cfg / 10 <= 4 && nrb % (cfg / 10) == 0) {
    R = cfg / 10;
    ks = cfg % 10;
  }
  *R_out = R;
  *ks_out = ks >= 8 && R != 3 ? 8 : 2;
}

hipError_t launch_decode_i32(const int8_t* Xi8, const int8_t* Wi8, int M, int N, int K,
                             int32_t* acc, hipStream_t st) {
  int R = 1, ks = 2;
  decode_config(N, &R, &ks, false);
  switch (R) {
    case 4: return run_decode_i32_ks<4>(ks, Xi8, Wi8, M, N, K, acc, st);
    case 3: return run_decode_i32_ks<3>(ks, Xi8, Wi8, M, N, K, acc, st);
    case 2: return run_decode_i32_ks<2>(ks, Xi8, Wi8, M, N, K, acc, st);
    default: return run_decode_i32_ks<1>(ks, Xi8, Wi8, M, N, K, acc, st);
  }
}

// K blocks per iteration of the decode K loop, double-buffered, so a
// wavefront keeps 2*R*U KB of weights in flight: 4 for the two-wavefront
// workgroups of 2 or 3 row blocks, else 2.  With weights streaming from
// HBM and M = 32 (2 paired runs each): N = K = 8192 (R = 2) 22.5 against
// 24.2 us per call, N = K = 12288 (R = 3) 35.6 against 36.25 us; R = 4
// (N = 15360, K = 5120) was 0.5 us slower with 4, and 6 gained nothing
// over 4.
// With 3 or 4 token blocks the activation fragments double the registers of
// a K step, so those keep U = 2.
constexpr int decode_unroll(int R, int KS, int T) {
  return T <= 2 && KS == 2 && (R == 2 || R == 3) ? 4 : 2;
}

// 49-64 tokens (4 token blocks) in the wide workgroups of 5 or 6 row
// blocks only (8-12 spilled).  Against the tiled GEMM (2 runs each):
// 56x12288x24576 64.0 against 93.8 us, 64x12288x20480 56.6 against 68.5
// us, 64x5120x20480 34.0 against 37.9 us, 49x5120x24576 37.3 against 37.5.
static bool wide_fits_4(int N) {
  const int cus = device_cu_count(), nrb = N / 16;
  return nrb % cus == 0 && (nrb / cus == 5 || nrb / cus == 6);
}

// M <= 32: always.  33-48 tokens (3 token blocks): always; against the
// tiled GEMM the call took 89.3 against 118.6 us at 48x12288x36864, 39.8
// against 65.1 us at 48x12288x12288, 22.3 against 32.1 us at 48x5120x5120,
// and 110.7-112.5 against 130.8-132.4 us at N = 49152 (with the wide
// workgroups of decode_choice).  49-64
// tokens (4 token blocks): for N <= 16384 (64x5120x15360: 30.5 against
// 37.2 us) and where the wide workgroups of 5 or 6 row blocks apply
// (wide_fits_4); with at most 4 row blocks, at 64x5120x20480 (38.7 against
// 37.4 us) and 64x12288x49152 (144.6 against 136.9 us) the tiled GEMM was
// faster.
bool use_decode(int M, int N) {
  if (M <= kDecodeMaxM) return true;
  if (M > decode_max_m()) return false;
  return M <= 48 || N <= 16384 || wide_fits_4(N);
}

int decode_max_m() {
  static const int m = [] {
    const char* s = getenv("I8MM_DECODE_MAXM");
    const int v = s ? atoi(s) : kDecodeWideMaxM;
    return v < kDecodeMaxM ? kDecodeMaxM : v > kDecodeWideMaxM ? kDecodeWideMaxM : v;
  }();
  return m;
}

template <int R, int KS, int T, bool ONE>
static hipError_t run_decode_mm(const int8_t* Wi8, int M, int N, int K, const Epilogue& epi,
                                const DecodeInputs& in, hipStream_t st, const KernelEvents* ev) {
  constexpr int U = decode_unroll(R, KS, T);
  constexpr size_t kMaxDyn = 8 * INT8MM_MAX_K_WORDS + 65536;
  const int KB = (int)(pack_kpad(K) / 64);
  const int nwords = (K + 31) / 32, nwp = (nwords + 3) & ~3;
  const size_t shm = ONE ? 8 * (size_t)nwp + (size_t)KB * 64 : 0;
  const dim3 grid(N / (16 * R)), block(KS * 64);
  auto kern = k_decode_mm<R, KS, U, T, ONE>;
  if constexpr (ONE) {  // the dynamic-LDS limit is raised once per device
    static std::atomic<uint64_t> attr_set{0};
    int dev = 0;
    (void)hipGetDevice(&dev);
    const uint64_t bit = 1ull << (dev & 63);
    if (!(attr_set.load(std::memory_order_relaxed) & bit)) {
      const hipError_t e = hipFuncSetAttribute(
          (const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxDyn);
      if (e != hipSuccess) return e;
      attr_set.fetch_or(bit, std::memory_order_relaxed);
    }
  }
  if (ev)
    hipExtLaunchKernelGGL(kern, grid, block, (uint32_t)shm, st, ev->start, ev->stop, 0u, Wi8, M, N,
                          KB, epi, in);
  else
    kern<<<grid, block, shm, st>>>(Wi8, M, N, KB, epi, in);
  return hipGetLastError();
}

template <int R, int KS>
static hipError_t run_decode_mm_t(const int8_t* Wi8, int M, int N, int K, const Epilogue& epi,
                                  const DecodeInputs& in, hipStream_t st, const KernelEvents* ev) {
  if (M == 1) return run_decode_mm<R, KS, 1, true>(Wi8, M, N, K, epi, in, st, ev);
  if (M <= 16) return run_decode_mm<R, KS, 1, false>(Wi8, M, N, K, epi, in, st, ev);
  // 33-64 tokens: two wavefronts (with eight, 256 registers per lane, 4
  // row blocks spilled); 3 token blocks also in the wide workgroups, 4 only
  // up to 4 row blocks (8-12 spilled)
  if constexpr (KS == 2) {
    if constexpr (R <= 6)
      if (M > 48) return run_decode_mm<R, KS, 4, false>(Wi8, M, N, K, epi, in, st, ev);
    if (M > 32) return run_decode_mm<R, KS, 3, false>(Wi8, M, N, K, epi, in, st, ev);
  }
  return run_decode_mm<R, KS, 2, false>(Wi8, M, N, K, epi, in, st, ev);
}

template <int R>
static hipError_t run_decode_mm_ks(int ks, const int8_t* Wi8, int M, int N, int K,
                                   const Epilogue& epi, const DecodeInputs& in, hipStream_t st,
                                   const KernelEvents* ev) {
  // the wide workgroups run two wavefronts; decode_config never gives
  // R = 3 eight
  if constexpr (R <= 4 && R != 3) {
    if (ks >= 8 && M <= kDecodeMaxM) return run_decode_mm_t<R, 8>(Wi8, M, N, K, epi, in, st, ev);
  }
  return run_decode_mm_t<R, 2>(Wi8, M, N, K, epi, in, st, ev);
}

// Up to 48 tokens the wide workgroups too (3 token blocks fit their
// registers; 4 spilled): 33-48 tokens at N = 49152 (R = 12) took 110.7-112.5
// against 130.5-132.7 us with R = 4, at N = 36864 (R = 9) 82.8-84.3 against
// 89.3-89.4 us, at N = 24576 (R = 6) 59.8-61.3 against 65.1-65.8 us, at
// N = 20480 (R = 5) 31.4-31.6 against 35.4-35.5 us.  Above 32 tokens two
// wavefronts.
void decode_choice(int M, int N, int* R, int* ks) {
  decode_config(N, R, ks, M <= 48 || wide_fits_4(N));
  if (M > kDecodeMaxM) *ks = 2;
}

hipError_t launch_decode_mm(const int8_t* Wi8, int M, int N, int K, const Epilogue& epi,
                            const DecodeCall& c, hipStream_t st, const KernelEvents* ev) {
  int R = 1, ks = 2;
  decode_choice(M, N, &R, &ks);
  const DecodeInputs in{c.X,    c.alpha, c.colmax, c.mask_out, c.Xi8, c.xabs,
                        c.Xout, c.WoutT, c.idx,    c.hdr,      c.src, K};
  switch (R) {
    case 12: return run_decode_mm_ks<12>(ks, Wi8, M, N, K, epi, in, st, ev);
    case 9: return run_decode_mm_ks<9>(ks, Wi8, M, N, K, epi, in, st, ev);
    case 8: return run_decode_mm_ks<8>(ks, Wi8, M, N, K, epi, in, st, ev);
    case 6: return run_decode_mm_ks<6>(ks, Wi8, M, N, K, epi, in, st, ev);
    case 5: return run_decode_mm_ks<5>(ks, Wi8, M, N, K, epi, in, st, ev);
    case 4: return run_decode_mm_ks<4>(ks, Wi8, M, N, K, epi, in, st, ev);
    case 3: return run_decode_mm_ks<3>(ks, Wi8, M, N, K, epi, in, st, ev);
    case 2: return run_decode_mm_ks<2>(ks, Wi8, M, N, K, epi, in, st, ev);
    default: return run_decode_mm_ks<1>(ks, Wi8, M, N, K, epi, in, st, ev);
  }
}

}  // namespace i8mm
