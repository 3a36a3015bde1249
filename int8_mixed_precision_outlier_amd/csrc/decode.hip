// Decode kernel (M <= 32): the int8 weight W_i8 (packed layout, pack.hpp)
// is streamed from HBM exactly once, every byte feeding a 16x16x64 int8
// MFMA whose 16 columns are tokens (two MFMAs per weight fragment when
// M > 16).  Bandwidth-bound: at M = 32 the product does 64 ops per weight
// byte, far below the chip's ops/byte ridge.
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
// the activations (X_i8, same layout, one or two row blocks) stay resident
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

#include <stdlib.h>

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

// R row blocks (16 features each) per workgroup; KS wavefronts split K; U
// K blocks per iteration; T token blocks of 16 (T = 2 when M > 16); F16:
// fused fp16 epilogue, else the int32 export.
template <int R, int KS, int U, int T, bool F16>
__global__ __launch_bounds__(KS * 64) void k_decode(
    const int8_t* __restrict__ Xi8, const int8_t* __restrict__ Wi8, int M, int N, int KB,
    Epilogue epi, int32_t* __restrict__ acc_out) {
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

  // lane l holds features n0 + 16r + fq .. +3 of token 16t + tl
  const int fq = 4 * (lane >> 4), tl = lane & 15;
  // epilogue operands (dequantization constants, bias, the first outlier
  // block), issued before the cross-wavefront reduction
  int n_out = 0, npad = 0;
  bool overflow = false;  // more outliers than n_cap: Y is all NaN
  float rx[T];
  float4 wv4[R];
  uint2 bv[R];
  v8h ow[R], ox[T];
  if constexpr (F16) {
    if (w == 0) {
      // clamped to the capacity the buffers were sized for
      n_out = min(max(__builtin_amdgcn_readfirstlane(epi.hdr[1]), 0), epi.n_cap);
      overflow = (__builtin_amdgcn_readfirstlane(epi.hdr[0]) & 1) != 0;
      npad = (n_out + 15) & ~15;
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const int m = 16 * t + tl;
        rx[t] = m < M ? epi.xabs[m] / 127.0f : 0.0f;
        ox[t] = n_out > 0 ? load_out16(epi.Xout, m, epi.KBo, 0, npad) : v8h{};
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int n = n0 + 16 * r;
        wv4[r] = *reinterpret_cast<const float4*>(epi.wabs + n + fq);
        bv[r] = epi.bias ? *reinterpret_cast<const uint2*>(epi.bias + n + fq) : make_uint2(0u, 0u);
        ow[r] = n_out > 0 ? load_out16(epi.WoutT, n + tl, epi.KBo, 0, npad) : v8h{};
      }
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

  if constexpr (F16) {
    const bool has_bias = epi.bias != nullptr;
    v4f y[R][T];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float wq[4] = {wv4[r].x / 127.0f, wv4[r].y / 127.0f, wv4[r].z / 127.0f,
                           wv4[r].w / 127.0f};
      const float bq[4] = {h2f((uint16_t)(bv[r].x & 0xffffu)), h2f((uint16_t)(bv[r].x >> 16)),
                           h2f((uint16_t)(bv[r].y & 0xffffu)), h2f((uint16_t)(bv[r].y >> 16))};
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          y[r][t][i] = (float)acc[r][t][i] * rx[t] * wq[i];
          if (has_bias) y[r][t][i] += bq[i];
        }
    }
    // outlier product, 32 columns (one packed block) per step, loads one
    // step ahead
    const int nblk = (n_out + 31) >> 5;
    for (int blk = 0; blk < nblk; ++blk) {
      v8h nw[R], nx[T];
      const bool more = blk + 1 < nblk;
#pragma unroll
      for (int r = 0; r < R; ++r)
        nw[r] = more ? load_out16(epi.WoutT, n0 + 16 * r + tl, epi.KBo, blk + 1, npad) : v8h{};
#pragma unroll
      for (int t = 0; t < T; ++t)
        nx[t] = more ? load_out16(epi.Xout, 16 * t + tl, epi.KBo, blk + 1, npad) : v8h{};
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int t = 0; t < T; ++t) y[r][t] = mfma16_f16(ow[r], ox[t], y[r][t]);
#pragma unroll
      for (int r = 0; r < R; ++r) ow[r] = nw[r];
#pragma unroll
      for (int t = 0; t < T; ++t) ox[t] = nx[t];
    }
    // outlier columns past the capacity were dropped: the result is not the
    // method's, so it leaves as NaN rather than as a plausible wrong value
    if (overflow) {
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int t = 0; t < T; ++t)
          y[r][t] = v4f{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""),
                        __builtin_nanf("")};
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int m = 16 * t + tl;
      if (m < M) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const uint32_t lo = (uint32_t)f2h(y[r][t][0]) | ((uint32_t)f2h(y[r][t][1]) << 16);
          const uint32_t hi = (uint32_t)f2h(y[r][t][2]) | ((uint32_t)f2h(y[r][t][3]) << 16);
          *reinterpret_cast<uint2*>(epi.Y + (size_t)m * N + n0 + 16 * r + fq) = make_uint2(lo, hi);
        }
      }
    }
  } else {
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
}

template <int R, int KS>
static hipError_t run_decode(const int8_t* Xi8, const int8_t* Wi8, int M, int N, int K,
                             const Epilogue* epi, int32_t* acc, hipStream_t st,
                             const KernelEvents* ev) {
  constexpr int U = 2;
  const int KB = (int)(pack_kpad(K) / 64);
  const dim3 grid(N / (16 * R)), block(KS * 64);
  const Epilogue e = epi ? *epi : Epilogue{};
  auto kern = M > 16 ? (epi ? k_decode<R, KS, U, 2, true> : k_decode<R, KS, U, 2, false>)
                     : (epi ? k_decode<R, KS, U, 1, true> : k_decode<R, KS, U, 1, false>);
  if (ev)
    hipExtLaunchKernelGGL(kern, grid, block, 0u, st, ev->start, ev->stop, 0u, Xi8, Wi8, M, N, KB, e,
                          acc);
  else
    kern<<<grid, block, 0, st>>>(Xi8, Wi8, M, N, KB, e, acc);
  return hipGetLastError();
}

template <int R>
static hipError_t run_decode_ks(int ks, const int8_t* Xi8, const int8_t* Wi8, int M, int N, int K,
                                const Epilogue* epi, int32_t* acc, hipStream_t st,
                                const KernelEvents* ev) {
  if (ks >= 8) return run_decode<R, 8>(Xi8, Wi8, M, N, K, epi, acc, st, ev);
  if (ks >= 4) return run_decode<R, 4>(Xi8, Wi8, M, N, K, epi, acc, st, ev);
  return run_decode<R, 2>(Xi8, Wi8, M, N, K, epi, acc, st, ev);
}

// Row blocks per workgroup R in {1,2,3,4} (dividing N/16) and K-splitting
// wavefronts KS in {2,4,8}.  Every weight fragment meets T activation
// fragments, so the activation reads from L2 are T/R of the weight bytes:
// R >= 3 streams fastest.  The workgroups all run at once, so the busiest
// compute unit sets the time: score(R) = speed(R) * (workgroups per unit
// on average / on the busiest unit), with speed 0.7, 0.88, 1.0, 1.0 for
// R = 1..4 (balanced 175B-scale shapes, M = 32).  At N = 36864 that picks
// R = 3 (768 workgroups, 3 per unit: 80 us against 90 us for R = 4 or
// R = 2 at 4.5 per unit); at N = 49152 R = 4.  KS then gives each unit
// about 6-8 wavefronts: 8 at one workgroup per unit or fewer, 4 at two, 2
// above (measured on the 13B- and 175B-scale QKV, output-projection and
// FFN shapes).  I8MM_DECODE_CFG = 10*R + KS forces a configuration for
// tuning sweeps.
void decode_config(int N, int* R_out, int* ks_out) {
  static const int cfg = [] {
    const char* s = getenv("I8MM_DECODE_CFG");
    return s ? atoi(s) : 0;
  }();
  const int nrb = N / 16;
  const int cus = device_cu_count();
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
  const int wgs = nrb / R;
  int ks = wgs <= cus ? 8 : wgs <= 2 * cus ? 4 : 2;
  if (cfg > 0 && cfg / 10 >= 1 && cfg / 10 <= 4 && nrb % (cfg / 10) == 0) {
    R = cfg / 10;
    ks = cfg % 10;
  }
  *R_out = R;
  *ks_out = ks >= 8 ? 8 : ks >= 4 ? 4 : 2;
}

hipError_t launch_decode(const int8_t* Xi8, const int8_t* Wi8, int M, int N, int K,
                         const Epilogue* epi, int32_t* acc, hipStream_t st, const KernelEvents* ev) {
  int R = 1, ks = 2;
  decode_config(N, &R, &ks);
  switch (R) {
    case 4: return run_decode_ks<4>(ks, Xi8, Wi8, M, N, K, epi, acc, st, ev);
    case 3: return run_decode_ks<3>(ks, Xi8, Wi8, M, N, K, epi, acc, st, ev);
    case 2: return run_decode_ks<2>(ks, Xi8, Wi8, M, N, K, epi, acc, st, ev);
    default: return run_decode_ks<1>(ks, Xi8, Wi8, M, N, K, epi, acc, st, ev);
  }
}

}  // namespace i8mm
