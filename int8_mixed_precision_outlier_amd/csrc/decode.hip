// Decode kernel (M <= 32): the int8 weight W_i8[N][K] is streamed from HBM
// exactly once, every byte feeding a 32x32x32 int8 MFMA whose 32 columns are
// the (at most 32) tokens.  Bandwidth-bound: at M = 32 the product does
// 64 ops per weight byte, far below the chip's ops/byte ridge.
//
// A workgroup owns FN*32 consecutive output features (W rows) over all of K,
// so no cross-workgroup reduction is needed.  Its KS wavefronts split K
// evenly and combine their int32 partial sums through LDS at the end (exact,
// order-independent).  Each lane streams U consecutive 16-byte chunks of one
// weight row per iteration (U*16 contiguous bytes, whole cache lines per
// lane pair), with the next iteration's loads issued before the current
// MFMAs; the matching activation chunks come from the small X_i8 that stays
// resident in L2.  The epilogue is the same fused dequantize + fp16 outlier
// MFMA + fp16 store as the prefill GEMM (epilogue.hpp).
#include "common.hpp"
#include "epilogue.hpp"
#include "launch.hpp"

#include <stdlib.h>

namespace i8mm {

template <int FN, int KS, int U, bool F16>
__global__ __launch_bounds__(KS * 64) void k_decode(
    const int8_t* __restrict__ Xi8, const int8_t* __restrict__ Wi8, int M, int N, int K,
    Epilogue epi, int32_t* __restrict__ acc_out) {
  __shared__ int32_t red[KS > 1 ? KS - 1 : 1][FN][16][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = lane & 31, h = lane >> 5;
  const int n0 = blockIdx.x * (32 * FN);
  constexpr int IT = 32 * U;  // K bytes per iteration
  const int iters = (K + IT - 1) / IT;
  const int per = (iters + KS - 1) / KS;
  const int it0 = w * per;
  const int it1 = min(iters, it0 + per);

  // Rows past M (tokens) or N (features) read a clamped valid row: they only
  // feed MFMA outputs that are never stored, so no per-load predicate is
  // needed and the loads stay straight-line.
  const int8_t* xp = Xi8 + (size_t)min(r, M - 1) * K + h * 16 * U;
  const int8_t* wp[FN];
#pragma unroll
  for (int f = 0; f < FN; ++f)
    wp[f] = Wi8 + (size_t)min(n0 + f * 32 + r, N - 1) * K + h * 16 * U;

  v16i acc[FN];
#pragma unroll
  for (int f = 0; f < FN; ++f) acc[f] = v16i{};

  v4i xa[U], wa[FN][U], xb[U], wb[FN][U];
  auto load = [&](int it, v4i (&xv)[U], v4i (&wv)[FN][U]) {
    const int kb = it * IT;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      xv[u] = *reinterpret_cast<const v4i*>(xp + kb + 16 * u);
#pragma unroll
      for (int f = 0; f < FN; ++f) wv[f][u] = *reinterpret_cast<const v4i*>(wp[f] + kb + 16 * u);
    }
  };
  auto compute = [&](const v4i (&xv)[U], const v4i (&wv)[FN][U]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int f = 0; f < FN; ++f) acc[f] = mfma_i8(wv[f][u], xv[u], acc[f]);
  };

  // iterations whose IT bytes all lie inside K run unmasked
  const int full = K / IT;
  const int f1 = min(it1, full);
  if (it0 < f1) load(it0, xa, wa);
  for (int it = it0; it < f1; it += 2) {
    if (it + 1 < f1) load(it + 1, xb, wb);
    compute(xa, wa);
    if (it + 1 < f1) {
      if (it + 2 < f1) load(it + 2, xa, wa);
      compute(xb, wb);
    }
  }
  if (it1 > full && full >= it0) {  // the partial last iteration (K % IT != 0)
    const int kb = full * IT;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool kok = kb + h * 16 * U + 16 * u < K;
      xa[u] = kok ? *reinterpret_cast<const v4i*>(xp + kb + 16 * u) : v4i{};
#pragma unroll
      for (int f = 0; f < FN; ++f)
        wa[f][u] = kok ? *reinterpret_cast<const v4i*>(wp[f] + kb + 16 * u) : v4i{};
    }
    compute(xa, wa);
  }

  if constexpr (KS > 1) {
    if (w > 0) {
#pragma unroll
      for (int f = 0; f < FN; ++f)
#pragma unroll
        for (int v = 0; v < 16; ++v) red[w - 1][f][v][lane] = acc[f][v];
    }
    __syncthreads();
    if (w > 0) return;
#pragma unroll
    for (int s = 0; s < KS - 1; ++s)
#pragma unroll
      for (int f = 0; f < FN; ++f)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[f][v] += red[s][f][v][lane];
  }

  int n16 = 0;
  if constexpr (F16) {
    const int n = epi.hdr[1];
    n16 = (n + 15) & ~15;
  }
#pragma unroll
  for (int f = 0; f < FN; ++f) {
    if constexpr (F16)
      store_block_f16(acc[f], n0 + f * 32, 0, M, N, n16, epi);
    else
      store_block_i32(acc[f], n0 + f * 32, 0, M, N, acc_out);
  }
}

template <int FN, int KS, int U>
static hipError_t run_decode(const int8_t* Xi8, const int8_t* Wi8, int M, int N, int K,
                             const Epilogue* epi, int32_t* acc, hipStream_t st) {
  const dim3 grid((N + 32 * FN - 1) / (32 * FN)), block(KS * 64);
  Epilogue e{};
  if (epi) {
    e = *epi;
    k_decode<FN, KS, U, true><<<grid, block, 0, st>>>(Xi8, Wi8, M, N, K, e, acc);
  } else {
    k_decode<FN, KS, U, false><<<grid, block, 0, st>>>(Xi8, Wi8, M, N, K, e, acc);
  }
  return hipGetLastError();
}

// Configuration: columns per workgroup = 32*FN, KS wavefronts splitting K,
// U chunks of 16 bytes per lane per iteration.  I8MM_DECODE_CFG selects
// another one for tuning sweeps.
hipError_t launch_decode(const int8_t* Xi8, const int8_t* Wi8, int M, int N, int K,
                         const Epilogue* epi, int32_t* acc, hipStream_t st) {
  static const int cfg = [] {
    const char* s = getenv("I8MM_DECODE_CFG");
    return s ? atoi(s) : 0;
  }();
  switch (cfg) {
    case 1: return run_decode<1, 4, 4>(Xi8, Wi8, M, N, K, epi, acc, st);
    case 2: return run_decode<2, 2, 8>(Xi8, Wi8, M, N, K, epi, acc, st);
    case 3: return run_decode<4, 4, 4>(Xi8, Wi8, M, N, K, epi, acc, st);
    case 4: return run_decode<1, 8, 4>(Xi8, Wi8, M, N, K, epi, acc, st);
    case 5: return run_decode<2, 4, 8>(Xi8, Wi8, M, N, K, epi, acc, st);
    case 6: return run_decode<1, 2, 8>(Xi8, Wi8, M, N, K, epi, acc, st);
    default: return run_decode<2, 4, 4>(Xi8, Wi8, M, N, K, epi, acc, st);
  }
}

}  // namespace i8mm
