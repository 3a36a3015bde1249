// Decode kernel (M <= 32): the int8 weight W_i8 (packed layout, pack.hpp)
// is streamed from HBM exactly once, every byte feeding a 32x32x32 int8
// MFMA whose 32 columns are the (at most 32) tokens.  Bandwidth-bound: at
// M = 32 the product does 64 ops per weight byte, far below the chip's
// ops/byte ridge.
//
// A workgroup owns FN*32 consecutive output features (two 16-row blocks
// each) over all of K, so no cross-workgroup reduction is needed.  Its KS
// wavefronts split the K blocks evenly and combine their int32 partial sums
// through LDS at the end (exact, order-independent).  For one 64-byte K
// block and one 32-row group, MFMA substep s takes k-chunks 2s and 2s+1:
// lane (r, h) loads row r%16 of block r/16, chunk 2s+h, so each 16-byte load
// instruction reads two contiguous 512-byte runs (whole cache lines), and a
// wavefront walks each of its row blocks contiguously along K.  U K blocks
// per iteration, the next iteration's loads issued before the current
// MFMAs; the activations (X_i8, same layout, at most two row blocks) stay
// resident in L2.  The epilogue takes the same steps as the prefill GEMM's
// (epilogue.hpp): dequantize (+ bias), fp16-MFMA outlier product, fp16
// store; its operands are loaded from global memory before the
// cross-wavefront reduction, so their latency overlaps it.
#include "common.hpp"
#include "epilogue.hpp"
#include "launch.hpp"
#include "pack.hpp"

#include <stdlib.h>

namespace i8mm {

template <int FN, int KS, int U, bool F16>
__global__ __launch_bounds__(KS * 64) void k_decode(
    const int8_t* __restrict__ Xi8, const int8_t* __restrict__ Wi8, int M, int N, int KB,
    Epilogue epi, int32_t* __restrict__ acc_out) {
  __shared__ int32_t red[KS > 1 ? KS - 1 : 1][FN][16][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = lane & 31, h = lane >> 5;
  const int n0 = blockIdx.x * (32 * FN);
  const int per = (KB + KS - 1) / KS;
  const int kb0 = min(KB, w * per);
  const int kb1 = min(KB, kb0 + per);

  // Row blocks past the padded M or past N are clamped to the last valid
  // one: they only feed MFMA outputs that are never stored.
  const int nrb = N >> 4, mrb = (M + 15) >> 4;
  const int loff = (h * 16 + (r & 15)) * 16;
  const int8_t* xp = Xi8 + (size_t)min(r >> 4, mrb - 1) * KB * 1024 + loff;
  const int8_t* wp[FN];
#pragma unroll
  for (int f = 0; f < FN; ++f)
    wp[f] = Wi8 + (size_t)min((n0 >> 4) + 2 * f + (r >> 4), nrb - 1) * KB * 1024 + loff;

  v16i acc[FN];
#pragma unroll
  for (int f = 0; f < FN; ++f) acc[f] = v16i{};

  // one iteration: U K blocks x 2 substeps
  v4i xa[U][2], wa[FN][U][2], xb[U][2], wb[FN][U][2];
  auto load = [&](int kb, v4i(&xv)[U][2], v4i(&wv)[FN][U][2]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const size_t o = (size_t)(kb + u) * 1024 + s * 512;
        xv[u][s] = *reinterpret_cast<const v4i*>(xp + o);
#pragma unroll
        for (int f = 0; f < FN; ++f) wv[f][u][s] = *reinterpret_cast<const v4i*>(wp[f] + o);
      }
  };
  auto compute = [&](const v4i(&xv)[U][2], const v4i(&wv)[FN][U][2]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int f = 0; f < FN; ++f) acc[f] = mfma_i8(wv[f][u][s], xv[u][s], acc[f]);
  };

  const int nit = (kb1 - kb0) / U;  // full iterations
  const int kbe = kb0 + nit * U;
  if (nit > 0) load(kb0, xa, wa);
  for (int it = 0; it < nit; it += 2) {
    const int kb = kb0 + it * U;
    if (it + 1 < nit) load(kb + U, xb, wb);
    compute(xa, wa);
    if (it + 1 < nit) {
      if (it + 2 < nit) load(kb + 2 * U, xa, wa);
      compute(xb, wb);
    }
  }
  for (int kb = kbe; kb < kb1; ++kb) {  // remaining blocks, one at a time
    v4i x1[1][2], w1[FN][1][2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const size_t o = (size_t)kb * 1024 + s * 512;
      x1[0][s] = *reinterpret_cast<const v4i*>(xp + o);
#pragma unroll
      for (int f = 0; f < FN; ++f) w1[f][0][s] = *reinterpret_cast<const v4i*>(wp[f] + o);
    }
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int f = 0; f < FN; ++f) acc[f] = mfma_i8(w1[f][0][s], x1[0][s], acc[f]);
  }

  // epilogue operands (dequantization constants, the first outlier k-step),
  // issued before the cross-wavefront reduction so their latency overlaps it
  int n_out = 0;
  float rx = 0.f;
  float4 wv[FN][4];
  uint2 bv[FN][4];
  const bool has_bias = epi.bias != nullptr;
  v8h ow[FN], ox = {};
  auto load_step = [&](int s2, v8h(&a)[FN], v8h& b2) {
#pragma unroll
    for (int f = 0; f < FN; ++f)
      a[f] = load_out_frag(epi.WoutT, n0 + f * 32, N, epi.KBo, s2 >> 1, s2 & 1);
    b2 = load_out_frag(epi.Xout, 0, M, epi.KBo, s2 >> 1, s2 & 1);
  };
  if constexpr (F16) {
    if (w == 0) {
      n_out = __builtin_amdgcn_readfirstlane(epi.hdr[1]);
      rx = load_rx(0, M, epi);
#pragma unroll
      for (int f = 0; f < FN; ++f) {
        load_w(n0 + f * 32, N, epi, wv[f]);
        load_bias(n0 + f * 32, N, epi, bv[f]);
      }
      if (n_out > 0) load_step(0, ow, ox);
    }
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

  if constexpr (F16) {
    v16f y[FN];
#pragma unroll
    for (int f = 0; f < FN; ++f) y[f] = dequant(acc[f], rx, wv[f], bv[f], has_bias);
    // outlier product in 16-column k-steps, loads one step ahead
    const int nsteps = (n_out + 15) >> 4;
    for (int s2 = 0; s2 < nsteps; ++s2) {
      v8h nw[FN], nx;
      if (s2 + 1 < nsteps) load_step(s2 + 1, nw, nx);
#pragma unroll
      for (int f = 0; f < FN; ++f) y[f] = mfma_f16(ow[f], ox, y[f]);
#pragma unroll
      for (int f = 0; f < FN; ++f) ow[f] = nw[f];
      ox = nx;
    }
#pragma unroll
    for (int f = 0; f < FN; ++f) store_f16(y[f], n0 + f * 32, 0, M, N, epi.Y);
  } else {
#pragma unroll
    for (int f = 0; f < FN; ++f) store_block_i32(acc[f], n0 + f * 32, 0, M, N, acc_out);
  }
}

template <int FN, int KS, int U>
static hipError_t run_decode(const int8_t* Xi8, const int8_t* Wi8, int M, int N, int K,
                             const Epilogue* epi, int32_t* acc, hipStream_t st) {
  const int KB = (int)(pack_kpad(K) / 64);
  const dim3 grid((N + 32 * FN - 1) / (32 * FN)), block(KS * 64);
  Epilogue e{};
  if (epi) {
    e = *epi;
    k_decode<FN, KS, U, true><<<grid, block, 0, st>>>(Xi8, Wi8, M, N, KB, e, acc);
  } else {
    k_decode<FN, KS, U, false><<<grid, block, 0, st>>>(Xi8, Wi8, M, N, KB, e, acc);
  }
  return hipGetLastError();
}

// Configuration: columns per workgroup = 32*FN, KS wavefronts splitting K,
// U K blocks (64 bytes) per iteration.  The default (32 columns, 2
// wavefronts, 4 blocks) streamed the 175B-scale QKV weights fastest in a
// sweep of FN in {1,2,4}, KS in {1,2,4,8}, U in {1,2,4,8}.  I8MM_DECODE_CFG selects
// another one for tuning sweeps.
hipError_t launch_decode(const int8_t* Xi8, const int8_t* Wi8, int M, int N, int K,
                         const Epilogue* epi, int32_t* acc, hipStream_t st) {
  static const int cfg = [] {
    const char* s = getenv("I8MM_DECODE_CFG");
    return s ? atoi(s) : 0;
  }();
  switch (cfg) {
    case 1: return run_decode<1, 4, 2>(Xi8, Wi8, M, N, K, epi, acc, st);
    case 2: return run_decode<2, 2, 2>(Xi8, Wi8, M, N, K, epi, acc, st);
    case 3: return run_decode<2, 4, 4>(Xi8, Wi8, M, N, K, epi, acc, st);
    case 4: return run_decode<1, 8, 2>(Xi8, Wi8, M, N, K, epi, acc, st);
    case 5: return run_decode<4, 4, 1>(Xi8, Wi8, M, N, K, epi, acc, st);
    case 6: return run_decode<2, 4, 2>(Xi8, Wi8, M, N, K, epi, acc, st);
    default: return run_decode<1, 2, 4>(Xi8, Wi8, M, N, K, epi, acc, st);
  }
}

}  // namespace i8mm
