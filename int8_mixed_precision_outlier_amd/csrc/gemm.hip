// Tiled int8 MFMA GEMM for the prefill shapes (M > 32) with the fused
// dequantize + fp16-outlier epilogue (gfx950).
//
//   Out_i32 = X_i8[M][K] . W_i8[N][K]^T   (developer.aliyun.com "LLM.int8()"
//   图2: the 8-bit matmul with int32 output), then epilogue.hpp.
//
// Structure: a workgroup owns a BM x BN output tile and walks K in BK-byte
// steps.  Both operands are K-contiguous, so each 16-byte global load feeds
// one 16-byte LDS row segment and each MFMA lane reads 16 consecutive k of
// one row back out of LDS.  LDS rows are padded by 16 bytes: the row stride
// is an odd number of 16-byte chunks, which keeps the 32 rows that one MFMA
// operand read touches on distinct bank groups.  Two LDS stages: while the
// MFMAs consume stage s, the next K step is already in flight in registers.
// Tiles are mapped XCD-aware: consecutive workgroup ids land on different
// XCDs round-robin, so the id is remapped to give each XCD a contiguous run
// of tiles, ordered M-fastest inside groups of `groupM` M-tiles so tiles
// sharing a weight panel run together on the same L2.
#include "common.hpp"
#include "epilogue.hpp"
#include "launch.hpp"

#include <stdlib.h>

namespace i8mm {

template <int BM, int BN, int BK, int WM, int WN>
struct GemmCfg {
  static constexpr int NT = WM * WN * kWave;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static constexpr int LDR = BK + 16;               // LDS row stride (bytes)
  static constexpr int KC = BK / 16;                // 16-byte chunks per row
  static constexpr int W_LD = BN * KC / NT;         // W chunks per thread
  static constexpr int X_LD = BM * KC / NT;         // X chunks per thread
  static constexpr int STAGE = (BM + BN) * LDR;     // bytes per LDS stage
  static constexpr int SMEM = 2 * STAGE;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be 32-aligned");
  static_assert((BN * KC) % NT == 0 && (BM * KC) % NT == 0, "load split");
  static_assert((KC & 1) == 1 || true, "");
};

template <int BM, int BN, int BK, int WM, int WN, bool F16>
__global__ __launch_bounds__(WM* WN * 64) void k_gemm(
    const int8_t* __restrict__ Xi8, const int8_t* __restrict__ Wi8, int M, int N, int K,
    Epilogue epi, int32_t* __restrict__ acc_out, int tilesM, int tilesN, int groupM) {
  using C = GemmCfg<BM, BN, BK, WM, WN>;
  extern __shared__ __align__(16) int8_t smem[];

  // ---- tile mapping (XCD-aware, grouped along M)
  int b = blockIdx.x;
  const int T = tilesM * tilesN;
  if ((T & 7) == 0) b = (b & 7) * (T >> 3) + (b >> 3);
  const int per_group = groupM * tilesN;
  const int g = b / per_group;
  const int first_m = g * groupM;
  const int gsz = min(tilesM - first_m, groupM);
  const int tm = first_m + (b % per_group) % gsz;
  const int tn = (b % per_group) / gsz;
  const int m0 = tm * BM, n0 = tn * BN;

  const int t = threadIdx.x;
  const int lane = t & 63, w = t >> 6;
  const int wn = w % WN, wm = w / WN;

  // ---- global -> register staging
  uint4 rw[C::W_LD], rx[C::X_LD];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < C::W_LD; ++i) {
      const int q = t + i * C::NT;
      const int row = q / C::KC, kc = q % C::KC;
      const int n = n0 + row, k = k0 + kc * 16;
      rw[i] = (n < N && k < K) ? *reinterpret_cast<const uint4*>(Wi8 + (size_t)n * K + k)
                               : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < C::X_LD; ++i) {
      const int q = t + i * C::NT;
      const int row = q / C::KC, kc = q % C::KC;
      const int m = m0 + row, k = k0 + kc * 16;
      rx[i] = (m < M && k < K) ? *reinterpret_cast<const uint4*>(Xi8 + (size_t)m * K + k)
                               : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int stage) {
    int8_t* sW = smem + stage * C::STAGE;
    int8_t* sX = sW + BN * C::LDR;
#pragma unroll
    for (int i = 0; i < C::W_LD; ++i) {
      const int q = t + i * C::NT;
      *reinterpret_cast<uint4*>(sW + (q / C::KC) * C::LDR + (q % C::KC) * 16) = rw[i];
    }
#pragma unroll
    for (int i = 0; i < C::X_LD; ++i) {
      const int q = t + i * C::NT;
      *reinterpret_cast<uint4*>(sX + (q / C::KC) * C::LDR + (q % C::KC) * 16) = rx[i];
    }
  };

  v16i acc[C::FN][C::FM];
#pragma unroll
  for (int i = 0; i < C::FN; ++i)
#pragma unroll
    for (int j = 0; j < C::FM; ++j) acc[i][j] = v16i{};

  const int KT = (K + BK - 1) / BK;
  const int r32 = lane & 31, h16 = (lane >> 5) * 16;
  if (KT > 0) {
    gload(0);
    sstore(0);
    __syncthreads();
  }
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) gload((kt + 1) * BK);
    const int8_t* sW = smem + cur * C::STAGE;
    const int8_t* sX = sW + BN * C::LDR;
#pragma unroll
    for (int s = 0; s < BK / 32; ++s) {
      v4i wf[C::FN], xf[C::FM];
#pragma unroll
      for (int i = 0; i < C::FN; ++i)
        wf[i] = *reinterpret_cast<const v4i*>(sW + (wn * C::WTN + i * 32 + r32) * C::LDR + s * 32 + h16);
#pragma unroll
      for (int j = 0; j < C::FM; ++j)
        xf[j] = *reinterpret_cast<const v4i*>(sX + (wm * C::WTM + j * 32 + r32) * C::LDR + s * 32 + h16);
#pragma unroll
      for (int i = 0; i < C::FN; ++i)
#pragma unroll
        for (int j = 0; j < C::FM; ++j) acc[i][j] = mfma_i8(wf[i], xf[j], acc[i][j]);
    }
    if (kt + 1 < KT) sstore(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue
  int n16 = 0;
  if constexpr (F16) {
    const int n = epi.hdr[1];
    n16 = (n + 15) & ~15;
  }
#pragma unroll
  for (int i = 0; i < C::FN; ++i)
#pragma unroll
    for (int j = 0; j < C::FM; ++j) {
      const int nb = n0 + wn * C::WTN + i * 32;
      const int mb = m0 + wm * C::WTM + j * 32;
      if constexpr (F16)
        store_block_f16(acc[i][j], nb, mb, M, N, n16, epi);
      else
        store_block_i32(acc[i][j], nb, mb, M, N, acc_out);
    }
}

template <int BM, int BN, int BK, int WM, int WN>
static hipError_t run_gemm(const int8_t* Xi8, const int8_t* Wi8, int M, int N, int K,
                           const Epilogue* epi, int32_t* acc, int groupM, hipStream_t st) {
  using C = GemmCfg<BM, BN, BK, WM, WN>;
  const int tilesM = (M + BM - 1) / BM, tilesN = (N + BN - 1) / BN;
  const int gm = groupM > 0 ? (groupM < tilesM ? groupM : tilesM) : tilesM;
  const dim3 grid(tilesM * tilesN), block(C::NT);
  Epilogue e{};
  if (epi) e = *epi;
  if (epi) {
    auto kern = k_gemm<BM, BN, BK, WM, WN, true>;
    hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, C::SMEM);
    kern<<<grid, block, C::SMEM, st>>>(Xi8, Wi8, M, N, K, e, acc, tilesM, tilesN, gm);
  } else {
    auto kern = k_gemm<BM, BN, BK, WM, WN, false>;
    hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, C::SMEM);
    kern<<<grid, block, C::SMEM, st>>>(Xi8, Wi8, M, N, K, e, acc, tilesM, tilesN, gm);
  }
  return hipGetLastError();
}

// Tile configuration: 0 = 256x256 tile, 4 wavefronts of 128x128;
// 1 = 256x256, 8 wavefronts of 128x64; 2 = 128x128, 4 wavefronts of 64x64.
// The I8MM_GEMM_CFG / I8MM_GEMM_GROUPM environment variables select another
// configuration for tuning sweeps.
hipError_t launch_gemm(const int8_t* Xi8, const int8_t* Wi8, int M, int N, int K,
                       const Epilogue* epi, int32_t* acc, hipStream_t st) {
  static const int cfg = [] {
    const char* s = getenv("I8MM_GEMM_CFG");
    return s ? atoi(s) : 1;
  }();
  static const int groupM = [] {
    const char* s = getenv("I8MM_GEMM_GROUPM");
    return s ? atoi(s) : 0;
  }();
  switch (cfg) {
    case 0: return run_gemm<256, 256, 64, 2, 2>(Xi8, Wi8, M, N, K, epi, acc, groupM, st);
    case 2: return run_gemm<128, 128, 64, 2, 2>(Xi8, Wi8, M, N, K, epi, acc, groupM, st);
    case 3: return run_gemm<256, 256, 128, 2, 4>(Xi8, Wi8, M, N, K, epi, acc, groupM, st);
    default: return run_gemm<256, 256, 64, 2, 4>(Xi8, Wi8, M, N, K, epi, acc, groupM, st);
  }
}

}  // namespace i8mm
