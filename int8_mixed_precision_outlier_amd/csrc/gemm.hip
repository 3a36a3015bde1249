// Tiled int8 MFMA GEMM for the prefill shapes (M > 32) with the fused
// dequantize + fp16-outlier epilogue (gfx950).
//
//   Out_i32 = X_i8[M][K] . W_i8[N][K]^T   (developer.aliyun.com "LLM.int8()"
//   图2: the 8-bit matmul with int32 output), then epilogue.hpp.
//
// Structure: a workgroup owns a BM x BN output tile and walks K in 64-byte
// tiles.  Both operands are K-contiguous, so each 16-byte global load feeds
// one 16-byte LDS row segment and each MFMA lane reads 16 consecutive k of
// one row back out of LDS.  LDS rows are padded by 16 bytes: the row stride
// is an odd number of 16-byte chunks, which keeps the rows that one MFMA
// operand read touches on distinct bank groups.
// Tiles are mapped XCD-aware: consecutive workgroup ids land on different
// XCDs round-robin, so the id is remapped to give each XCD a contiguous run
// of tiles, ordered M-fastest inside groups of `groupM` M-tiles so tiles
// sharing a weight panel run together on the same L2.
#include "common.hpp"
#include "epilogue.hpp"
#include "launch.hpp"

#include <stdlib.h>

#include <type_traits>
#include <utility>

namespace i8mm {

template <int BM, int BN, int WM, int WN, int PF>
struct GemmCfg {
  static_assert(PF >= 1 && PF <= 3, "prefetch depth");
  static constexpr int BK = 64;                     // K bytes per stage
  static constexpr int STAGES = 3;                  // LDS ring depth
  static constexpr int NT = WM * WN * kWave;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static constexpr int LDR = BK + 16;               // LDS row stride: 5 x 16 B
  static constexpr int KC = BK / 16;                // 16-byte chunks per row
  static constexpr int W_LD = BN * KC / NT;         // W chunks per thread
  static constexpr int X_LD = BM * KC / NT;         // X chunks per thread
  static constexpr int NL = W_LD + X_LD;
  static constexpr int STAGE = (BM + BN) * LDR;     // bytes per LDS stage
  static constexpr int SMEM = STAGES * STAGE;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be 32-aligned");
  static_assert((BN * KC) % NT == 0 && (BM * KC) % NT == 0, "load split");
  static_assert(NT % KC == 0, "a thread's chunks share one column offset");
  static_assert(SMEM <= 160 * 1024, "LDS budget");
};

// Instruction interleaving for one half of a K tile: H MFMAs, with NR LDS
// reads followed by NW instructions of class MASKW (LDS writes or global
// loads) spread evenly in front of them.  sched_group_barrier pins the
// order; without it the scheduler issues each LDS read right before the
// MFMA that consumes it and the matrix pipe waits on LDS latency.
constexpr int kSgMfma = 0x008, kSgDsRead = 0x100, kSgDsWrite = 0x200, kSgVmemRead = 0x020;

template <int I, int H, int NR, int NW, int MASKW>
__device__ __forceinline__ void interleave_slot() {
  constexpr int L = NR + NW;
  constexpr int a = I * L / H, b = (I + 1) * L / H;
  constexpr int nr = (b < NR ? b : NR) - (a < NR ? a : NR);
  constexpr int nw = (b > NR ? b - NR : 0) - (a > NR ? a - NR : 0);
  if constexpr (nr > 0) __builtin_amdgcn_sched_group_barrier(kSgDsRead, nr, 0);
  if constexpr (nw > 0) __builtin_amdgcn_sched_group_barrier(MASKW, nw, 0);
  __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
}

template <int H, int NR, int NW, int MASKW, int... Is>
__device__ __forceinline__ void interleave(std::integer_sequence<int, Is...>) {
  (interleave_slot<Is, H, NR, NW, MASKW>(), ...);
}

// Pipeline (per K tile kt; LDS stage kt % 3):
//   * tiles kt and kt+1 are in LDS, the fragments of tile kt's first 32-byte
//     substep are in registers, tiles kt+2 .. kt+1+PF are in flight in PF
//     sets of staging registers;
//   * read substep 1 of tile kt, run the MFMAs of substep 0; read substep 0
//     of tile kt+1, run the MFMAs of substep 1;
//   * write tile kt+2 into the stage that tile kt-1 used, reuse its
//     registers for the loads of tile kt+2+PF; one barrier.
// The MFMAs never wait for the barrier: the fragments they use were read
// before it.  A global load has PF whole K tiles of MFMAs to land, which is
// what hides the L2-miss latency with one workgroup per CU.
template <int BM, int BN, int WM, int WN, int PF, bool F16>
__global__ __launch_bounds__(WM* WN * 64) void k_gemm(
    const int8_t* __restrict__ Xi8, const int8_t* __restrict__ Wi8, int M, int N, int K,
    Epilogue epi, int32_t* __restrict__ acc_out, int tilesM, int tilesN, int groupM) {
  using C = GemmCfg<BM, BN, WM, WN, PF>;
  constexpr int BK = C::BK;
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

  // ---- global -> register staging through buffer loads.  One descriptor
  // per operand whose base advances with k0 (scalar work); each thread's
  // chunk offsets are fixed 32-bit VGPR values.  The hardware range check
  // returns 0 for tile rows past M or N (those only feed outputs that are
  // never stored).  Only a K tail (K % BK != 0) needs explicit masking: its
  // out-of-range chunks get an offset beyond the descriptor's range.
  constexpr int RSTEP = C::NT / C::KC;  // rows between a thread's chunks
  const int row0 = t / C::KC, kc0 = (t % C::KC) * 16;
  const uint32_t wv0 = (uint32_t)(n0 + row0) * (uint32_t)K + kc0;
  const uint32_t xv0 = (uint32_t)(m0 + row0) * (uint32_t)K + kc0;
  const uint32_t vstep = (uint32_t)RSTEP * (uint32_t)K;
  const int lds0 = row0 * C::LDR + kc0;
  const int KT = (K + BK - 1) / BK;  // all K tiles
  const int KTF = K / BK;            // tiles without a K tail
  const uint32_t wsize = (uint32_t)N * (uint32_t)K, xsize = (uint32_t)M * (uint32_t)K;
  // Tiles at or past KT load as zeros: their chunks are all out of range
  // (the descriptor's record count is clamped at 0, so nothing past the
  // buffer is ever addressed).
  auto gload = [&](int tile, uint4(&r)[C::NL]) {
    // tile is wave-uniform; say so, or the descriptor is built per lane
    const int k0 = __builtin_amdgcn_readfirstlane(tile * BK);
    const uint32_t uk0 = (uint32_t)k0;
    // (the clamped subtraction lowers to a vector instruction; readfirstlane
    // keeps the whole descriptor in scalar registers)
    const int wrec = __builtin_amdgcn_readfirstlane((int)(wsize > uk0 ? wsize - uk0 : 0u));
    const int xrec = __builtin_amdgcn_readfirstlane((int)(xsize > uk0 ? xsize - uk0 : 0u));
    const __amdgpu_buffer_rsrc_t rw =
        __builtin_amdgcn_make_buffer_rsrc((void*)(Wi8 + k0), (short)0, wrec, 0x00020000);
    const __amdgpu_buffer_rsrc_t rx =
        __builtin_amdgcn_make_buffer_rsrc((void*)(Xi8 + k0), (short)0, xrec, 0x00020000);
    const bool kok = tile < KTF || k0 + kc0 < K;
#pragma unroll
    for (int i = 0; i < C::W_LD; ++i) {
      const uint32_t off = kok ? wv0 + i * vstep : 0x80000000u;
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)off, 0, 0);
      r[i] = make_uint4(v[0], v[1], v[2], v[3]);
    }
#pragma unroll
    for (int i = 0; i < C::X_LD; ++i) {
      const uint32_t off = kok ? xv0 + i * vstep : 0x80000000u;
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)off, 0, 0);
      r[C::W_LD + i] = make_uint4(v[0], v[1], v[2], v[3]);
    }
  };
  auto sstore = [&](int stage, const uint4(&r)[C::NL]) {
    int8_t* base = smem + stage * C::STAGE + lds0;
#pragma unroll
    for (int i = 0; i < C::W_LD; ++i)
      *reinterpret_cast<uint4*>(base + i * RSTEP * C::LDR) = r[i];
#pragma unroll
    for (int i = 0; i < C::X_LD; ++i)
      *reinterpret_cast<uint4*>(base + BN * C::LDR + i * RSTEP * C::LDR) = r[C::W_LD + i];
  };

  // ---- MFMA fragments
  const int r32 = lane & 31, h16 = (lane >> 5) * 16;
  const int fw_off = (wn * C::WTN + r32) * C::LDR + h16;
  const int fx_off = BN * C::LDR + (wm * C::WTM + r32) * C::LDR + h16;
  auto fread = [&](int stage, int sub, v4i(&fw)[C::FN], v4i(&fx)[C::FM]) {
    const int8_t* base = smem + stage * C::STAGE + sub * 32;
#pragma unroll
    for (int i = 0; i < C::FN; ++i)
      fw[i] = *reinterpret_cast<const v4i*>(base + fw_off + i * 32 * C::LDR);
#pragma unroll
    for (int j = 0; j < C::FM; ++j)
      fx[j] = *reinterpret_cast<const v4i*>(base + fx_off + j * 32 * C::LDR);
  };
  v16i acc[C::FN][C::FM];
#pragma unroll
  for (int i = 0; i < C::FN; ++i)
#pragma unroll
    for (int j = 0; j < C::FM; ++j) acc[i][j] = v16i{};
  auto mma = [&](const v4i(&fw)[C::FN], const v4i(&fx)[C::FM]) {
#pragma unroll
    for (int i = 0; i < C::FN; ++i)
#pragma unroll
      for (int j = 0; j < C::FM; ++j) acc[i][j] = mfma_i8(fw[i], fx[j], acc[i][j]);
  };

  // tile j is staged in register set j % PF; its loads are issued PF
  // iterations before its registers are written to LDS
  uint4 rg[PF][C::NL];
  v4i fw0[C::FN], fx0[C::FM], fw1[C::FN], fx1[C::FM];
  // K tiles rounded up to the unroll factor; the extra tiles are zeros
  const int KTP = (KT + 2) / 3 * 3;
  if (KT > 0) {
    gload(0, rg[0]);
    sstore(0, rg[0]);
    gload(1, rg[0]);
    sstore(1, rg[0]);
    __syncthreads();
    fread(0, 0, fw0, fx0);
#pragma unroll
    for (int j = 2; j < 2 + PF; ++j) gload(j, rg[j % PF]);
  }
  int kt = 0;
  // one K tile; ST = kt % 3 (LDS stage of tile kt), P = (kt + 2) % PF
  auto step = [&](auto ST, auto P) {
    constexpr int st = decltype(ST)::value, p = decltype(P)::value;
    v4i nw0[C::FN], nx0[C::FM];
    fread(st, 1, fw1, fx1);
    mma(fw0, fx0);
    sstore((st + 2) % 3, rg[p]);
    fread((st + 1) % 3, 0, nw0, nx0);
    mma(fw1, fx1);
    gload(kt + 2 + PF, rg[p]);
    constexpr int H = C::FN * C::FM;
    interleave<H, C::FN + C::FM, C::NL, kSgDsWrite>(std::make_integer_sequence<int, H>{});
    interleave<H, C::FN + C::FM, C::NL, kSgVmemRead>(std::make_integer_sequence<int, H>{});
#pragma unroll
    for (int i = 0; i < C::FN; ++i) fw0[i] = nw0[i];
#pragma unroll
    for (int j = 0; j < C::FM; ++j) fx0[j] = nx0[j];
    __syncthreads();
    ++kt;
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  // three iterations per trip make kt % 3 and (for PF = 1 or 3) the staging
  // set static; the loop has a single exit
  static_assert(PF == 1 || PF == 3, "PF must divide the unroll factor");
  for (kt = 0; kt < KTP;) {
    step(I0{}, std::integral_constant<int, 2 % PF>{});
    step(I1{}, std::integral_constant<int, 3 % PF>{});
    step(I2{}, std::integral_constant<int, 4 % PF>{});
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

// ---------------------------------------------------------------------------
// Direct-to-LDS variant (K % 64 == 0): the global loads write LDS themselves
// (buffer_load ... lds), so no staging registers, no ds_write instructions
// and no wait for load data sits on the wavefront's critical path.
//
// LDS holds 4 stages of one 64-byte K tile: rows [0, BN) are W rows, rows
// [BN, BN+BM) X rows, 64 bytes each.  A DMA instruction writes 64 lanes x
// 16 bytes contiguously (16 rows), so the layout is fixed by the lane order
// and the bank swizzle is applied on the source side: the 16-byte chunk of
// k-offset c of row r sits at position c ^ ((r >> 2) & 3).  With that, the
// 16 lanes of every MFMA operand read phase touch 16 distinct 16-byte bank
// groups (64 banks x 4 bytes), i.e. the reads are conflict-free.
//
// Per K tile kt (stage kt % 4): issue the DMA of tile kt+3 (its stage held
// tile kt-1, finished before the last barrier); read substep 1 of tile kt,
// run the MFMAs of substep 0; read substep 0 of tile kt+1, run the MFMAs of
// substep 1; wait until this wavefront's DMA of tile kt+2 has landed
// (vmcnt <= one tile of DMAs) and barrier, which publishes tile kt+2 to the
// whole workgroup.  A DMA has two K tiles of MFMAs to complete.
template <int BM, int BN, int WM, int WN, int STAGES, bool F16>
__global__ __launch_bounds__(WM* WN * 64) void k_gemm_dma(
    const int8_t* __restrict__ Xi8, const int8_t* __restrict__ Wi8, int M, int N, int K,
    Epilogue epi, int32_t* __restrict__ acc_out, int tilesM, int tilesN, int groupM) {
  constexpr int NWAVE = WM * WN;
  constexpr int BK = 64, ROW = 64;
  static_assert(STAGES >= 4 && STAGES <= 5, "ring depth");
  constexpr int AHEAD = STAGES - 1;            // DMA runs this many tiles ahead
  constexpr int INFLIGHT = (STAGES - 3) * (((BM + BN) / 16) / (WM * WN));
  constexpr int STAGE = (BM + BN) * ROW;
  constexpr int NDMA = (BM + BN) / 16;   // DMA instructions per stage
  constexpr int DPW = NDMA / NWAVE;      // per wavefront
  constexpr int WTM = BM / WM, WTN = BN / WN, FM = WTM / 32, FN = WTN / 32;
  static_assert(NDMA % NWAVE == 0 && BN % 16 == 0, "DMA split");
  static_assert(STAGES * STAGE <= 160 * 1024, "LDS budget");
  extern __shared__ __align__(16) int8_t smem[];

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

  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wn = w % WN, wm = w / WN;

  // ---- DMA sources: lane i of a DMA instruction fills LDS slot i of its
  // 16-row block: row i/4, position i%4, i.e. global chunk (i%4) ^ ((i>>4)&3)
  const int dchunk = ((lane & 3) ^ ((lane >> 4) & 3)) * 16;
  const int drow = lane >> 2;
  uint32_t voff[DPW];
  bool isw[DPW];
#pragma unroll
  for (int j = 0; j < DPW; ++j) {
    const int r0 = (w * DPW + j) * 16;  // first stage row of this instruction
    isw[j] = r0 < BN;
    voff[j] = isw[j] ? (uint32_t)(n0 + r0 + drow) * (uint32_t)K + dchunk
                     : (uint32_t)(m0 + r0 - BN + drow) * (uint32_t)K + dchunk;
  }
  const int KT = K / BK;
  const uint32_t wsize = (uint32_t)N * (uint32_t)K, xsize = (uint32_t)M * (uint32_t)K;
  // tiles at or past KT get an empty descriptor: every lane reads zeros
  auto dma = [&](int tile, int stage) {
    const int k0 = __builtin_amdgcn_readfirstlane(tile * BK);
    const bool live = tile < KT;
    const int wrec = __builtin_amdgcn_readfirstlane(live ? (int)(wsize - (uint32_t)k0) : 0);
    const int xrec = __builtin_amdgcn_readfirstlane(live ? (int)(xsize - (uint32_t)k0) : 0);
    const __amdgpu_buffer_rsrc_t rw =
        __builtin_amdgcn_make_buffer_rsrc((void*)(Wi8 + k0), (short)0, wrec, 0x00020000);
    const __amdgpu_buffer_rsrc_t rx =
        __builtin_amdgcn_make_buffer_rsrc((void*)(Xi8 + k0), (short)0, xrec, 0x00020000);
    int8_t* dst = smem + stage * STAGE + w * DPW * 1024;
#pragma unroll
    for (int j = 0; j < DPW; ++j)
      dma16(isw[j] ? rw : rx, dst + j * 1024, (int)voff[j]);
  };

  // ---- MFMA fragments (swizzled reads)
  const int r32 = lane & 31, hh = lane >> 5, fsw = (r32 >> 2) & 3;
  const int off0 = r32 * ROW + ((hh ^ fsw) * 16);
  const int off1 = r32 * ROW + (((2 + hh) ^ fsw) * 16);
  auto fread = [&](int stage, int sub, v4i(&fw)[FN], v4i(&fx)[FM]) {
    const int8_t* base = smem + stage * STAGE + (sub ? off1 : off0);
#pragma unroll
    for (int i = 0; i < FN; ++i)
      fw[i] = *reinterpret_cast<const v4i*>(base + (wn * WTN + i * 32) * ROW);
#pragma unroll
    for (int j = 0; j < FM; ++j)
      fx[j] = *reinterpret_cast<const v4i*>(base + (BN + wm * WTM + j * 32) * ROW);
  };
  v16i acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = v16i{};
  auto mma = [&](const v4i(&fw)[FN], const v4i(&fx)[FM]) {
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j) acc[i][j] = mfma_i8(fw[i], fx[j], acc[i][j]);
  };

  v4i fw0[FN], fx0[FM], fw1[FN], fx1[FM];
  const int KTP = (KT + STAGES - 1) / STAGES * STAGES;  // rounded up to the unroll factor
  if (KT > 0) {
#pragma unroll
    for (int j = 0; j < AHEAD; ++j) dma(j, j);
    barrier_vm<INFLIGHT>();  // tiles 0 and 1 landed in every wavefront
    fread(0, 0, fw0, fx0);
  }
  int kt = 0;
  auto step = [&](auto ST) {
    constexpr int st = decltype(ST)::value;
    v4i nw0[FN], nx0[FM];
    constexpr int H = FN * FM;
    // first half: substep-1 reads and the DMAs of tile kt+AHEAD (into the
    // stage tile kt-1 used) under the MFMAs of substep 0
    dma(kt + AHEAD, (st + AHEAD) % STAGES);
    fread(st, 1, fw1, fx1);
    mma(fw0, fx0);
    interleave<H, FN + FM, DPW, kSgVmemRead>(std::make_integer_sequence<int, H>{});
    __builtin_amdgcn_sched_barrier(0);
    // second half: the next tile's substep-0 reads under substep 1's MFMAs
    fread((st + 1) % STAGES, 0, nw0, nx0);
    mma(fw1, fx1);
    interleave<H, FN + FM, 0, kSgVmemRead>(std::make_integer_sequence<int, H>{});
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < FN; ++i) fw0[i] = nw0[i];
#pragma unroll
    for (int j = 0; j < FM; ++j) fx0[j] = nx0[j];
    barrier_vm<INFLIGHT>();  // every wavefront's DMA of tile kt+2 landed
    __builtin_amdgcn_sched_barrier(0);
    ++kt;
  };
  for (kt = 0; kt < KTP;) {
    step(std::integral_constant<int, 0>{});
    step(std::integral_constant<int, 1>{});
    step(std::integral_constant<int, 2>{});
    step(std::integral_constant<int, 3>{});
    if constexpr (STAGES == 5) step(std::integral_constant<int, 4>{});
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // no DMA may still write LDS at exit

  int n16 = 0;
  if constexpr (F16) {
    const int n = epi.hdr[1];
    n16 = (n + 15) & ~15;
  }
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int nb = n0 + wn * WTN + i * 32;
      const int mb = m0 + wm * WTM + j * 32;
      if constexpr (F16)
        store_block_f16(acc[i][j], nb, mb, M, N, n16, epi);
      else
        store_block_i32(acc[i][j], nb, mb, M, N, acc_out);
    }
}

template <int BM, int BN, int WM, int WN, int STAGES>
static hipError_t run_gemm_dma(const int8_t* Xi8, const int8_t* Wi8, int M, int N, int K,
                               const Epilogue* epi, int32_t* acc, int groupM, hipStream_t st) {
  constexpr int SMEM = STAGES * (BM + BN) * 64;
  const int tilesM = (M + BM - 1) / BM, tilesN = (N + BN - 1) / BN;
  const int gm = groupM > 0 ? (groupM < tilesM ? groupM : tilesM) : tilesM;
  const dim3 grid(tilesM * tilesN), block(WM * WN * 64);
  Epilogue e{};
  if (epi) e = *epi;
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute((const void*)k_gemm_dma<BM, BN, WM, WN, STAGES, true>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, SMEM);
    (void)hipFuncSetAttribute((const void*)k_gemm_dma<BM, BN, WM, WN, STAGES, false>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, SMEM);
    attr_set = true;
  }
  if (epi)
    k_gemm_dma<BM, BN, WM, WN, STAGES, true><<<grid, block, SMEM, st>>>(Xi8, Wi8, M, N, K, e, acc,
                                                                       tilesM, tilesN, gm);
  else
    k_gemm_dma<BM, BN, WM, WN, STAGES, false><<<grid, block, SMEM, st>>>(Xi8, Wi8, M, N, K, e,
                                                                        acc, tilesM, tilesN, gm);
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, int PF>
static hipError_t run_gemm(const int8_t* Xi8, const int8_t* Wi8, int M, int N, int K,
                           const Epilogue* epi, int32_t* acc, int groupM, hipStream_t st) {
  using C = GemmCfg<BM, BN, WM, WN, PF>;
  const int tilesM = (M + BM - 1) / BM, tilesN = (N + BN - 1) / BN;
  const int gm = groupM > 0 ? (groupM < tilesM ? groupM : tilesM) : tilesM;
  const dim3 grid(tilesM * tilesN), block(C::NT);
  Epilogue e{};
  if (epi) e = *epi;
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute((const void*)k_gemm<BM, BN, WM, WN, PF, true>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, C::SMEM);
    (void)hipFuncSetAttribute((const void*)k_gemm<BM, BN, WM, WN, PF, false>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, C::SMEM);
    attr_set = true;
  }
  if (epi)
    k_gemm<BM, BN, WM, WN, PF, true><<<grid, block, C::SMEM, st>>>(Xi8, Wi8, M, N, K, e, acc, tilesM,
                                                               tilesN, gm);
  else
    k_gemm<BM, BN, WM, WN, PF, false><<<grid, block, C::SMEM, st>>>(Xi8, Wi8, M, N, K, e, acc, tilesM,
                                                                tilesN, gm);
  return hipGetLastError();
}

// Tile configuration (tile, wavefront grid, tiles in flight): 0 = 256x256,
// 2x2 wavefronts of 128x128, 3 tiles in flight (default); 1 = same with 2;
// 2 = 128x128, 2x2 of 64x64, 3; 3 = 256x256 2x2, 1; 4 = 256x256, 2x4 of
// 128x64, 2.
// I8MM_GEMM_CFG / I8MM_GEMM_GROUPM select another configuration or M-group
// size for tuning sweeps.
hipError_t launch_gemm(const int8_t* Xi8, const int8_t* Wi8, int M, int N, int K,
                       const Epilogue* epi, int32_t* acc, hipStream_t st) {
  static const int cfg = [] {
    const char* s = getenv("I8MM_GEMM_CFG");
    return s ? atoi(s) : 0;
  }();
  static const int groupM = [] {
    const char* s = getenv("I8MM_GEMM_GROUPM");
    return s ? atoi(s) : 0;
  }();
  if (K % 64 == 0) {
    switch (cfg) {
      case 0: return run_gemm_dma<256, 256, 2, 4, 4>(Xi8, Wi8, M, N, K, epi, acc, groupM, st);
      case 5: return run_gemm_dma<256, 256, 2, 4, 5>(Xi8, Wi8, M, N, K, epi, acc, groupM, st);
      case 6: return run_gemm_dma<256, 256, 2, 2, 4>(Xi8, Wi8, M, N, K, epi, acc, groupM, st);
      case 7: return run_gemm_dma<256, 256, 2, 2, 5>(Xi8, Wi8, M, N, K, epi, acc, groupM, st);
      default: break;
    }
  }
  switch (cfg) {
    case 1: return run_gemm<256, 256, 2, 2, 1>(Xi8, Wi8, M, N, K, epi, acc, groupM, st);
    case 2: return run_gemm<128, 128, 2, 2, 3>(Xi8, Wi8, M, N, K, epi, acc, groupM, st);
    case 3: return run_gemm<256, 256, 2, 2, 1>(Xi8, Wi8, M, N, K, epi, acc, groupM, st);
    case 4: return run_gemm<256, 256, 2, 4, 1>(Xi8, Wi8, M, N, K, epi, acc, groupM, st);
    default: return run_gemm<256, 256, 2, 2, 3>(Xi8, Wi8, M, N, K, epi, acc, groupM, st);
  }
}

}  // namespace i8mm
