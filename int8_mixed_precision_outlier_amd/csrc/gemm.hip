// Tiled int8 MFMA GEMM for the prefill shapes (M above the decode range) with the fused
// dequantize + fp16-outlier epilogue (gfx950).
//
//   Out_i32 = X_i8[M][K] . W_i8[N][K]^T   (developer.aliyun.com "LLM.int8()"
//   图2: the 8-bit matmul with int32 output), then epilogue.hpp.
//
// Both operands arrive in the packed layout of pack.hpp (16-row x 64-byte
// blocks, chunk-major inside, K zero-padded to 64).  A workgroup owns a
// BM x BN output tile and walks K one 64-byte block at a time.
//
// The product runs as 16x16x64 int8 MFMAs: one 16-row x 64-byte packed
// block is exactly one MFMA operand (lane l: row l%16, chunk l/16), read
// from LDS as 1 KB contiguous.  Under random operands the chip is
// power-bound, and this shape does more work per joule than 32x32x32: an
// MFMA-only loop with changing random operands ran at 3.64 POP/s with it
// against 2.94 with 32x32x32 (4.7 and 4.6 on zeros), and the C5-scale GEMM
// went from 1.95 to 1.81 ms.
//
// Global -> LDS: direct DMA (buffer_load ... lds).  One DMA instruction moves
// one 1 KB block, contiguous in memory and in LDS, so there are no staging
// registers, no ds_write instructions and no wait for load data on the
// wavefront's critical path.  LDS holds a ring of STAGES K-tiles; a stage is
// BN/16 W blocks followed by BM/16 X blocks.  MFMA operands are read straight
// out of the chunk-major blocks: a wavefront's read takes 1 KB of
// contiguous bytes, so the reads are bank-conflict-free.
//
// Tiles are mapped XCD-aware: consecutive workgroup ids land on different
// XCDs round-robin, so the id is remapped to give each XCD a contiguous run
// of tiles, ordered M-fastest inside groups of `groupM` (4) M-tiles, so the
// tiles an XCD runs at once form a compact 4 x 8 block sharing panels in
// its L2.
#include <hip/hip_ext.h>

#include "common.hpp"
#include "epilogue.hpp"
#include "launch.hpp"
#include "pack.hpp"

#include <stdlib.h>

#include <atomic>
#include <type_traits>
#include <utility>

namespace i8mm {

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

constexpr int kOutI32 = 0, kOutF16 = 1;

// LDS of the fp16-output kernel beyond the K-loop ring: the tile's
// x_absmax, w_absmax and bias (1 KB each, filled by DMA at kernel start)
// and the first 16 outlier columns of its X_out / W_out^T rows (half a
// packed block, 512 B per 16 rows).
template <int BM, int BN>
constexpr int epi_lds_bytes() {
  return 3 * 1024 + (BM + BN) / 16 * 512;
}

// When a tile's 1 KB blocks do not split evenly over the wavefronts, every
// wavefront still issues the same number of DMAs (so the vmcnt allowances
// hold for all of them): the surplus ones read through an empty descriptor
// (no memory traffic) into a 1 KB junk region of LDS that nothing reads.
template <int BM, int BN, int NWAVE>
constexpr int junk_lds_bytes() {
  constexpr int nb = (BM + BN) / 16;
  return (nb % NWAVE != 0 || (nb / 2) % NWAVE != 0) ? 1024 : 0;
}

// The K loop: per K tile kt (stage kt % STAGES), issue the DMAs of tile
// kt+STAGES-1 into the stage tile kt-1 used (finished before the last
// barrier), half under each MFMA half.  The MFMAs of a tile run in two
// halves (the first and second half of the wavefront's activation
// fragments); the second half's activation fragments are read under the
// first half, and tile kt+1's weight and first-half activation fragments
// under the second.  Then wait until this wavefront's DMA of tile kt+2 has
// landed (the vmcnt allowance is the DMAs of the tile issued after it) and
// barrier, which publishes tile kt+2 to the whole workgroup.  A DMA has
// STAGES-2 K tiles of MFMAs to complete.  The bare barrier keeps later DMAs
// in flight (a __syncthreads fence would wait for all of them).
//
// It runs over the int8 operands with int32 accumulators.  The fp16
// output then takes the dequantized accumulators (+ bias) and adds the
// outlier product X_out . W_out with 16x16x32 fp16 MFMAs, all operands
// from LDS: the epilogue constants and the first 16 outlier columns are
// DMA'd there at kernel start, further columns (alpha -> 0) stream through
// the K loop's LDS ring, free by then.
template <int BM, int BN, int WM, int WN, int STAGES, int OUT>
__global__ __launch_bounds__(WM* WN * 64) void k_gemm(
    const int8_t* __restrict__ Xi8, const int8_t* __restrict__ Wi8, int M, int N, int KB,
    Epilogue epi, int32_t* __restrict__ acc_out, int tilesM, int tilesN, int groupM, int nbase) {
  constexpr int NWAVE = WM * WN;
  constexpr int STAGE = (BM + BN) * 64;
  constexpr int NDMA = (BM + BN) / 16;                // DMA instructions (1 KB blocks) per stage
  constexpr int DPW = (NDMA + NWAVE - 1) / NWAVE;     // per wavefront (the surplus: junk)
  constexpr int AHEAD = STAGES - 1;      // DMA runs this many tiles ahead
  constexpr int INFLIGHT = (STAGES - 3) * DPW;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 16, FN = WTN / 16;  // 16-row fragments of the wavefront tile
  constexpr int FMH = FM / 2;                  // activation fragments per half tile
  static_assert(BN % 16 == 0 && BM % 16 == 0 && FM % 2 == 0 && WTN % 16 == 0, "tiling");
  constexpr int EPI = STAGES * STAGE;  // offset of the epilogue region
  // the junk region (surplus DMAs) after the epilogue region
  constexpr int JUNK = EPI + (OUT == kOutF16 ? epi_lds_bytes<BM, BN>() : 0);
  static_assert(STAGES >= 3 && JUNK + junk_lds_bytes<BM, BN, NWAVE>() <= 160 * 1024, "LDS budget");
  extern __shared__ __align__(16) int8_t smem[];

  const int T = tilesM * tilesN;
  const int b = xcd_remap(blockIdx.x, T);
  const int per_group = groupM * tilesN;
  const int g = b / per_group;
  const int first_m = g * groupM;
  const int gsz = min(tilesM - first_m, groupM);
  const int tm = first_m + (b % per_group) % gsz;
  const int tn = (b % per_group) / gsz;
  // the launch covers the columns from nbase on, tilesN tiles of BN
  const int m0 = tm * BM, n0 = nbase + tn * BN;

  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wn = w % WN, wm = w / WN;
  const int nrb = N >> 4, mrb = (M + 15) >> 4;
  // a lane's 16 bytes of a 1 KB block: both the DMA destination and the
  // 16x16 MFMA fragment (row lane%16, k-chunk lane/16 of the chunk-major
  // block), so fragment reads are whole contiguous blocks
  const int voff = lane * 16;
  const int q4 = lane >> 4, r16 = lane & 15;
  int n_out = 0;  // outlier columns (fp16 output only)
  bool overflow = false;  // more outliers than n_cap: Y is all NaN
  // clamped to the capacity the buffers were sized for, so no workspace
  // content can send a read past them
  if constexpr (OUT != kOutI32) {
    n_out = min(max(__builtin_amdgcn_readfirstlane(epi.hdr[1]), 0), epi.n_cap);
    overflow = (__builtin_amdgcn_readfirstlane(epi.hdr[0]) & 1) != 0;
  }
  // Every column an outlier (alpha -> 0): X_i8 is all zeros and the whole
  // product is the fp16 one.  It then runs through the K loop below with
  // fp16 MFMAs over X_out / W_out^T, 32 columns per 64-byte block, except
  // for a last block whose columns stop within its first 16 (its chunks 2-3
  // are not written), which goes through the half-block path.
  const int nb32 = (n_out + 31) >> 5;
  const bool half_tail = (n_out & 31) != 0 && (n_out & 31) <= 16;
  const bool all_out = OUT == kOutF16 && n_out >= epi.K && n_out > 32;

  // The half-blocks of one 16-column outlier k-step of the tile: BN/16 of
  // W_out^T rows, then BM/16 of X_out rows; one DMA instruction moves two
  // half-blocks of one matrix (lanes 0-31 and 32-63).
  constexpr int HB = (BN + BM) / 16;
  constexpr int NHB = HB / 2;                       // DMA instructions per outlier k-step
  constexpr int DPW2 = (NHB + NWAVE - 1) / NWAVE;   // per wavefront (the surplus: junk)
  static_assert((BN / 16) % 2 == 0 && (BM / 16) % 2 == 0, "outlier DMA split");
  bool ow_w[DPW2];
  int ow_vo[DPW2];  // per-lane byte offset of the lane's row block
  auto out_dma = [&](int step, int8_t* dst, int nsteps) {
    const bool live = step < nsteps;
    const int wrecs = (int)((uint32_t)nrb * (uint32_t)epi.KBo * 1024u);
    const int xrecs = (int)((uint32_t)mrb * (uint32_t)epi.KBo * 1024u);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        (void*)epi.WoutT, (short)0, live ? wrecs : 0, 0x00020000);
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        (void*)epi.Xout, (short)0, live ? xrecs : 0, 0x00020000);
    const __amdgpu_buffer_rsrc_t r0 =
        __builtin_amdgcn_make_buffer_rsrc((void*)epi.Xout, (short)0, 0, 0x00020000);
    const int so = live ? (step >> 1) * 1024 + (step & 1) * 512 : 0;
#pragma unroll
    for (int d = 0; d < DPW2; ++d) {
      const int D = w * DPW2 + d;
      const bool real = NHB % NWAVE == 0 || D < NHB;
      dma16(real ? (ow_w[d] ? rw : rx) : r0, real ? dst + D * 1024 : smem + JUNK, ow_vo[d], so);
    }
  };
  if constexpr (OUT == kOutF16) {
    const int r32 = lane & 31, hh = lane >> 5;
#pragma unroll
    for (int d = 0; d < DPW2; ++d) {
      const int hb = (w * DPW2 + d) * 2 + hh;
      ow_w[d] = (w * DPW2 + d) * 2 < BN / 16;
      const int rb = ow_w[d] ? min(n0 / 16 + hb, nrb - 1) : min(m0 / 16 + hb - BN / 16, mrb - 1);
      ow_vo[d] = (int)((uint32_t)rb * (uint32_t)epi.KBo * 1024u) + r32 * 16;
    }
    // dequantization constants and bias of the tile (lanes past M / N read
    // zeros), and the first outlier k-step; these DMAs are older than every
    // K-loop DMA, so the K loop's waits cover them
    if (w == 0) {
      // descriptors start at the tile, so the record count bounds the lanes
      const __amdgpu_buffer_rsrc_t rxa = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(epi.xabs + m0), (short)0, (M - m0) * 4, 0x00020000);
      const __amdgpu_buffer_rsrc_t rwa = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(epi.wabs + n0), (short)0, (N - n0) * 4, 0x00020000);
      const __amdgpu_buffer_rsrc_t rbi = __builtin_amdgcn_make_buffer_rsrc(
          epi.bias ? (void*)(epi.bias + n0) : (void*)epi.wabs, (short)0, epi.bias ? (N - n0) * 2 : 0,
          0x00020000);
#pragma unroll
      for (int q = 0; q < BM / 64; ++q) dma4(rxa, smem + EPI + q * 256, lane * 4 + q * 256, 0);
#pragma unroll
      for (int q = 0; q < (BN + 63) / 64; ++q)
        dma4(rwa, smem + EPI + 1024 + q * 256, lane * 4 + q * 256, 0);
#pragma unroll
      for (int q = 0; q < (BN + 127) / 128; ++q)
        dma4(rbi, smem + EPI + 2048 + q * 256, lane * 4 + q * 256, 0);
    }
    if (n_out > 0)
      out_dma(all_out ? 2 * (nb32 - 1) : 0, smem + EPI + 3 * 1024, all_out && !half_tail ? 0 : 1 + 2 * (nb32 - 1));
  }

  // K loop over NB packed blocks of a weight-side operand Wp (N rows) and
  // an activation-side operand Xp (padded M rows), both RS blocks per row
  // block: W_i8 / X_i8 (KB blocks) with int8 MFMAs into int32
  // accumulators, or W_out^T / X_out (KBo blocks of 32 fp16 columns) with
  // fp16 MFMAs into fp32 ones.  A 16-row x 64-byte block is one MFMA
  // operand either way (16x16x64 int8, 16x16x32 fp16).  accs[i][j] covers
  // features n0 + wn*WTN + 16i .. +15 and tokens m0 + wm*WTM + 16j .. +15.
  // on_start runs once every wavefront's first tiles (and every DMA issued
  // before the loop) have landed.  Row blocks past N (or past the padded M)
  // are clamped to the last valid one: those rows only feed outputs that
  // are never stored.  Tiles at or past NB get empty descriptors (zeros).
  auto kloop = [&](auto F16, const int8_t* Wp, const int8_t* Xp, int NB, int RS, auto& accs,
                   auto&& on_start) {
    constexpr bool f16 = decltype(F16)::value;
    int sblk[DPW];  // source block row offset (row block * RS), wave-uniform
    bool isw[DPW], real[DPW];  // weight block; a real block (else a surplus DMA)
#pragma unroll
    for (int j = 0; j < DPW; ++j) {
      const int J = w * DPW + j;
      isw[j] = J < BN / 16;
      real[j] = NDMA % NWAVE == 0 || J < NDMA;
      const int rb = isw[j] ? min(n0 / 16 + J, nrb - 1) : min(m0 / 16 + J - BN / 16, mrb - 1);
      sblk[j] = __builtin_amdgcn_readfirstlane(rb * RS);
    }
    // byte counts and offsets reach 2^31 at the size limit: unsigned arithmetic
    const int wrec = (int)((uint32_t)nrb * (uint32_t)RS * 1024u);
    const int xrec = (int)((uint32_t)mrb * (uint32_t)RS * 1024u);
    auto dma = [&](int tile, int stage, int j0, int j1) {
      const bool live = tile < NB;
      const __amdgpu_buffer_rsrc_t rw =
          __builtin_amdgcn_make_buffer_rsrc((void*)Wp, (short)0, live ? wrec : 0, 0x00020000);
      const __amdgpu_buffer_rsrc_t rx =
          __builtin_amdgcn_make_buffer_rsrc((void*)Xp, (short)0, live ? xrec : 0, 0x00020000);
      const __amdgpu_buffer_rsrc_t r0 =
          __builtin_amdgcn_make_buffer_rsrc((void*)Xp, (short)0, 0, 0x00020000);
      const int kt = live ? tile : 0;
      int8_t* dst = smem + stage * STAGE + w * DPW * 1024;
#pragma unroll
      for (int j = 0; j < DPW; ++j)
        if (j >= j0 && j < j1)
          dma16(real[j] ? (isw[j] ? rw : rx) : r0, real[j] ? dst + j * 1024 : smem + JUNK, voff,
                (int)((uint32_t)(sblk[j] + kt) * 1024u));
    };
    // weight fragments of a stage, and half h of its activation fragments
    auto read_w = [&](int stage, v4i(&fw)[FN]) {
      const int8_t* base = smem + stage * STAGE + voff + (wn * WTN / 16) * 1024;
#pragma unroll
      for (int i = 0; i < FN; ++i) fw[i] = *reinterpret_cast<const v4i*>(base + i * 1024);
    };
    auto read_x = [&](int stage, int h, v4i(&fx)[FMH]) {
      const int8_t* base =
          smem + stage * STAGE + voff + (BN / 16 + wm * WTM / 16 + h * FMH) * 1024;
#pragma unroll
      for (int j = 0; j < FMH; ++j) fx[j] = *reinterpret_cast<const v4i*>(base + j * 1024);
    };
    auto mma = [&](const v4i(&fw)[FN], const v4i(&fx)[FMH], auto H) {
      constexpr int h = decltype(H)::value;
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FMH; ++j) {
          if constexpr (f16)
            accs[i][h * FMH + j] =
                mfma16_f16(__builtin_bit_cast(v8h, fw[i]), __builtin_bit_cast(v8h, fx[j]),
                           accs[i][h * FMH + j]);
          else
            accs[i][h * FMH + j] = mfma16_i8(fw[i], fx[j], accs[i][h * FMH + j]);
        }
    };

    v4i fw[FN], fxa[FMH], fxb[FMH];
    const int KTP = (NB + STAGES - 1) / STAGES * STAGES;  // rounded up to the unroll factor
    if (NB > 0) {
#pragma unroll
      for (int j = 0; j < AHEAD; ++j) dma(j, j, 0, DPW);
      barrier_vm<INFLIGHT>();  // tiles 0 and 1 landed in every wavefront
      on_start();
      read_w(0, fw);
      read_x(0, 0, fxa);
    }
    int kt = 0;
    auto step = [&](auto ST) {
      constexpr int st = decltype(ST)::value;
      v4i nw[FN], nxa[FMH];
      constexpr int H = FN * FMH;
      // first half: the second half of tile kt's activation fragments, and
      // half of the DMAs of tile kt+AHEAD, under the first half's MFMAs
      dma(kt + AHEAD, (st + AHEAD) % STAGES, 0, DPW / 2);
      read_x(st, 1, fxb);
      mma(fw, fxa, std::integral_constant<int, 0>{});
      interleave<H, FMH, DPW / 2, kSgVmemRead>(std::make_integer_sequence<int, H>{});
      __builtin_amdgcn_sched_barrier(0);
      // second half: tile kt+1's weight and first activation fragments, and
      // the other DMAs
      dma(kt + AHEAD, (st + AHEAD) % STAGES, DPW / 2, DPW);
      read_w((st + 1) % STAGES, nw);
      read_x((st + 1) % STAGES, 0, nxa);
      mma(fw, fxb, std::integral_constant<int, 1>{});
      interleave<H, FN + FMH, DPW - DPW / 2, kSgVmemRead>(std::make_integer_sequence<int, H>{});
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < FN; ++i) fw[i] = nw[i];
#pragma unroll
      for (int j = 0; j < FMH; ++j) fxa[j] = nxa[j];
      // every wavefront's DMA of tile kt+2 landed.  The FN + FMH reads of
      // tile kt+1 just issued may stay in flight: that stage is not
      // overwritten before the next barrier, and every read of tile kt's
      // stage (overwritten next) was consumed by this step's MFMAs.
      barrier_vm<INFLIGHT, FN + FMH>();
      __builtin_amdgcn_sched_barrier(0);
      ++kt;
    };
    for (kt = 0; kt < KTP;) {
      step(std::integral_constant<int, 0>{});
      step(std::integral_constant<int, 1>{});
      step(std::integral_constant<int, 2>{});
      if constexpr (STAGES >= 4) step(std::integral_constant<int, 3>{});
      if constexpr (STAGES >= 5) step(std::integral_constant<int, 4>{});
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // no DMA may still write LDS
  };

  if constexpr (OUT == kOutI32) {
    v4i acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j) acc[i][j] = v4i{};
    kloop(std::false_type{}, Wi8, Xi8, KB, KB, acc, [] {});
    // the feature blocks of one token block back to back, so each row
    // segment of the output is written by consecutive stores (merged in L2)
#pragma unroll
    for (int j = 0; j < FM; ++j)
#pragma unroll
      for (int i = 0; i < FN; ++i)
        store16_i32(acc[i][j], n0 + wn * WTN + i * 16, m0 + wm * WTM + j * 16, M, N, acc_out);
  } else {
    const float* s_xabs = reinterpret_cast<const float*>(smem + EPI);
    const float* s_wabs = reinterpret_cast<const float*>(smem + EPI + 1024);
    // (the bias region holds zeros when the layer has no bias)
    const uint16_t* s_bias = reinterpret_cast<const uint16_t*>(smem + EPI + 2048);
    constexpr float kInv127 = 1.0f / 127.0f;
    v4f y[FN][FM];
    // y = the dequantized int32 accumulators acc_of(i, j) (+ bias)
    auto dequant = [&](auto&& acc_of) {
#pragma unroll
      for (int i = 0; i < FN; ++i) {
        const int nl = wn * WTN + i * 16 + 4 * q4;  // first of the lane's 4 features in the tile
        const float4 wv = *reinterpret_cast<const float4*>(s_wabs + nl);
        const uint2 bv = *reinterpret_cast<const uint2*>(s_bias + nl);
        const float4 sw =
            make_float4(wv.x * kInv127, wv.y * kInv127, wv.z * kInv127, wv.w * kInv127);
        const float4 bf = make_float4(h2f((uint16_t)(bv.x & 0xffffu)), h2f((uint16_t)(bv.x >> 16)),
                                      h2f((uint16_t)(bv.y & 0xffffu)), h2f((uint16_t)(bv.y >> 16)));
#pragma unroll
        for (int j = 0; j < FM; ++j) {
          const float rx = s_xabs[wm * WTM + j * 16 + r16] * kInv127;
          y[i][j] = dequant16(acc_of(i, j), rx, sw, bf);
        }
      }
    };
    if (all_out) {
      // Out_i32 = 0: y starts at its dequantized value (the bias), set once
      // the epilogue constants (DMA'd before the loop) have landed
      kloop(std::true_type{}, (const int8_t*)epi.WoutT, (const int8_t*)epi.Xout,
            nb32 - (half_tail ? 1 : 0), epi.KBo, y,
            [&] { dequant([](int, int) { return v4i{}; }); });
      barrier_vm<0>();  // the half-block tail landed in every wavefront
    } else {
      v4i acc[FN][FM];
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = v4i{};
      // with every column an outlier X_i8 is all zeros: Out_i32 = 0
      if (n_out < epi.K) kloop(std::false_type{}, Wi8, Xi8, KB, KB, acc, [] {});
      // every wavefront's epilogue DMAs landed (the K loop may not have run)
      barrier_vm<0>();
      dequant([&](int i, int j) { return acc[i][j]; });
    }
    // the outlier product, fp16 MFMAs reading X_out / W_out^T from LDS;
    // lane l takes row l%16, 16-byte chunk l/16 (8 outlier columns) of a
    // 16-row block of `rbs` bytes (512: the half-blocks of the first 16
    // columns, whose chunks 2-3 do not exist; 1024: whole blocks of 32
    // columns, chunks 2-3 only where within roundup(n, 16))
    const int nsteps = (n_out + 15) >> 4;
    auto out_mma = [&](const int8_t* st, int rbs, bool hi) {
      const bool use = q4 < 2 || hi;
      v8h fw[FN], fx[FM];
#pragma unroll
      for (int i = 0; i < FN; ++i)
        fw[i] = use ? *reinterpret_cast<const v8h*>(st + (wn * WTN / 16 + i) * rbs + voff) : v8h{};
#pragma unroll
      for (int j = 0; j < FM; ++j)
        fx[j] = use ? *reinterpret_cast<const v8h*>(st + (BN / 16 + wm * WTM / 16 + j) * rbs + voff)
                    : v8h{};
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) y[i][j] = mfma16_f16(fw[i], fx[j], y[i][j]);
    };
    // Up to 16 outlier columns: the half-blocks DMA'd at kernel start.
    // More (alpha -> 0): whole 64-byte blocks (32 columns) through a ring of
    // four stages, DMA'd three blocks ahead, one barrier per block.  One
    // loop body serves both, so the two cases share their registers.
    constexpr int STG = (BM + BN) * 64;  // a whole block per 16 rows
    constexpr int NST = 4;
    static_assert(NST * STG <= EPI, "LDS");
    constexpr int DPB = DPW;  // block DMAs per wavefront per step (the surplus: junk)
    const bool big = nsteps > 1 && !all_out;
    const int nblk = all_out ? (half_tail ? 1 : 0) : big ? (n_out + 31) >> 5 : nsteps;
    const int wrecb = (int)((uint32_t)nrb * (uint32_t)epi.KBo * 1024u);
    const int xrecb = (int)((uint32_t)mrb * (uint32_t)epi.KBo * 1024u);
    auto blk_dma = [&](int blk) {
      const bool live = blk < nblk;
      const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
          (void*)epi.WoutT, (short)0, live ? wrecb : 0, 0x00020000);
      const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
          (void*)epi.Xout, (short)0, live ? xrecb : 0, 0x00020000);
      const __amdgpu_buffer_rsrc_t r0 =
          __builtin_amdgcn_make_buffer_rsrc((void*)epi.Xout, (short)0, 0, 0x00020000);
      int8_t* dst = smem + (blk % NST) * STG;
#pragma unroll
      for (int d = 0; d < DPB; ++d) {
        const int J = w * DPB + d;
        const bool isw = J < BN / 16;
        const bool real = NDMA % NWAVE == 0 || J < NDMA;
        const int rb = isw ? min(n0 / 16 + J, nrb - 1) : min(m0 / 16 + J - BN / 16, mrb - 1);
        const int so = (int)(((uint32_t)rb * (uint32_t)epi.KBo + (uint32_t)(live ? blk : 0)) * 1024u);
        dma16(real ? (isw ? rw : rx) : r0, real ? dst + J * 1024 : smem + JUNK, voff,
              __builtin_amdgcn_readfirstlane(so));
      }
    };
    if (big) {
      blk_dma(0);
      blk_dma(1);
      blk_dma(2);
    }
    for (int s2 = 0; s2 < nblk; ++s2) {
      const int8_t* st = smem + EPI + 3 * 1024;
      int rbs = 512;
      bool hi = false;
      if (big) {
        // block s2 landed in every wavefront, which are all done with the
        // stage the next DMA overwrites (that of block s2 - 1)
        barrier_vm<2 * DPB>();
        blk_dma(s2 + 3);
        st = smem + (s2 % NST) * STG;
        rbs = 1024;
        hi = 2 * s2 + 1 < nsteps;  // columns 16-31 of the block hold data
      }
      out_mma(st, rbs, hi);
    }
    if (big) __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // no DMA may still write LDS
    // outlier columns past the capacity were dropped: the result is not the
    // method's, so it leaves as NaN rather than as a plausible wrong value
    if (overflow) {
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) y[i][j] = v4f{__builtin_nanf(""), __builtin_nanf(""),
                                                   __builtin_nanf(""), __builtin_nanf("")};
    }
    // the FN blocks of one token block in a row, two at a time (an odd last
    // one alone): each 128-byte line of Y is written by consecutive stores,
    // which merge in L2
#pragma unroll
    for (int j = 0; j < FM; ++j) {
#pragma unroll
      for (int i = 0; i + 1 < FN; i += 2)
        store32_f16(y[i][j], y[i + 1][j], n0 + wn * WTN + i * 16, m0 + wm * WTM + j * 16, M, N,
                    epi.Y);
      if constexpr (FN % 2 != 0)
        store16_f16(y[FN - 1][j], n0 + wn * WTN + (FN - 1) * 16, m0 + wm * WTM + j * 16, M, N,
                    epi.Y);
    }
  }
}

// One launch over the output columns [nbase, nend) of the M x N product
// (N is also the row stride of Y and of the int32 output).  nend is N or a
// multiple of BN above nbase, so no tile crosses it.  ev: the dispatch
// records ev->start at its start (start_ev) and ev->stop at its end
// (stop_ev).
template <int BM, int BN, int WM, int WN, int STAGES>
static hipError_t run_gemm(const int8_t* Xi8, const int8_t* Wi8, int M, int N, int nbase,
                           int nend, int KB, const Epilogue* epi, int32_t* acc, int groupM,
                           hipStream_t st, const KernelEvents* ev, bool start_ev, bool stop_ev) {
  constexpr int JB = junk_lds_bytes<BM, BN, WM * WN>();
  constexpr int SMEM = STAGES * (BM + BN) * 64 + JB;
  constexpr int SMEM16 = SMEM + epi_lds_bytes<BM, BN>();  // fp16 output variant
  const int tilesM = (M + BM - 1) / BM, tilesN = (nend - nbase + BN - 1) / BN;
  // groups of 4 M-tiles: the 32 tiles an XCD runs at once then share 4
  // activation and 8 weight panels (the 175B FFN shape runs 5 % faster than
  // with all 16 M-tiles per group: less last-level-cache traffic, and the
  // kernel is power-bound)
  const int want = groupM > 0 ? groupM : 4;
  const int gm = want < tilesM ? want : tilesM;
  const dim3 grid(tilesM * tilesN), block(WM * WN * 64);
  // the dynamic-LDS limit is raised once per device the kernels run on
  static std::atomic<uint64_t> attr_set{0};
  int dev = 0;
  (void)hipGetDevice(&dev);
  const uint64_t bit = 1ull << (dev & 63);
  if (!(attr_set.load(std::memory_order_relaxed) & bit)) {
    hipError_t e = hipFuncSetAttribute((const void*)k_gemm<BM, BN, WM, WN, STAGES, kOutI32>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, SMEM);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void*)k_gemm<BM, BN, WM, WN, STAGES, kOutF16>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, SMEM16);
    if (e != hipSuccess) return e;
    attr_set.fetch_or(bit, std::memory_order_relaxed);
  }
  const Epilogue e = epi ? *epi : Epilogue{};
  auto kern = epi ? k_gemm<BM, BN, WM, WN, STAGES, kOutF16> : k_gemm<BM, BN, WM, WN, STAGES, kOutI32>;
  const uint32_t shm = epi ? SMEM16 : SMEM;
  if (ev && (start_ev || stop_ev))
    hipExtLaunchKernelGGL(kern, grid, block, shm, st, start_ev ? ev->start : nullptr,
                          stop_ev ? ev->stop : nullptr, 0u, Xi8, Wi8, M, N, KB, e, acc, tilesM,
                          tilesN, gm, nbase);
  else
    kern<<<grid, block, shm, st>>>(Xi8, Wi8, M, N, KB, e, acc, tilesM, tilesN, gm, nbase);
  return hipGetLastError();
}

int device_cu_count() {
  static std::atomic<int> cus[64];  // per device; 0 until queried
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::atomic<int>& c = cus[dev & 63];
  int n = c.load(std::memory_order_relaxed);
  if (n == 0) {
    int v = 0;
    n = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0
            ? v
            : 256;
    c.store(n, std::memory_order_relaxed);
  }
  return n;
}

// Tile configuration: 256x256 tiles (8 wavefronts of 64 tokens x 128
// features, 4 LDS stages, one workgroup per CU), 256x160 or 256x128 tiles (8
// wavefronts of 64 x 80 or 64 x 64, one per CU) or 128x128 tiles (4
// wavefronts of 64x64, two workgroups per CU).  The cost of a launch is
// counted in rounds of workgroups over the chip, in units of a 256x256
// round:
//   128x128  0.72 per round of two workgroups per CU (fitted to the 175B-
//            and 13B-scale FFN shapes for M from 48 to 1024, where it costs
//            0.65-0.82: the smaller tiles fill the chip at small M but move
//            more operand bytes per MFMA), 0.65 of that for a last round of
//            at most one workgroup per CU (1024x4096x4096: 24.6 against
//            38.0 us for 2048x4096x4096);
//   256x160  0.77 (5/8 of the work per tile, but more LDS reads per MFMA and
//            the same per-tile pipeline fill and epilogue; measured at K =
//            5120, M = 2048: 48 against 62.5 us per full round);
//   256x128  0.65 (half the work per tile; against two 128x128 workgroups
//            per CU it does the same MFMAs on 25 % fewer operand bytes:
//            2048x4096x4096 34.6 against 38.0 us, 1536x5120x5120 38.1
//            against 42.4 us).
// At M = 2048 the 256x160 tiles fill 256 CUs in one round when N = 5120,
// and the 256x128 tiles when N = 4096, where 256x256 tiles leave CUs idle.
//
// When 256x256 tiles would leave the last round partly empty, the columns
// can also be split: [0, n1) in whole rounds of 256x256 tiles, then [n1, N)
// in a second launch of the smaller tiles (the second launch's pipeline
// fill and drain counted as kGap of a round; the split is taken when it
// saves more than kMargin of a round).  2048x5120x20480 takes two rounds
// of 256x256 tiles and one round of smaller tiles instead of three 256x256
// rounds, the last one half empty.
//
// I8MM_GEMM_CFG (1: always 256x256, 3: always 128x128, 4: always 256x160,
// 5: always 256x128) and I8MM_GEMM_GROUPM select other configurations for
// tuning sweeps; I8MM_GEMM_SPLIT=0 turns the column split off and
// I8MM_GEMM_T128=0 leaves the 256x128 tiles out of the rule.
constexpr double kF128 = 0.72, kF128Half = 0.65, kF160 = 0.77, kF256x128 = 0.65, kGap = 0.04,
                 kMargin = 0.05;

static double launch_cost(int cfg, long M, long N, long cus) {
  if (N <= 0 || M <= 0) return 0.0;
  if (cfg == 3) {
    const long t = (M + 127) / 128 * ((N + 127) / 128);
    const long full = t / (2 * cus), rest = t % (2 * cus);
    return kF128 * ((double)full + (rest == 0 ? 0.0 : rest <= cus ? kF128Half : 1.0));
  }
  if (cfg == 4) return kF160 * (double)(((M + 255) / 256 * ((N + 159) / 160) + cus - 1) / cus);
  if (cfg == 5) return kF256x128 * (double)(((M + 255) / 256 * ((N + 127) / 128) + cus - 1) / cus);
  return (double)(((M + 255) / 256 * ((N + 255) / 256) + cus - 1) / cus);
}

GemmPlan gemm_plan(int M, int N) {
  static const int cfg = [] {
    const char* s = getenv("I8MM_GEMM_CFG");
    return s ? atoi(s) : 0;
  }();
  static const bool split_ok = [] {
    const char* s = getenv("I8MM_GEMM_SPLIT");
    return !(s && atoi(s) == 0);
  }();
  static const bool t128_ok = [] {
    const char* s = getenv("I8MM_GEMM_T128");
    return !(s && atoi(s) == 0);
  }();
  if (cfg == 1 || cfg == 3 || cfg == 4 || cfg == 5) return GemmPlan{cfg, N, 0};
  const long cus = device_cu_count();
  // the cheapest single launch (ties keep the earlier configuration)
  const int order[3] = {3, 4, 5};
  GemmPlan best{1, N, 0};
  double cbest = launch_cost(1, M, N, cus);
  for (int c : order) {
    if (c == 5 && !t128_ok) continue;
    const double v = launch_cost(c, M, N, cus);
    if (v < cbest) {
      best = GemmPlan{c, N, 0};
      cbest = v;
    }
  }
  if (!split_ok) return best;
  // whole rounds of 256x256 tiles over the leading columns, the cheapest
  // smaller tiles over the rest
  const long tm = (M + 255) / 256;
  const long t256 = tm * ((N + 255) / 256);
  for (long R = 1; R * cus < t256; ++R) {
    const long n1 = (R * cus / tm) * 256;
    if (n1 <= 0 || n1 >= N) continue;
    int rc = 3;
    double rest = launch_cost(3, M, N - n1, cus);
    for (int c : {4, 5}) {
      if (c == 5 && !t128_ok) continue;
      const double v = launch_cost(c, M, N - n1, cus);
      if (v < rest) {
        rest = v;
        rc = c;
      }
    }
    const double c = launch_cost(1, M, n1, cus) + kGap + rest;
    if (c < cbest - kMargin) {
      best = GemmPlan{1, (int)n1, rc};
      cbest = c;
    }
  }
  return best;
}

template <int CFG>
static hipError_t run_cfg(const int8_t* Xi8, const int8_t* Wi8, int M, int N, int nbase, int nend,
                          int KB, const Epilogue* epi, int32_t* acc, int groupM, hipStream_t st,
                          const KernelEvents* ev, bool start_ev, bool stop_ev) {
  if constexpr (CFG == 3)
    return run_gemm<128, 128, 2, 2, 4>(Xi8, Wi8, M, N, nbase, nend, KB, epi, acc, groupM, st, ev,
                                       start_ev, stop_ev);
  else if constexpr (CFG == 4)
    return run_gemm<256, 160, 4, 2, 4>(Xi8, Wi8, M, N, nbase, nend, KB, epi, acc, groupM, st, ev,
                                       start_ev, stop_ev);
  else if constexpr (CFG == 5)
    return run_gemm<256, 128, 4, 2, 4>(Xi8, Wi8, M, N, nbase, nend, KB, epi, acc, groupM, st, ev,
                                       start_ev, stop_ev);
  else
    return run_gemm<256, 256, 4, 2, 4>(Xi8, Wi8, M, N, nbase, nend, KB, epi, acc, groupM, st, ev,
                                       start_ev, stop_ev);
}

static hipError_t run_any(int cfg, const int8_t* Xi8, const int8_t* Wi8, int M, int N, int nbase,
                          int nend, int KB, const Epilogue* epi, int32_t* acc, int groupM,
                          hipStream_t st, const KernelEvents* ev, bool start_ev, bool stop_ev) {
  switch (cfg) {
    case 3:
      return run_cfg<3>(Xi8, Wi8, M, N, nbase, nend, KB, epi, acc, groupM, st, ev, start_ev,
                        stop_ev);
    case 4:
      return run_cfg<4>(Xi8, Wi8, M, N, nbase, nend, KB, epi, acc, groupM, st, ev, start_ev,
                        stop_ev);
    case 5:
      return run_cfg<5>(Xi8, Wi8, M, N, nbase, nend, KB, epi, acc, groupM, st, ev, start_ev,
                        stop_ev);
    default:
      return run_cfg<1>(Xi8, Wi8, M, N, nbase, nend, KB, epi, acc, groupM, st, ev, start_ev,
                        stop_ev);
  }
}

hipError_t launch_gemm(const int8_t* Xi8, const int8_t* Wi8, int M, int N, int K,
                       const Epilogue* epi, int32_t* acc, hipStream_t st, const KernelEvents* ev) {
  static const int groupM = [] {
    const char* s = getenv("I8MM_GEMM_GROUPM");
    return s ? atoi(s) : 0;
  }();
  const int KB = (int)(pack_kpad(K) / 64);
  const GemmPlan p = gemm_plan(M, N);
  if (p.n1 >= N)
    return run_any(p.first, Xi8, Wi8, M, N, 0, N, KB, epi, acc, groupM, st, ev, true, true);
  // column split (n1 is a multiple of 256): the events span both launches
  hipError_t e =
      run_any(p.first, Xi8, Wi8, M, N, 0, p.n1, KB, epi, acc, groupM, st, ev, true, false);
  if (e != hipSuccess) return e;
  return run_any(p.second, Xi8, Wi8, M, N, p.n1, N, KB, epi, acc, groupM, st, ev, false, true);
}

}  // namespace i8mm
