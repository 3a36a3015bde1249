// Internal launchers (host side) of the gfx950 kernels.  Each enqueues its
// kernels on `st` and returns hipGetLastError(); argument checking is done by
// the C-ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#define INT8MM_MAX_K_WORDS 2048  // 65536 columns / 32 bits

namespace i8mm {

// Compute units of the current device (queried once per device; 256 if the
// query fails).
int device_cu_count();

// M at or below this takes the bandwidth-bound decode kernel after the
// decode prologue (the few-row detector with per-strip row maxima, the
// strip quantizer).
constexpr int kDecodeMaxM = 32;
// Up to this M the decode kernel can also run, with 3 or 4 token blocks of
// 16, after the general detector and quantizer (decode_max_m(): this, or
// I8MM_DECODE_MAXM for tuning sweeps, at least kDecodeMaxM).
constexpr int kDecodeWideMaxM = 64;
int decode_max_m();
// Whether an M x N call takes the decode kernel (else the tiled GEMM).
bool use_decode(int M, int N);

hipError_t launch_quantize_weight(const uint16_t* W, int K, int N, int8_t* Wq, float* aw,
                                  hipStream_t st);
hipError_t launch_pack_rows(const int8_t* src, int R, int K, int8_t* dst, hipStream_t st);
// With more than this many rows and at least this many elements (the 175B
// FFN prefill has 50M; below ~30M the extra launch costs more than the
// coalesced pass saves) the column absmax runs in two passes through
// `scratch` (ceil(M/32) x K fp16, at most M*K/16 + 2K bytes; null: one pass).
constexpr int kDetectTwoPassM = 512;
constexpr int64_t kDetectTwoPassElems = 32ll << 20;
// rowpart (M <= 32 only; null: not written): per-row absmax of each
// 32-column strip over its non-outlier columns, fp16 magnitude bits,
// [M][rowpart_stride(K)].
hipError_t launch_detect(const uint16_t* X, int M, int K, float alpha, float* colmax,
                         uint32_t* mask, uint16_t* scratch, hipStream_t st,
                         uint16_t* rowpart = nullptr);
// Row stride (fp16 entries) of the strip maxima: ceil(K/32) rounded up to
// 8 (16-byte rows), at least 8.
inline int rowpart_stride(int K) {
  const int s = ((K + 31) / 32 + 7) / 8 * 8;
  return s > 8 ? s : 8;
}
// Ascending outlier list idx[0 .. min(n, n_cap)) and header {overflow flag,
// min(n, n_cap), n, 0} from the mask of K columns (one workgroup).
hipError_t launch_mask_index(const uint32_t* mask, int K, int n_cap, int32_t* idx, int32_t* hdr,
                             hipStream_t st);
// Tag in the first word of an outlier-row cache's header {magic, K, N,
// n_dims}.
constexpr int32_t kCacheMagic = 0x3148434f;

// Where the fp16 rows of the outlier dims come from: the whole fp16 W
// [K][N], or (W null) an outlier-row cache: header {magic, K, N, n_dims},
// slot[k] = row of dim k in rows [n_dims][N] or -1, with the int8 weights
// (packed, W_i8) and their column absmax as the stand-in for dims outside
// the cache.  W and cache both null: no outlier rows are gathered (N == 0).
struct OutlierSource {
  const uint16_t* W;
  const int32_t* cache;  // cache header, or null
  const int32_t* slot;
  const uint16_t* rows;
  const int8_t* Wi8;
  const float* wabs;
};

// gather: also gather W_out^T (the prefill path and the stage export); the
// decode kernel gathers its own slices instead.
hipError_t launch_quant_act(const uint16_t* X, int M, int K, uint32_t* mask, int n_cap,
                            int8_t* Xi8, float* xabs, uint16_t* Xout, int32_t* hdr, int32_t* idx,
                            const OutlierSource& src, int N, uint16_t* WoutT, int KBo, bool gather,
                            hipStream_t st);
// The decode calls' row quantizer (M <= 32) after launch_detect with
// rowpart: one wavefront per (row, 1024 columns), no W_out^T gather.
hipError_t launch_quant_strips(const uint16_t* X, int M, int K, const uint32_t* mask,
                               const uint16_t* rowpart, int n_cap, int8_t* Xi8, float* xabs,
                               uint16_t* Xout, int32_t* hdr, int32_t* idx,
                               const OutlierSource& src, int N, int KBo, hipStream_t st);
// The former form: one workgroup per row (kept for comparison).
hipError_t launch_quant_rows(const uint16_t* X, int M, int K, uint32_t* mask, int n_cap,
                             int8_t* Xi8, float* xabs, uint16_t* Xout, int32_t* hdr, int32_t* idx,
                             const OutlierSource& src, int N, int KBo, hipStream_t st);
hipError_t launch_cache_rows(const uint16_t* W, int N, const int32_t* dims, int n_dims,
                             uint16_t* rows, hipStream_t st);

// Epilogue inputs of the fused fp16 output (null for the int32 export).
// X_out and W_out^T are fp16 matrices in the packed layout (pack.hpp) over
// bytes, KBo 64-byte blocks (32 outlier columns each) per row, zero past n
// up to roundup(n, 16).
struct Epilogue {
  const float* xabs;      // [M] row absmax of the int8 activations
  const float* wabs;      // [N] column absmax of the int8 weights
  const uint16_t* Xout;   // packed fp16 [rpad(M)][32*KBo] outlier activations
  const uint16_t* WoutT;  // packed fp16 [N][32*KBo] outlier weights, transposed
  const int32_t* hdr;     // hdr[1] = n (outlier count actually used)
  uint16_t* Y;            // [M][N] fp16 output
  int KBo;                // blocks per packed outlier row: kpad(2*n_cap)/64
  int n_cap;              // capacity of the outlier list (n <= n_cap)
  int K;                  // inner dimension (n == K: no int8 product)
  const uint16_t* bias;   // [N] fp16 layer bias, or null
};

// Optional events that the dispatch of the main kernel itself records at
// its start and end (hipExtLaunchKernel), for per-kernel timing without
// extra stream packets around it.
struct KernelEvents {
  hipEvent_t start, stop;
};

// Kernel choices, shared by the launchers and the configuration query:
// tiled GEMM 1 = 256x256 tiles, 3 = 128x128, 4 = 256x160, 5 = 256x128; decode row blocks per
// workgroup R (1-4, or with `wide` also 5, 6, 8, 9, 12 when that gives
// exactly one workgroup per compute unit) and K-splitting wavefronts (2, 4
// or 8).  The int32 export's K-loop kernel takes R <= 4 only.
// The tiled GEMM's launches for M x N: columns [0, n1) with configuration
// `first`, then (n1 < N) columns [n1, N) with `second`.
struct GemmPlan {
  int first;
  int n1;
  int second;
};
GemmPlan gemm_plan(int M, int N);
void decode_config(int N, int* R, int* ks, bool wide);
// The decode kernel's configuration for an M x N call: decode_config, with
// the wide workgroups for up to 48 tokens (and 5-6 row blocks up to 64) and
// two wavefronts above 32.
void decode_choice(int M, int N, int* R, int* ks);

hipError_t launch_gemm(const int8_t* Xi8, const int8_t* Wi8, int M, int N, int K,
                       const Epilogue* epi, int32_t* acc, hipStream_t st,
                       const KernelEvents* ev = nullptr);
// The decode call's GEMM (M <= 64): it gathers the outlier weight rows of
// its own output features (and writes that slice of W_out^T).  M >= 2 reads
// the detector's and the row quantizer's results from the workspace; M == 1
// derives the mask and quantizes the one row itself (no earlier launch) and
// writes the intermediates those kernels would have.
struct DecodeCall {
  const uint16_t* X;   // [M][K] fp16 activations
  float alpha;
  float* colmax;       // M == 1: written (the detector's field)
  uint32_t* mask_out;  // M == 1: written (the detector's field)
  int8_t* Xi8;
  float* xabs;
  uint16_t* Xout;
  uint16_t* WoutT;
  int32_t* idx;
  int32_t* hdr;
  OutlierSource src;
};
hipError_t launch_decode_mm(const int8_t* Wi8, int M, int N, int K, const Epilogue& epi,
                            const DecodeCall& c, hipStream_t st, const KernelEvents* ev = nullptr);

// The decode kernel's K loop with int32 output (the int8_gemm_i32 export).
hipError_t launch_decode_i32(const int8_t* Xi8, const int8_t* Wi8, int M, int N, int K,
                             int32_t* acc, hipStream_t st);

}  // namespace i8mm
