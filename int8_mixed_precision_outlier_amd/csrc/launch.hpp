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

// M at or below this takes the bandwidth-bound decode kernel.
constexpr int kDecodeMaxM = 32;

hipError_t launch_quantize_weight(const uint16_t* W, int K, int N, int8_t* Wq, float* aw,
                                  hipStream_t st);
hipError_t launch_pack_rows(const int8_t* src, int R, int K, int8_t* dst, hipStream_t st);
// With more than this many rows and at least this many elements (the 175B
// FFN prefill has 50M; below ~30M the extra launch costs more than the
// coalesced pass saves) the column absmax runs in two passes through
// `scratch` (ceil(M/32) x K fp16, at most M*K/16 + 2K bytes; null: one pass).
constexpr int kDetectTwoPassM = 512;
constexpr int64_t kDetectTwoPassElems = 32ll << 20;
hipError_t launch_detect(const uint16_t* X, int M, int K, float alpha, float* colmax,
                         uint32_t* mask, uint16_t* scratch, hipStream_t st);
// Ascending outlier list idx[0 .. min(n, n_cap)) and header {overflow flag,
// min(n, n_cap), n, 0} from the mask of K columns (one workgroup).
hipError_t launch_mask_index(const uint32_t* mask, int K, int n_cap, int32_t* idx, int32_t* hdr,
                             hipStream_t st);
// Where the fp16 rows of the outlier dims come from: the whole fp16 W
// [K][N], or (W null) an outlier-row cache: slot[k] = row of dim k in
// rows [n_dims][N] or -1, with the int8 weights (packed, W_i8) and their
// column absmax as the stand-in for dims outside the cache.
struct OutlierSource {
  const uint16_t* W;
  const int32_t* slot;
  const uint16_t* rows;
  const int8_t* Wi8;
  const float* wabs;
};

// One-row X (M == 1): the quantizer derives the outlier mask from the row
// itself (its column absmax is |x|) and writes the detector's fields, so no
// detection launch precedes it.
struct OneRowDetect {
  float alpha;
  float* colmax;  // the detector's column absmax field
};
hipError_t launch_quant_act(const uint16_t* X, int M, int K, uint32_t* mask, int n_cap,
                            int8_t* Xi8, float* xabs, uint16_t* Xout, int32_t* hdr, int32_t* idx,
                            const OutlierSource& src, int N, uint16_t* WoutT, int KBo,
                            const OneRowDetect* one_row, hipStream_t st);
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

hipError_t launch_gemm(const int8_t* Xi8, const int8_t* Wi8, int M, int N, int K,
                       const Epilogue* epi, int32_t* acc, hipStream_t st,
                       const KernelEvents* ev = nullptr);
hipError_t launch_decode(const int8_t* Xi8, const int8_t* Wi8, int M, int N, int K,
                         const Epilogue* epi, int32_t* acc, hipStream_t st,
                         const KernelEvents* ev = nullptr);

}  // namespace i8mm
