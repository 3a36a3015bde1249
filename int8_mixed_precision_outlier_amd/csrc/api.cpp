// C-ABI layer of the int8 mixed-precision outlier matmul: argument checks,
// workspace layout and kernel dispatch.  Host code only; it never allocates,
// frees or synchronizes.  The operations are described in include/int8mm.h.
#include "../../include/int8mm.h"
#include "api_internal.hpp"
#include "launch.hpp"
#include "pack.hpp"

#include <math.h>
#include <stdint.h>

#include <vector>

using namespace i8mm;

namespace {

thread_local int g_last_hip_error = 0;

// Event pairs of the profiling aid (int8mm_timing_*).
struct EventPair {
  hipEvent_t start, stop;
};
std::vector<EventPair> g_events;
size_t g_events_used = 0;
bool g_timing = false;

EventPair* timing_slot() {
  if (!g_timing) return nullptr;
  if (g_events_used == g_events.size()) {
    EventPair p{};
    if (hipEventCreate(&p.start) != hipSuccess) return nullptr;
    if (hipEventCreate(&p.stop) != hipSuccess) {
      (void)hipEventDestroy(p.start);  // best effort: the slot is not created
      return nullptr;
    }
    g_events.push_back(p);
  }
  return &g_events[g_events_used++];
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline int64_t up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

int hip_status(hipError_t e) {
  if (e == hipSuccess) return INT8MM_OK;
  g_last_hip_error = (int)e;
  return INT8MM_EHIP;
}

// Shape checks common to the matmul entry points (sizes include the
// padding of the packed int8 layout).
int check_shape(int64_t M, int64_t K, int64_t N) {
  if (M < 0 || K < 0 || N < 0) return INT8MM_EINVAL;
  if (K > INT8MM_MAX_K) return INT8MM_EINVAL;
  if (M > INT8MM_MAX_MN || N > INT8MM_MAX_MN) return INT8MM_EINVAL;
  const int64_t Kp = pack_kpad(K);
  if (pack_rpad(M) * Kp > INT8MM_MAX_MN || N * Kp > INT8MM_MAX_MN || M * K > INT8MM_MAX_MN ||
      M * N > INT8MM_MAX_MN)
    return INT8MM_EINVAL;
  if (K % 16 != 0 || N % 16 != 0) return INT8MM_EALIGN;
  return INT8MM_OK;
}

// The packed fp16 outlier matrices stay within the byte range the kernels
// address with 32-bit buffer offsets.
bool outlier_fits(int64_t M, int64_t N, int64_t n_cap) {
  const int64_t ob = pack_kpad(2 * n_cap);
  return pack_rpad(M) * ob <= INT8MM_MAX_MN && N * ob <= INT8MM_MAX_MN;
}

// Workspace layout; returns the total size.  Every field starts on a
// 256-byte boundary.
size_t layout(int64_t M, int64_t K, int64_t N, int64_t n_cap, int64_t* off) {
  const int64_t ob = pack_kpad(2 * n_cap);  // bytes per packed fp16 outlier row
  const int64_t sizes[INT8MM_WS_NFIELDS] = {
      16,                       // header
      4 * K,                    // colmax
      4 * ((K + 31) / 32),      // mask
      4 * n_cap,                // idx
      4 * M,                    // x_absmax
      pack_rpad(M) * pack_kpad(K),  // X_i8 (packed)
      pack_rpad(M) * ob,        // X_out (packed fp16)
      N * ob,                   // W_out^T (packed fp16)
      // decode calls (2 <= M <= 32): per-row maxima of the 32-column strips
      M > 1 && M <= kDecodeMaxM ? 2 * M * rowpart_stride((int)K) : 0,
  };
  int64_t o = 0;
  for (int i = 0; i < INT8MM_WS_NFIELDS; ++i) {
    if (off) off[i] = o;
    o += up(sizes[i] > 0 ? sizes[i] : 1, 256);
  }
  return (size_t)o;
}

// Typed pointers to the workspace fields.
struct Ws {
  int32_t* hdr;
  float* colmax;
  uint32_t* mask;
  int32_t* idx;
  float* xabs;
  int8_t* Xi8;
  uint16_t* Xout;
  uint16_t* WoutT;
  uint16_t* rowmax;
};

Ws carve(void* workspace, const int64_t* off) {
  char* ws = static_cast<char*>(workspace);
  return Ws{reinterpret_cast<int32_t*>(ws + off[INT8MM_WS_HEADER]),
            reinterpret_cast<float*>(ws + off[INT8MM_WS_COLMAX]),
            reinterpret_cast<uint32_t*>(ws + off[INT8MM_WS_MASK]),
            reinterpret_cast<int32_t*>(ws + off[INT8MM_WS_IDX]),
            reinterpret_cast<float*>(ws + off[INT8MM_WS_XABS]),
            reinterpret_cast<int8_t*>(ws + off[INT8MM_WS_XI8]),
            reinterpret_cast<uint16_t*>(ws + off[INT8MM_WS_XOUT]),
            reinterpret_cast<uint16_t*>(ws + off[INT8MM_WS_WOUT]),
            reinterpret_cast<uint16_t*>(ws + off[INT8MM_WS_ROWMAX])};
}

// Stage 1: column absmax and outlier mask.  The X_i8 field (written only
// after detection) is the scratch of the two-pass column absmax.
hipError_t enqueue_detect(const uint16_t* X, int64_t M, int64_t K, float alpha, const Ws& w,
                          hipStream_t st, uint16_t* rowpart = nullptr) {
  return launch_detect(X, (int)M, (int)K, alpha, w.colmax, w.mask,
                       reinterpret_cast<uint16_t*>(w.Xi8), st, rowpart);
}

// Stage 2: row absmax, int8 quantization, X_out / W_out^T gather; also the
// outlier list and the header.
hipError_t enqueue_quant(const uint16_t* X, int64_t M, int64_t K, const OutlierSource& src,
                         int64_t N, int64_t n_cap, const Ws& w, hipStream_t st,
                         bool gather = true) {
  const int KBo = (int)(pack_kpad(2 * n_cap) / 64);
  return launch_quant_act(X, (int)M, (int)K, w.mask, (int)n_cap, w.Xi8, w.xabs, w.Xout, w.hdr,
                          w.idx, src, (int)N, w.WoutT, KBo, gather, st);
}

}  // namespace

extern "C" {

const char* int8mm_status_string(int status) {
  switch (status) {
    case INT8MM_OK: return "ok";
    case INT8MM_EINVAL: return "invalid argument (null pointer, size out of range, or alpha NaN/negative)";
    case INT8MM_EALIGN: return "alignment (K and N must be multiples of 16, pointers 16-byte aligned)";
    case INT8MM_EWORKSPACE: return "workspace too small";
    case INT8MM_EHIP: return "HIP kernel launch failed";
    case INT8MM_ESCRATCH:
      return "the call needs more scratch than the no-allocation entry point's static array holds";
    default: return "unknown status";
  }
}

int int8mm_last_hip_error(void) { return g_last_hip_error; }

int64_t int8_packed_size(int64_t rows, int64_t K) {
  if (rows < 0 || K < 0 || K > INT8MM_MAX_K) return -1;
  return pack_rpad(rows) * pack_kpad(K);
}

int int8_pack_rows(const int8_t* src, int64_t R, int64_t K, int8_t* dst, hipStream_t stream) {
  if (R < 0 || K < 0 || K > INT8MM_MAX_K || pack_rpad(R) * pack_kpad(K) > INT8MM_MAX_MN)
    return INT8MM_EINVAL;
  if (K % 16 != 0) return INT8MM_EALIGN;
  if (R == 0 || K == 0) return INT8MM_OK;
  if (!src || !dst) return INT8MM_EINVAL;
  if (!aligned16(src) || !aligned16(dst)) return INT8MM_EALIGN;
  return hip_status(launch_pack_rows(src, (int)R, (int)K, dst, stream));
}

int int8_quantize_weight(const void* W_f16, int64_t K, int64_t N, int8_t* W_i8, float* w_absmax,
                         hipStream_t stream) {
  if (K < 0 || N < 0 || K > INT8MM_MAX_K || N > INT8MM_MAX_MN || pack_kpad(K) * N > INT8MM_MAX_MN)
    return INT8MM_EINVAL;
  if (K % 16 != 0 || N % 16 != 0) return INT8MM_EALIGN;
  if (N == 0) return INT8MM_OK;
  if (!w_absmax) return INT8MM_EINVAL;
  if (K > 0 && (!W_f16 || !W_i8)) return INT8MM_EINVAL;
  if (!aligned16(w_absmax) || (K > 0 && (!aligned16(W_f16) || !aligned16(W_i8))))
    return INT8MM_EALIGN;
  return hip_status(launch_quantize_weight(static_cast<const uint16_t*>(W_f16), (int)K, (int)N,
                                           W_i8, w_absmax, stream));
}

size_t int8_mixed_matmul_workspace_size(int64_t M, int64_t K, int64_t N, int64_t n_cap,
                                        int64_t* offsets) {
  if (check_shape(M, K, N) != INT8MM_OK) return 0;
  if (n_cap < 0 || n_cap > K || !outlier_fits(M, N, n_cap)) return 0;
  return layout(M, K, N, n_cap, offsets);
}

}  // extern "C"

namespace {

// Outlier-row cache layout (bytes from the cache base, 256-byte aligned):
// header int32[4] = {magic, K, N, n_dims}; slot int32[K] (row of dim k in
// rows, or -1); rows fp16 [n_dims][N]; dims int32[n_dims].  slot and rows
// sit at offsets that depend on K only.
struct CacheLayout {
  int64_t slot, rows, dims, total;
};
CacheLayout cache_layout(int64_t K, int64_t N, int64_t n_dims) {
  CacheLayout c;
  c.slot = 256;
  c.rows = c.slot + up(4 * (K > 0 ? K : 1), 256);
  c.dims = c.rows + up(2 * (n_dims * N > 0 ? n_dims * N : 1), 256);
  c.total = c.dims + up(4 * (n_dims > 0 ? n_dims : 1), 256);
  return c;
}

}  // namespace

namespace i8mm {

int hip_error_status(hipError_t e) { return hip_status(e); }

// Shared body of the matmul entry points; exactly one of W_f16 and cache
// is non-null.
int run_mixed(const void* X_f16, int64_t M, int64_t K, const int8_t* W_i8,
              const float* w_absmax, const void* W_f16, const void* cache, int64_t N,
              float alpha, const void* bias_f16, void* Y_f16, void* workspace,
              size_t workspace_bytes, int64_t n_cap, hipStream_t stream) {
  int st = check_shape(M, K, N);
  if (st != INT8MM_OK) return st;
  if (isnan(alpha) || alpha < 0.0f) return INT8MM_EINVAL;
  if (n_cap < 0 || n_cap > K || !outlier_fits(M, N, n_cap)) return INT8MM_EINVAL;
  if (M == 0 || N == 0) return INT8MM_OK;
  if (!X_f16 && K > 0) return INT8MM_EINVAL;
  if (!W_i8 && K > 0) return INT8MM_EINVAL;
  if (!w_absmax || (!W_f16 && !cache && K > 0) || !Y_f16 || !workspace) return INT8MM_EINVAL;
  if ((K > 0 && (!aligned16(X_f16) || !aligned16(W_i8) || (W_f16 && !aligned16(W_f16)))) ||
      !aligned16(w_absmax) || !aligned16(Y_f16) || (bias_f16 && !aligned16(bias_f16)) ||
      (cache && (reinterpret_cast<uintptr_t>(cache) & 255u) != 0) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return INT8MM_EALIGN;
  int64_t off[INT8MM_WS_NFIELDS];
  const size_t need = layout(M, K, N, n_cap, off);
  if (workspace_bytes < need) return INT8MM_EWORKSPACE;

  const Ws w = carve(workspace, off);
  const uint16_t* X = static_cast<const uint16_t*>(X_f16);

  OutlierSource src{static_cast<const uint16_t*>(W_f16), nullptr, nullptr, nullptr, W_i8,
                    w_absmax};
  if (!W_f16) {
    const CacheLayout c = cache_layout(K, N, 0);
    const char* cb = static_cast<const char*>(cache);
    src.cache = reinterpret_cast<const int32_t*>(cb);
    src.slot = reinterpret_cast<const int32_t*>(cb + c.slot);
    src.rows = reinterpret_cast<const uint16_t*>(cb + c.rows);
  }

  const int KBo = (int)(pack_kpad(2 * n_cap) / 64);
  Epilogue epi{w.xabs, w_absmax, w.Xout, w.WoutT, w.hdr, static_cast<uint16_t*>(Y_f16), KBo,
               (int)n_cap, (int)K, static_cast<const uint16_t*>(bias_f16)};
  EventPair* ev = timing_slot();
  const KernelEvents kev{ev ? ev->start : nullptr, ev ? ev->stop : nullptr};
  hipError_t e = hipSuccess;
  if (M <= kDecodeMaxM) {
    // decode: the weight-streaming kernel gathers the outlier rows of its own
    // output features; one row needs no detector or quantizer launch (the
    // kernel quantizes the row itself)
    if (M > 1 && K > 0) {
      // the detector also leaves each row's strip maxima, so the quantizer
      // spreads every row over many wavefronts
      e = enqueue_detect(X, M, K, alpha, w, stream, w.rowmax);
      if (e == hipSuccess)
        e = launch_quant_strips(X, (int)M, (int)K, w.mask, w.rowmax, (int)n_cap, w.Xi8, w.xabs,
                                w.Xout, w.hdr, w.idx, src, (int)N, KBo, stream);
      if (e != hipSuccess) return hip_status(e);
    } else if (M > 1) {
      e = launch_quant_rows(X, (int)M, (int)K, w.mask, (int)n_cap, w.Xi8, w.xabs, w.Xout, w.hdr,
                            w.idx, src, (int)N, KBo, stream);
      if (e != hipSuccess) return hip_status(e);
    }
    const DecodeCall c{X, alpha, w.colmax, w.mask, w.Xi8, w.xabs, w.Xout, w.WoutT, w.idx, w.hdr,
                       src};
    e = launch_decode_mm(W_i8, (int)M, (int)N, (int)K, epi, c, stream, ev ? &kev : nullptr);
    return hip_status(e);
  }
  if (use_decode((int)M, (int)N)) {
    // 33-64 tokens: still bound by the weight stream, so the decode kernel
    // with 3 or 4 token blocks, after the general detector and quantizer
    // (no W_out^T gather: the decode kernel gathers its own features')
    e = enqueue_detect(X, M, K, alpha, w, stream);
    if (e == hipSuccess) e = enqueue_quant(X, M, K, src, N, n_cap, w, stream, false);
    if (e != hipSuccess) return hip_status(e);
    const DecodeCall c{X, alpha, w.colmax, w.mask, w.Xi8, w.xabs, w.Xout, w.WoutT, w.idx, w.hdr,
                       src};
    e = launch_decode_mm(W_i8, (int)M, (int)N, (int)K, epi, c, stream, ev ? &kev : nullptr);
    return hip_status(e);
  }
  e = enqueue_detect(X, M, K, alpha, w, stream);
  if (e != hipSuccess) return hip_status(e);
  e = enqueue_quant(X, M, K, src, N, n_cap, w, stream);
  if (e != hipSuccess) return hip_status(e);
  e = launch_gemm(w.Xi8, W_i8, (int)M, (int)N, (int)K, &epi, nullptr, stream, ev ? &kev : nullptr);
  return hip_status(e);
}

}  // namespace i8mm

extern "C" {

int int8_mixed_matmul(const void* X_f16, int64_t M, int64_t K, const int8_t* W_i8,
                      const float* w_absmax, const void* W_f16, int64_t N, float alpha,
                      const void* bias_f16, void* Y_f16, void* workspace,
                      size_t workspace_bytes, int64_t n_cap, hipStream_t stream) {
  if (!W_f16 && K > 0 && M > 0 && N > 0) return INT8MM_EINVAL;
  return run_mixed(X_f16, M, K, W_i8, w_absmax, W_f16, nullptr, N, alpha, bias_f16, Y_f16,
                   workspace, workspace_bytes, n_cap, stream);
}

int int8_detect_outliers(const void* X_f16, int64_t M, int64_t K, float alpha, int64_t n_cap,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_shape(M, K, 0);
  if (st != INT8MM_OK) return st;
  if (isnan(alpha) || alpha < 0.0f) return INT8MM_EINVAL;
  if (n_cap < 0 || n_cap > K || !outlier_fits(M, 0, n_cap)) return INT8MM_EINVAL;
  if (M == 0) return INT8MM_OK;
  if ((!X_f16 && K > 0) || !workspace) return INT8MM_EINVAL;
  if ((K > 0 && !aligned16(X_f16)) || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return INT8MM_EALIGN;
  int64_t off[INT8MM_WS_NFIELDS];
  layout(M, K, 0, n_cap, off);
  if (workspace_bytes < (size_t)off[INT8MM_WS_XOUT]) return INT8MM_EWORKSPACE;
  const Ws w = carve(workspace, off);
  hipError_t e = enqueue_detect(static_cast<const uint16_t*>(X_f16), M, K, alpha, w, stream);
  if (e == hipSuccess) e = launch_mask_index(w.mask, (int)K, (int)n_cap, w.idx, w.hdr, stream);
  return hip_status(e);
}

int int8_quantize_activations(const void* X_f16, int64_t M, int64_t K, const void* W_f16,
                              int64_t N, int64_t n_cap, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
  int st = check_shape(M, K, N);
  if (st != INT8MM_OK) return st;
  if (n_cap < 0 || n_cap > K || !outlier_fits(M, N, n_cap)) return INT8MM_EINVAL;
  if (M == 0) return INT8MM_OK;
  if ((K > 0 && (!X_f16 || (N > 0 && !W_f16))) || !workspace) return INT8MM_EINVAL;
  if ((K > 0 && (!aligned16(X_f16) || (W_f16 && !aligned16(W_f16)))) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return INT8MM_EALIGN;
  int64_t off[INT8MM_WS_NFIELDS];
  if (workspace_bytes < layout(M, K, N, n_cap, off)) return INT8MM_EWORKSPACE;
  const Ws w = carve(workspace, off);
  const OutlierSource src{static_cast<const uint16_t*>(W_f16), nullptr, nullptr, nullptr, nullptr,
                          nullptr};
  return hip_status(enqueue_quant(static_cast<const uint16_t*>(X_f16), M, K, src, N, n_cap, w,
                                  stream));
}

int64_t int8_outlier_cache_size(int64_t K, int64_t N, int64_t n_dims) {
  if (K < 0 || N < 0 || K > INT8MM_MAX_K || N > INT8MM_MAX_MN || n_dims < 0 || n_dims > K ||
      n_dims * N > INT8MM_MAX_MN)
    return -1;
  return cache_layout(K, N, n_dims).total;
}

int int8_build_outlier_cache(const void* W_f16, int64_t K, int64_t N, const int32_t* dims,
                             int64_t n_dims, void* cache, size_t cache_bytes,
                             hipStream_t stream) {
  const int64_t need = int8_outlier_cache_size(K, N, n_dims);
  if (need < 0) return INT8MM_EINVAL;
  if (K % 16 != 0 || N % 16 != 0) return INT8MM_EALIGN;
  if (!cache || (n_dims > 0 && (!dims || !W_f16))) return INT8MM_EINVAL;
  if ((reinterpret_cast<uintptr_t>(cache) & 255u) != 0 || (W_f16 && !aligned16(W_f16)))
    return INT8MM_EALIGN;
  if (cache_bytes < (size_t)need) return INT8MM_EWORKSPACE;
  for (int64_t s = 0; s < n_dims; ++s)
    if (dims[s] < 0 || dims[s] >= K || (s > 0 && dims[s] <= dims[s - 1])) return INT8MM_EINVAL;
  const CacheLayout c = cache_layout(K, N, n_dims);
  // header + slot map, and the dims, assembled on the host
  std::vector<int32_t> head((size_t)(c.rows / 4), 0);
  head[0] = kCacheMagic;
  head[1] = (int32_t)K;
  head[2] = (int32_t)N;
  head[3] = (int32_t)n_dims;
  for (int64_t k = 0; k < K; ++k) head[(size_t)(c.slot / 4 + k)] = -1;
  for (int64_t s = 0; s < n_dims; ++s) head[(size_t)(c.slot / 4 + dims[s])] = (int32_t)s;
  char* cb = static_cast<char*>(cache);
  hipError_t e = hipMemcpyAsync(cb, head.data(), (size_t)c.rows, hipMemcpyHostToDevice, stream);
  if (e == hipSuccess && n_dims > 0)
    e = hipMemcpyAsync(cb + c.dims, dims, (size_t)(4 * n_dims), hipMemcpyHostToDevice, stream);
  if (e == hipSuccess)
    e = launch_cache_rows(static_cast<const uint16_t*>(W_f16), (int)N,
                          reinterpret_cast<const int32_t*>(cb + c.dims), (int)n_dims,
                          reinterpret_cast<uint16_t*>(cb + c.rows), stream);
  // the host buffers must outlive the copies
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  return hip_status(e);
}

int int8_mixed_matmul_cached(const void* X_f16, int64_t M, int64_t K, const int8_t* W_i8,
                             const float* w_absmax, const void* cache, int64_t N, float alpha,
                             const void* bias_f16, void* Y_f16, void* workspace,
                             size_t workspace_bytes, int64_t n_cap, hipStream_t stream) {
  if (!cache && K > 0 && M > 0 && N > 0) return INT8MM_EINVAL;
  return run_mixed(X_f16, M, K, W_i8, w_absmax, nullptr, cache, N, alpha, bias_f16, Y_f16,
                   workspace, workspace_bytes, n_cap, stream);
}

int int8mm_timing_enable(int on) {
  g_timing = on != 0;
  g_events_used = 0;
  return INT8MM_OK;
}

int int8mm_timing_read(double* total_ms, int64_t* launches) {
  double sum = 0.0;
  for (size_t i = 0; i < g_events_used; ++i) {
    hipError_t e = hipEventSynchronize(g_events[i].stop);
    if (e != hipSuccess) return hip_status(e);
    float ms = 0.0f;
    e = hipEventElapsedTime(&ms, g_events[i].start, g_events[i].stop);
    if (e != hipSuccess) return hip_status(e);
    sum += ms;
  }
  if (total_ms) *total_ms = sum;
  if (launches) *launches = (int64_t)g_events_used;
  g_events_used = 0;
  return INT8MM_OK;
}

int int8mm_kernel_config(int64_t M, int64_t N, int64_t K, int32_t* cfg) {
  if (!cfg) return INT8MM_EINVAL;
  const int st = check_shape(M, K, N);
  if (st != INT8MM_OK) return st;
  if (use_decode((int)M, (int)N)) {
    int R = 1, ks = 2;
    if (N > 0) decode_choice((int)M, (int)N, &R, &ks);
    cfg[0] = 0;
    cfg[1] = R;
    cfg[2] = ks;
    cfg[3] = M > 16 ? (int)((M + 15) / 16) : 1;
  } else {
    const GemmPlan p = gemm_plan((int)M, (int)N);
    const int g = p.n1 < N ? p.second : p.first;
    cfg[0] = p.n1 < N ? 2 : 1;
    cfg[1] = p.n1 < N ? p.n1 : g == 3 ? 128 : 256;
    cfg[2] = g == 3 || g == 5 ? 128 : g == 4 ? 160 : 256;
    cfg[3] = g == 3 ? 4 : 8;
  }
  return INT8MM_OK;
}

int int8_gemm_i32(const int8_t* X_i8, int64_t M, int64_t K, const int8_t* W_i8, int64_t N,
                  int32_t* acc, hipStream_t stream) {
  int st = check_shape(M, K, N);
  if (st != INT8MM_OK) return st;
  if (M == 0 || N == 0) return INT8MM_OK;
  if (!acc || (K > 0 && (!X_i8 || !W_i8))) return INT8MM_EINVAL;
  if (!aligned16(acc) || (K > 0 && (!aligned16(X_i8) || !aligned16(W_i8)))) return INT8MM_EALIGN;
  hipError_t e = use_decode((int)M, (int)N)
                     ? launch_decode_i32(X_i8, W_i8, (int)M, (int)N, (int)K, acc, stream)
                     : launch_gemm(X_i8, W_i8, (int)M, (int)N, (int)K, nullptr, acc, stream);
  return hip_status(e);
}

}  // extern "C"
