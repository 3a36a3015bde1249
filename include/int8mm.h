/*
 * int8mm.h -- C-ABI of the LLM.int8() mixed-precision decomposed matmul for
 * AMD Instinct MI355X (gfx950).
 *
 *     Y[M,N] = X[M,K] . W[K,N]   computed as
 *     Y = Out_i32 / (c_x (x) c_w) + X_out . W_out
 *
 * Pages the operations follow (cited by title and section):
 *   [JS]  "LLM.int8() — 大模型激活值里藏着几个超大异常通道" (Jason's Study):
 *         方法 1 (vector-wise quantization), 方法 2 (mixed-precision
 *         decomposition with threshold alpha = 6.0), 观察 2 (the outlier
 *         dims are fixed, so they can be identified statically).
 *   [ALI] developer.aliyun.com article 1691675 "LLM.int8()": §2.2 and 图2
 *         (the pipeline: decompose, vector-wise int8 matmul -> Out_i32,
 *         dequantize by the outer product of C_x and C_w, add the fp16
 *         outlier product, fp16 output).
 *   [GB]  brain.gartu.xyz "LLM.int8()": "Seuil de détection α"
 *         (max(|X[:,j]|) > α), "Vector-wise INT8 Quantization",
 *         "Exemple pratique" (the int8 layer replaces a linear layer with
 *         bias and threshold 6.0).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller (the
 *     dims list of int8_build_outlier_cache is a host array).  The library
 *     never allocates or frees; every kernel is enqueued on `stream` (0 =
 *     the null stream) and the call returns as soon as the launches are
 *     queued.  Only the load-time int8_build_outlier_cache synchronizes.
 *   - Matrices are row-major.  fp16 data is IEEE binary16 passed as void*.
 *   - Constants are stored as absmax values (fp32 copies of fp16 magnitudes);
 *     the pages' constants are c = 127 / absmax.  An all-zero vector has
 *     absmax 0 and quantizes to 0.
 *   - Rounding: s = RN_fp32(127 / absmax), q = round-half-even(RN_fp32(x*s)),
 *     range [-127, 127].  The int8 tensors, absmax vectors, outlier list and
 *     int32 accumulators are therefore unique and reproducible bit for bit.
 *   - Errors are returned as int8mm_status before anything is launched
 *     (argument checks) or right after a failed launch (INT8MM_EHIP).  No
 *     exception crosses the ABI.  Inputs must be finite.
 *   - Calls on one stream are ordered; calls that share a workspace must not
 *     overlap (different streams need different workspaces).
 */
#ifndef INT8MM_H
#define INT8MM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  INT8MM_OK = 0,
  INT8MM_EINVAL = 1,     /* null pointer, size out of range, alpha NaN or < 0 */
  INT8MM_EALIGN = 2,     /* K or N not a multiple of 16, pointer misaligned   */
  INT8MM_EWORKSPACE = 3, /* workspace smaller than the size query returns     */
  INT8MM_EHIP = 4,       /* a kernel launch failed (see int8mm_last_hip_error) */
  INT8MM_ESCRATCH = 5    /* int8_mixed_matmul_noalloc: the shape needs more than
                            INT8MM_NOALLOC_SCRATCH_BYTES of workspace */
} int8mm_status;

/* Size limits checked by every entry point. */
#define INT8MM_MAX_K 65536      /* int32 accumulators stay exact up to K=133144 */
#define INT8MM_MAX_MN (1LL << 31)

/* Human-readable name of a status code (static string, never NULL). */
const char *int8mm_status_string(int status);

/* The hipError_t of the last failed launch in this thread (0 if none). */
int int8mm_last_hip_error(void);

/*
 * int8_quantize_weight -- vector-wise int8 weights, done once offline.
 * [JS 方法 1]: one constant per column of the weight, c_w[j]; [GB
 * "Vector-wise INT8 Quantization"]: scale by the column absmax.
 *
 *   W_f16    in   [K][N] fp16, row-major (K input features, N outputs).
 *   W_i8     out  the N x K int8 matrix W_i8[j][k] =
 *                 round-half-even(RN(W[k][j] * RN(127 / w_absmax[j]))) in the
 *                 PACKED layout below: int8_packed_size(N, K) bytes.
 *   w_absmax out  [N] fp32, max_k |W[k][j]| over all K rows.
 *   Requirements: 0 <= K <= INT8MM_MAX_K, N >= 0, K % 16 == 0, N % 16 == 0,
 *   N * roundup(K, 64) <= INT8MM_MAX_MN, pointers 16-byte aligned (they may
 *   be NULL only if the matrix they describe is empty).  K == 0 gives
 *   w_absmax = 0.
 */
int int8_quantize_weight(const void *W_f16, int64_t K, int64_t N,
                         int8_t *W_i8, float *w_absmax, hipStream_t stream);

/*
 * Packed int8 layout (W_i8, the workspace's X_i8, int8_gemm_i32's inputs).
 * An R x K int8 matrix (row r, column k; both GEMM operands are indexed
 * along K) is stored in 1 KB blocks of 16 rows x 64 k, rows padded to a
 * multiple of 16 and K to a multiple of 64 (padding holds zeros when written
 * by this library):
 *     byte offset of (r, k) = ((r/16) * KB + k/64) * 1024
 *                             + (((k/16) % 4) * 16 + r % 16) * 16 + k % 16,
 *     KB = roundup(K, 64) / 64.
 * A block is one 64-lane x 16-byte load, so the GEMM moves it to LDS with
 * one contiguous DMA and the decode kernel streams whole cache lines.
 */
/* Bytes of an R x K matrix in the packed layout (-1 if out of range). */
int64_t int8_packed_size(int64_t rows, int64_t K);

/* Pack a row-major int8 matrix src [R][K] into dst (int8_packed_size(R, K)
 * bytes, zero-filling the padding).  K % 16 == 0; 16-byte aligned pointers. */
int int8_pack_rows(const int8_t *src, int64_t R, int64_t K, int8_t *dst,
                   hipStream_t stream);

/*
 * Workspace of int8_mixed_matmul.  The layout is public so tests can read
 * the intermediates of a production call.  Offsets are in bytes from the
 * workspace base and 256-byte aligned.
 *   INT8MM_WS_HEADER  int32[4]: [0] status flags (bit 0: the call found more
 *                     outlier columns than n_cap; the columns past n_cap
 *                     were dropped and every element of Y is then a quiet
 *                     NaN; bit 1: int8_mixed_matmul_cached met outlier dims
 *                     outside its cache; bit 2: the cache passed to
 *                     int8_mixed_matmul_cached was not built for this K and
 *                     N, so no cached row was used (bit 1 is then set too if
 *                     there were outliers)),
 *                     [1] n = number of outlier columns used (<= n_cap),
 *                     [2] number of outlier columns found (may exceed n_cap).
 *   INT8MM_WS_COLMAX  float[K]   max_i |X[i,k]|.
 *   INT8MM_WS_MASK    uint32[ceil(K/32)] bit k%32 of word k/32 set iff column
 *                     k is an outlier.
 *   INT8MM_WS_IDX     int32[n_cap] ascending outlier columns (first n valid).
 *   INT8MM_WS_XABS    float[M]   row absmax over the non-outlier columns.
 *   INT8MM_WS_XI8     int8 M x K quantized activations (0 at outlier cols), in
 *                     the packed layout (int8_packed_size(M, K) bytes).  For
 *                     large X (M > 512, M*K >= 2^25) it first serves as the
 *                     detector's scratch.
 *   INT8MM_WS_XOUT    X_out = X[:, idx] as fp16, in the packed layout over
 *                     bytes: row i is a packed row of 2*n_cap bytes, value t
 *                     at bytes 2t, 2t+1 (int8_packed_size(M, 2*n_cap) bytes).
 *                     Values n .. roundup(n, 16)-1 are zero.
 *   INT8MM_WS_WOUT    W_out transposed, W_outT[j][t] = W[idx[t]][j], packed
 *                     the same way with N rows (int8_packed_size(N, 2*n_cap)
 *                     bytes; values n .. roundup(n, 16)-1 zero).
 *   INT8MM_WS_ROWMAX  2 <= M <= 32 (decode calls), K > 0: uint16[M][S],
 *                     S = ceil(K/32) rounded up to a multiple of 8: the
 *                     fp16 magnitude bits of each row's absmax over the
 *                     non-outlier columns of each 32-column strip (the
 *                     detector's by-product; x_absmax is their max).
 *                     Otherwise unused (256 bytes).
 */
enum {
  INT8MM_WS_HEADER = 0,
  INT8MM_WS_COLMAX = 1,
  INT8MM_WS_MASK = 2,
  INT8MM_WS_IDX = 3,
  INT8MM_WS_XABS = 4,
  INT8MM_WS_XI8 = 5,
  INT8MM_WS_XOUT = 6,
  INT8MM_WS_WOUT = 7,
  INT8MM_WS_ROWMAX = 8,
  INT8MM_WS_NFIELDS = 9
};

/* Total workspace bytes for a call of this shape; 0 if the shape is invalid.
 * If `offsets` is not NULL it receives INT8MM_WS_NFIELDS byte offsets. */
size_t int8_mixed_matmul_workspace_size(int64_t M, int64_t K, int64_t N,
                                        int64_t n_cap, int64_t *offsets);

/*
 * int8_mixed_matmul -- the decomposed matmul, one call per activation batch.
 * [JS 方法 2] / [GB "Seuil de détection α"]: column k of X is an outlier iff
 * max_i |X[i,k]| > alpha (strict, compared in fp32); [ALI 图2]: outlier
 * columns and the matching rows of W are multiplied in fp16 (fp32
 * accumulation), every other column is quantized per row (c_x[i] = 127 /
 * absmax of row i over its non-outlier columns) and multiplied in int8 with
 * int32 accumulation; the result Out_i32 * (x_absmax[i]/127) *
 * (w_absmax[j]/127) + X_out . W_out is rounded once to fp16.
 *
 *   X_f16     in  [M][K] fp16 activations.
 *   W_i8      in  packed N x K int8 and w_absmax [N] fp32 from
 *                 int8_quantize_weight.
 *   W_f16     in  [K][N] fp16 weights; only the outlier rows are read.
 *   alpha     in  outlier threshold (6.0 in the pages); +inf disables the fp16
 *                 path, 0 sends every nonzero column to it.  NaN or < 0 is
 *                 INT8MM_EINVAL.
 *   bias_f16  in  [N] fp16 layer bias or NULL ([GB "Exemple pratique"]: the
 *                 int8 layer replaces a linear layer with bias); added to
 *                 every output row in fp32 before the fp16 rounding.
 *   Y_f16     out [M][N] fp16.
 *   workspace     device buffer of >= int8_mixed_matmul_workspace_size(M, K,
 *                 N, n_cap, NULL) bytes, 256-byte aligned; no initial
 *                 contents required; holds the intermediates afterwards.
 *   n_cap         capacity for outlier columns, 0 <= n_cap <= K.  n_cap = K
 *                 is always enough; a smaller value is a promise, checked on
 *                 the device without a host sync: if the call finds more
 *                 outlier columns, header flag bit 0 is set and every
 *                 element of Y is a quiet NaN (never a plausible wrong
 *                 value).  The
 *                 packed X_out and W_outT must each stay within 2^31 bytes
 *                 (INT8MM_EINVAL otherwise).
 * M <= 32 takes the bandwidth-bound decode kernel, and so do 33-48 tokens
 * and 49-64 tokens with N <= 16384 or N = 16 * 256 * {5, 6} on a 256-CU
 * device (3 or 4 token blocks); larger M takes
 * the tiled int8-MFMA kernel; both give identical int32 accumulators.  The fp16
 * outlier product runs in the GEMM's epilogue: up to 16 outlier columns
 * from operands staged while the K loop runs, more (alpha -> 0) streamed
 * through LDS 32 columns at a time.
 * M == 0 or N == 0 is a no-op; K == 0 writes Y = bias (0 without one).
 */
int int8_mixed_matmul(const void *X_f16, int64_t M, int64_t K,
                      const int8_t *W_i8, const float *w_absmax,
                      const void *W_f16, int64_t N, float alpha,
                      const void *bias_f16, void *Y_f16, void *workspace,
                      size_t workspace_bytes, int64_t n_cap,
                      hipStream_t stream);

/*
 * Stage exports: the first two stages of int8_mixed_matmul, run by the same
 * kernels, alone.  For bit-exact tests of the intermediates and per-stage
 * timing; int8_mixed_matmul does not need them.  Both use the workspace of
 * int8_mixed_matmul for the same M, K, n_cap (and N) and leave their results
 * in its documented fields.
 *
 * int8_detect_outliers -- stage 1 ([JS 方法 2] / [GB "Seuil de détection
 * α"]): column k is an outlier iff max_i |X[i,k]| > alpha (strict, in fp32).
 *   X_f16     in  [M][K] fp16 activations.
 *   alpha     in  as for int8_mixed_matmul (NaN or < 0: INT8MM_EINVAL).
 *   n_cap     in  0 <= n_cap <= K: capacity of the outlier list.
 *   workspace     device, 256-byte aligned; the fields before INT8MM_WS_XOUT
 *                 must fit (any N gives the same offsets for them).
 * Writes COLMAX, MASK, IDX (ascending, first min(n, n_cap) valid) and HEADER
 * ([0] bit 0 set iff n > n_cap, [1] min(n, n_cap), [2] n, [3] 0), where n is
 * the number of outlier columns.  X_i8 is used as scratch.  M == 0 is a
 * no-op.
 */
int int8_detect_outliers(const void *X_f16, int64_t M, int64_t K, float alpha,
                         int64_t n_cap, void *workspace, size_t workspace_bytes,
                         hipStream_t stream);

/*
 * int8_quantize_activations -- stage 2 ([JS 方法 1]: vector-wise absmax
 * quantization of X per row; [ALI 图2]: outlier columns of X and the
 * matching rows of W leave for the fp16 path).  Reads MASK from a workspace
 * that int8_detect_outliers filled for the same X_f16, M, K and n_cap
 * (earlier on the same stream); anything else there gives undefined
 * results.
 *   X_f16     in  [M][K] fp16 activations.
 *   W_f16     in  [K][N] fp16 weights; only the outlier rows are read.
 *   workspace     device, 256-byte aligned, >= int8_mixed_matmul_workspace_
 *                 size(M, K, N, n_cap, NULL) bytes.
 * Writes XABS, XI8 (outlier columns 0), XOUT, WOUT, IDX and HEADER as
 * int8_mixed_matmul does before its GEMM.  M == 0 is a no-op.
 */
int int8_quantize_activations(const void *X_f16, int64_t M, int64_t K,
                              const void *W_f16, int64_t N, int64_t n_cap,
                              void *workspace, size_t workspace_bytes,
                              hipStream_t stream);

/*
 * Memory-lean outlier weights ([JS 观察 2]: the outlier dims are few and
 * fixed across tokens and batches, so they can be identified once;
 * [ALI §2.2]: the fp16 outlier part costs about 0.1 % extra memory).
 * Instead of keeping the whole fp16 W resident, keep only the fp16 rows of
 * a static set of outlier dims in a cache built once at load time.
 *
 * Cache layout (bytes, 256-byte aligned fields): int32[4] header {magic, K,
 * N, n_dims}; int32 slot[K] (row of dim k in the cache, -1 if absent);
 * fp16 rows [n_dims][N] (row s = W[dims[s], :]); int32 dims[n_dims].
 */
/* Bytes of the cache for n_dims static dims; -1 if out of range. */
int64_t int8_outlier_cache_size(int64_t K, int64_t N, int64_t n_dims);

/* Build the cache from W_f16 [K][N] (device) for the dims given in a HOST
 * array, strictly ascending, each in [0, K) (INT8MM_EINVAL otherwise).
 * cache: device, 256-byte aligned, >= int8_outlier_cache_size bytes.
 * Load-time call: it synchronizes `stream` before returning (the host
 * arrays it copies from must outlive the copies). */
int int8_build_outlier_cache(const void *W_f16, int64_t K, int64_t N,
                             const int32_t *dims, int64_t n_dims, void *cache,
                             size_t cache_bytes, hipStream_t stream);

/* int8_mixed_matmul with the outlier rows taken from a cache instead of the
 * whole fp16 W (same arguments otherwise, same workspace).  Detection is
 * unchanged.  A runtime outlier dim that is not in the cache uses its int8
 * row dequantized to fp16, fp16(fp32(q) * fp32(w_absmax/127)), and sets
 * bit 1 of the workspace status word: the result then departs from the
 * method.  With every runtime outlier cached the result is bit-identical
 * to int8_mixed_matmul's.  The kernels check the cache header: a cache
 * built for another K or N (or any buffer without the header) is not read
 * beyond its 16-byte header; every outlier then takes the dequantized
 * stand-in and status bit 2 is set.  The cache buffer must hold at least
 * those 16 bytes. */
int int8_mixed_matmul_cached(const void *X_f16, int64_t M, int64_t K,
                             const int8_t *W_i8, const float *w_absmax,
                             const void *cache, int64_t N, float alpha,
                             const void *bias_f16, void *Y_f16, void *workspace,
                             size_t workspace_bytes, int64_t n_cap,
                             hipStream_t stream);

/*
 * int8_mixed_matmul_noalloc -- int8_mixed_matmul without a workspace
 * argument, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.
 * The workspace is a static device array of INT8MM_NOALLOC_SCRATCH_BYTES
 * inside the library; each GPU the library runs on holds its own copy from
 * the first call on it until the process ends.  The call allocates and
 * frees nothing (the first call on a device looks the array's address up
 * once, so make that first call outside graph capture).
 *   Arguments as for int8_mixed_matmul (no workspace).  A shape whose
 *   workspace, int8_mixed_matmul_workspace_size(M, K, N, n_cap, NULL),
 *   exceeds INT8MM_NOALLOC_SCRATCH_BYTES returns INT8MM_ESCRATCH before any
 *   launch.  64 MiB holds, e.g., the 175B-scale QKV decode (M = 32,
 *   K = 12288, N = 36864) and the 175B-scale FFN prefill (M = 4096,
 *   K = 12288, N = 49152) with n_cap <= 128.
 *   Every call on one GPU shares that GPU's array and leaves its
 *   intermediates there: calls that overlap on one GPU (different streams,
 *   or different host threads) race and give undefined results; calls on
 *   one stream are ordered and safe.  Nothing in the array needs clearing
 *   between calls.
 */
#define INT8MM_NOALLOC_SCRATCH_BYTES (64u << 20)
int int8_mixed_matmul_noalloc(const void *X_f16, int64_t M, int64_t K,
                              const int8_t *W_i8, const float *w_absmax,
                              const void *W_f16, int64_t N, float alpha,
                              const void *bias_f16, void *Y_f16, int64_t n_cap,
                              hipStream_t stream);

/*
 * int8_gemm_i32 -- the int8 x int8 -> int32 product alone ([ALI 图2]:
 * Out_i32), run by the same K-loop as int8_mixed_matmul (decode kernel or
 * tiled MFMA kernel, chosen as there) with a plain int32 store instead of
 * the fp16 epilogue.  For bit-exact tests and per-kernel timing.
 *   X_i8  packed M x K int8, W_i8 packed N x K int8 (see int8_pack_rows),
 *   acc [M][N] int32 (out): acc[i][j] = sum_k X[i][k] * W[j][k].
 */
int int8_gemm_i32(const int8_t *X_i8, int64_t M, int64_t K, const int8_t *W_i8,
                  int64_t N, int32_t *acc, hipStream_t stream);

/*
 * The kernel configuration int8_mixed_matmul (and int8_gemm_i32) launches
 * for an M x K x N call on the current device; host only, no GPU work (256
 * compute units are assumed when no device can be queried).  cfg[4]:
 *   decode kernel (M <= 32, and up to 64 as above): {0, row blocks of 16
 *     features per workgroup (1-4, or 5, 6, 8, 9, 12 for the wide
 *     workgroups of M <= 32), K-splitting wavefronts (2 or 8; 2 above 32
 *     tokens), token blocks of 16 (1-4)};
 *   tiled GEMM: {1, tile rows BM, tile columns BN, wavefronts};
 *   tiled GEMM in two launches: {2, n1, tile columns BN, wavefronts of the
 *     second}: columns [0, n1) in 256x256 tiles, [n1, N) in BN-column tiles
 *     (128x128 with 4 wavefronts, 256x128 or 256x160 with 8).
 * For tuning sweeps and for tests that must reach every configuration.
 * Returns INT8MM_EINVAL / INT8MM_EALIGN for shapes the matmul rejects.
 */
int int8mm_kernel_config(int64_t M, int64_t N, int64_t K, int32_t *cfg);

/*
 * Profiling aid (not thread-safe; for benchmarks).  While enabled, every
 * int8_mixed_matmul call has the dispatch of its main kernel (the tiled
 * int8 GEMM, or the decode kernel for M <= 32) record a pair of HIP events
 * at that kernel's start and end (hipExtLaunchKernel), with no extra
 * packets on the stream.
 * int8mm_timing_read waits for the recorded events, returns the summed
 * kernel milliseconds and the number of timed launches, and clears them.
 * Events are created on first use and reused; no device memory is involved.
 */
int int8mm_timing_enable(int on);
int int8mm_timing_read(double *total_ms, int64_t *launches);

#ifdef __cplusplus
}
#endif

#endif /* INT8MM_H */
