/*
 * int8mm_probes.h -- peak probes for MI355X (gfx950), the measured ceilings
 * that the int8mm kernels' roofline fractions are also reported against
 * (besides the published peaks: 5.0 POP/s dense int8 MFMA, 8 TB/s HBM3E).
 *
 * Not part of the matmul: these kernels only measure the chip.  Each entry
 * point enqueues one kernel on `stream` and returns at once; the caller
 * times it (events on the same stream) and divides the work the comment
 * states by the time.  Pointers are device pointers owned by the caller.
 * Return value: 0 on success, otherwise the hipError_t of the launch.
 */
#ifndef INT8MM_PROBES_H
#define INT8MM_PROBES_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Dense int8 MFMA rate with no memory traffic in the loop: `blocks`
 * workgroups of 256 threads (4 wavefronts); every wavefront runs `iters`
 * iterations of 8 v_mfma_i32_16x16x64_i8 (32768 ops each) on 4 independent
 * accumulators.  Work = blocks * 4 * iters * 8 * 32768 ops.
 *   operands  device, >= 8 KB: the wavefronts' A/B fragments (lane l reads
 *             bytes 16*l .. of eight 1 KB fragments).  random != 0: the
 *             eight fragments differ, so consecutive MFMAs switch operands
 *             (the power behaviour of a real GEMM); random == 0: every MFMA
 *             sees the first fragment only.
 *   sink      device int32 [blocks * 256]: the accumulators' sums (kept
 *             so nothing is optimized away).
 */
int int8mm_probe_mfma_i8(const int8_t *operands, int random, int64_t blocks, int64_t iters,
                         int32_t *sink, hipStream_t stream);

/*
 * Dense fp16 MFMA rate, the same loop with v_mfma_f32_16x16x32_f16 (16384
 * flops each, fp32 accumulators): the ceiling of the outlier product's
 * fp16 path.  Work = blocks * 4 * iters * 8 * 16384 flops.
 *   operands  device, >= 8 KB of fp16 values (eight 1 KB fragments, as
 *             above); finite values, so the sums stay finite.
 *   sink      device float [blocks * 256].
 */
int int8mm_probe_mfma_f16(const void *operands, int random, int64_t blocks, int64_t iters,
                          float *sink, hipStream_t stream);

/*
 * Streaming read rate: `blocks` workgroups of 256 threads read all of
 * buf [bytes] (bytes a multiple of 16) with 16-byte loads, four in flight
 * per thread, grid-stride; nontemporal != 0 uses nontemporal loads (as the
 * decode kernel's weight stream does).  Work = bytes read.
 *   sink      device uint32 [blocks]: per-workgroup XOR of the data.
 */
int int8mm_probe_read(const void *buf, size_t bytes, int nontemporal, int64_t blocks,
                      uint32_t *sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* INT8MM_PROBES_H */
