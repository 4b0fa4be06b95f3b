/* Peak micro-benchmarks exported by libavey.so.
 *
 * Not part of the Avey-B hot path: they measure the two ceilings the hot path's roofline
 * fractions are also reported against, next to the MI355X datasheet peaks (bf16 dense MFMA
 * 2.5 PFLOP/s, HBM3E 8 TB/s): the bf16 matrix-core rate and the device-memory copy bandwidth.
 * Same conventions as avey.h: device pointers owned by the caller, work enqueued on `stream`
 * (a hipStream_t; NULL is the default stream), never synchronises, returns an avey_status from
 * host-side checks and the launch.
 */
#ifndef AVEY_PROBE_H
#define AVEY_PROBE_H

#include "avey.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * avey_probe_mfma_flops -- bf16 FLOPs that one avey_probe_mfma_bf16 launch with `iters`
 * iterations performs on the current device (one workgroup per compute unit), or a negative
 * avey_status: AVEY_ERR_SHAPE if iters < 1, AVEY_ERR_HIP if the device cannot be queried.
 */
int64_t avey_probe_mfma_flops(int64_t iters);

/*
 * avey_probe_mfma_bf16 -- matrix-core throughput on register operands.
 *
 * One 8-wave workgroup per compute unit; per iteration every wave issues 16 independent
 * 32x32x16 bf16 MFMAs (8 accumulator blocks, two k-steps), with no memory traffic.
 *   iters     iterations, >= 1 (AVEY_ERR_SHAPE otherwise)
 *   changing  0: the same operands throughout; non-zero: new operand bit patterns every
 *             iteration (random signs and mantissas, exponents near 1), made by a few integer
 *             operations, as operands streamed from memory would change. The chip's power draw,
 *             and so its clock, depends on how much the operand bits toggle.
 *   sink      device buffer of at least one float per compute unit (AVEY_ERR_NULL if NULL,
 *             AVEY_ERR_ALIGN if not 4-byte aligned); written only in a case that does not occur,
 *             so that the work cannot be removed.
 * FLOPs per launch: avey_probe_mfma_flops(iters).
 */
avey_status avey_probe_mfma_bf16(int64_t iters, int32_t changing, float* sink, void* stream);

/*
 * avey_probe_copy -- dst[0, bytes) = src[0, bytes), with 16-byte vector loads and stores.
 *   src, dst  device buffers, 16-byte aligned (AVEY_ERR_ALIGN), not overlapping, non-NULL
 *             unless bytes == 0 (AVEY_ERR_NULL)
 *   bytes     a multiple of 16, >= 0 (AVEY_ERR_SHAPE); 0 is a no-op
 * Bytes moved through memory per launch: 2 * bytes (read and written once).
 */
avey_status avey_probe_copy(const void* src, void* dst, int64_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* AVEY_PROBE_H */
