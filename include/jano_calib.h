/* Calibration aid for measurements (not part of the Jano path).
 *
 * jano_calib_mfma_loop launches `workgroups` workgroups of 512 threads
 * (8 waves, two per SIMD, one workgroup per CU) that each run `iters`
 * iterations of a register-only loop of independent bf16 MFMAs, 524288 flop
 * per wave per iteration: shape 0 uses v_mfma_f32_16x16x32_bf16, shape 1
 * v_mfma_f32_32x32x16_bf16. Timed with events on `stream`, it gives the
 * matrix-core rate the part sustains under full load, a measured ceiling to
 * set beside the published peak.
 *
 *   sink    device buffer of workgroups * 512 floats; written only in a case
 *           that does not occur (it keeps the loop from being removed)
 *   cycles  NULL, or a device buffer of workgroups * 8 int64 that receives
 *           each wave's shader-clock cycles for its loop
 *   stream  hipStream_t, or NULL for the default stream
 *
 * Returns 0 on success, 1 for a bad argument (shape not 0 or 1, workgroups or
 * iters < 1, sink NULL; nothing is launched), 2 when the launch fails.
 * Buffers belong to the caller. The call is asynchronous.
 *
 * jano_calib_stream streams `bytes` bytes (a multiple of 16, buffers 16-byte
 * aligned) with `workgroups` workgroups of 256 threads, grid-stride, four
 * 16-byte non-temporal loads in flight per thread. Timed with events, it
 * gives the HBM rate plain streaming reaches on the part.
 *
 *   mode 0  copy: dst[0 .. bytes) = src[0 .. bytes) (non-temporal stores);
 *           sink unused
 *   mode 1  read: src is read and summed per thread; dst unused; sink is a
 *           device buffer of workgroups * 256 floats, written only in a case
 *           that does not occur (it keeps the loads from being removed)
 *
 * Returns 0 on success, 1 for a bad argument (mode not 0 or 1, src NULL or
 * misaligned, bytes 0 or not a multiple of 16, workgroups < 1, dst NULL or
 * misaligned in mode 0, sink NULL in mode 1; nothing is launched), 2 when
 * the launch fails. The buffers must not overlap.
 */
#ifndef JANO_CALIB_H
#define JANO_CALIB_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

int jano_calib_mfma_loop(int shape, int workgroups, int iters, float *sink, long long *cycles,
                         void *stream);
int jano_calib_stream(int mode, const void *src, void *dst, size_t bytes, int workgroups, float *sink,
                      void *stream);

#ifdef __cplusplus
}
#endif

#endif /* JANO_CALIB_H */
