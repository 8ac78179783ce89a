/*
 * swa_peaks.h -- microbenchmarks that measure the roofline denominators the
 * bench reports beside the vendor peaks: a streaming read of device memory
 * and a stream of bf16 matrix-core instructions.  They are measurement
 * tools, not part of the SWA(w,s) attention path (libswa_peaks.so, built
 * next to libswa.so).  Both enqueue one kernel on hip_stream and return 0,
 * or 1 for a bad argument (nothing enqueued), or 2 if the launch failed.
 */
#ifndef SWA_PEAKS_H
#define SWA_PEAKS_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads the bytes/16 sixteen-byte words of buf (device, 16-byte aligned,
 * caller-owned) once, with `blocks` workgroups of 256 threads, `unroll`
 * (4 or 8) loads in flight per thread and, if nt != 0, the non-temporal
 * cache policy.  sink: device, at least `blocks` unsigned ints; written
 * only if the xor of the data equals a fixed magic value (never for a
 * zeroed buffer).  Bytes moved: bytes (rounded down to 16). */
int swa_peak_stream_read(const void *buf, size_t bytes, unsigned *sink, int blocks, int unroll, int nt,
                         void *hip_stream);

/* `blocks` workgroups of 4 waves, each wave issuing 4 * iters
 * v_mfma_f32_32x32x16_bf16 (32768 flops each) on four independent
 * accumulators.  in: device, >= 2048 bytes, 16-byte aligned (operands);
 * sink: device, >= `blocks` floats, written only under a condition that a
 * zero input never meets.  Flops: blocks * 4 * 4 * iters * 32768. */
int swa_peak_mfma(const void *in, float *sink, int blocks, int iters, void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* SWA_PEAKS_H */
