/*
 * dar_calib.h -- calibration kernels used by the benchmark (libdar_calib.so).
 *
 * Not part of the DAR ABI in dar.h: these measure what this device reaches
 * on plain work, so that the DAR kernels' rates can be reported against the
 * measured peaks as well as the vendor figures.  Device pointers, work
 * enqueued on `stream`; the int results are hipError_t values (0 = success,
 * hipErrorInvalidValue for bad arguments, checked before any launch).
 */
#ifndef DAR_CALIB_H
#define DAR_CALIB_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* FLOP performed by one dar_calib_mfma(workgroups, iters, shape) call. */
double dar_calib_mfma_flops(int workgroups, int iters, int shape);

/* Dense fp16 MFMA rate: `workgroups` workgroups of 4 waves, each wave issuing
 * 4*iters independent fp16 MFMAs from registers (shape 0: 32x32x16,
 * shape 1: 16x16x32).  sink: device buffer of workgroups*256 floats (written
 * only in an impossible case). */
int dar_calib_mfma(float* sink, int workgroups, int iters, int shape, hipStream_t stream);

/* Device-to-device copy of `bytes` (multiple of 16; 16-byte aligned pointers)
 * with 16-byte loads and stores. */
int dar_calib_copy(const void* src, void* dst, size_t bytes, hipStream_t stream);

/* Device read of `bytes` (multiple of 16; 16-byte aligned) with 16-byte
 * loads, eight in flight per thread.  sink: device buffer of >= 8192
 * unsigned (written only in an impossible case). */
int dar_calib_read(const void* src, size_t bytes, unsigned* sink, hipStream_t stream);

/* Device read of `bytes` (multiple of 16384; 16-byte aligned) by direct
 * buffer loads into LDS, 16 KB per workgroup step: the load path of the DAR
 * kernels' tile staging, for scaling traffic counters. */
int dar_calib_read_lds(const void* src, size_t bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DAR_CALIB_H */
