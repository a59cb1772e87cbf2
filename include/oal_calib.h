/*
 * oal_calib.h -- measurement aids shipped in liboal.so beside the OAL calls.
 *
 * These are not steps of the attention method. They measure, on the device at hand, the two
 * ceilings the OAL kernels are compared with: the dense bf16 matrix-core rate (a loop of
 * independent v_mfma_f32_16x16x32_bf16 chains, the instruction the prefill readout issues) and
 * the streaming HBM rate (a plain device-to-device copy with 16-byte accesses). A benchmark
 * brackets each call with timing events and divides the work the call reports by the time.
 *
 * Errors follow oal.h: arguments are checked on the host; on error nothing is enqueued.
 */
#ifndef OAL_CALIB_H
#define OAL_CALIB_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#include "oal.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Matrix-core loop: `blocks` workgroups of 256 threads (4 wavefronts); each wavefront runs
 * `iters` rounds of 8 independent 16x16x32 bf16 MFMA chains on register operands and writes
 * one float per thread to `out` (device, blocks * 256 floats) so the work is kept. *flops
 * (host, may be NULL) receives the dense flop count: blocks * 4 * iters * 8 * 2 * 16 * 16 * 32.
 * blocks in [1, 65536], iters in [1, 1 << 20]; otherwise OAL_E_ARG. */
oal_status oal_calib_mfma_bf16(int blocks, int iters, float *out, double *flops, hipStream_t stream);

/* Streaming copy of `bytes` from `src` to `dst` (device, non-overlapping, 16-byte aligned,
 * bytes a multiple of 16): one 16-byte load and store per thread, a flat grid (capped at
 * 1024 workgroups per compute unit, which then stride). Moves 2 * bytes of HBM traffic when
 * the buffers exceed the caches. Misaligned pointers give OAL_E_ALIGN, a size not a multiple of 16 OAL_E_ARG. */
oal_status oal_calib_copy(const void *src, void *dst, size_t bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif
