/* bitlinear_ceiling.h -- measurement kernels for the two rooflines of the BitLinear path on
 * MI355X (gfx950): HBM streaming read and int8 MFMA issue rate.  They sit in their own library
 * (libbitlinear_ceiling.so) next to libbitlinear.so and compute nothing of the method; bench.py
 * times them the way it times the path's kernels, to report each roofline fraction against a
 * ceiling measured on the same GPU in the same run as well as against the published peak.
 *
 * All pointers are device memory owned by the caller; calls are asynchronous on `stream`.
 * Return 0 on success, -1 for an invalid argument, -5 for a HIP launch error. */
#ifndef BITLINEAR_CEILING_H
#define BITLINEAR_CEILING_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* One pass of a streaming read over `bytes` bytes at `src` (16-byte aligned, bytes a multiple
 * of 16): every byte is loaded once with 128-bit non-temporal loads, all loads of a thread
 * issued before any is used; the XOR of everything read goes to sink[0..1023] only if it hits
 * a fixed improbable value, so the loads cannot be removed.  sink: 1024 ints. */
int bitlinear_ceiling_read(const void* src, size_t bytes, int* sink, hipStream_t stream);

/* `blocks` workgroups of 256 threads, each wave issuing `iters` x 16 independent
 * v_mfma_i32_32x32x32_i8 on operands taken from `operands` (65536 ints, read once; random
 * values make the realistic power draw, constant ones the best case).  *ops_out (host) receives
 * the int8 operations of the launch: blocks * 4 * iters * 16 * 2 * 32 * 32 * 32.  sink: 1024 ints. */
int bitlinear_ceiling_mfma(int blocks, int iters, const int* operands, int* sink, int64_t* ops_out,
                           hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif
