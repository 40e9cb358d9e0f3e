/*
 * bitlinear_ceilings.h - measured machine ceilings for the benchmark
 * (libbitlinear_ceilings.so).  Not part of the BitLinear ABI: these kernels
 * compute nothing of the method; they bound what the BitLinear kernels can
 * reach on the device they run on.
 *
 * All calls are asynchronous on `stream` and return 0, or -1 for a bad
 * argument (nothing launched), -2 for a failed launch.
 */
#ifndef BITLINEAR_CEILINGS_H
#define BITLINEAR_CEILINGS_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` (a multiple of 16) of device memory at `src` (16-byte
 * aligned) once, with non-temporal 16-byte loads from `blocks` blocks of 256
 * threads striding over the buffer; writes nothing (`sink`, one device word,
 * is a store target the kernel never reaches). */
int blc_read_stream(const void *src, int64_t bytes, int blocks, uint32_t *sink,
                    hipStream_t stream);

/* int8 matrix-core work of blc_mfma_i8_loop(iters, blocks): multiply-add
 * operations counted as two each. */
int64_t blc_mfma_i8_ops(int iters, int blocks);

/* `blocks` blocks of four waves, each wave advancing eight independent 32x32
 * int32 accumulators with v_mfma_i32_32x32x32_i8 `iters` times on register
 * operands (no memory traffic); `sink` as above. */
int blc_mfma_i8_loop(int iters, int blocks, int32_t *sink, hipStream_t stream);

/* One block of one wave that does nothing: the cost of a launch. */
int blc_empty(hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* BITLINEAR_CEILINGS_H */
