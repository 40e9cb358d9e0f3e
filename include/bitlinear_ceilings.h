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

/* LDS traffic in the tiled GEMM's patterns, `blocks` blocks of 512 threads.
 * Waves 0-3 run `it_r` steps of four 16-byte LDS reads per lane (rows of a
 * padded 144-byte-pitch tile, the fragment pattern: 4 KB per wave and step);
 * waves 4-7 run `it_w` 16-byte LDS writes per lane: mode 0 none, mode 1
 * ds_write_b128 stores (8 lanes per 128-byte row of the same layout), mode 2
 * direct global-to-LDS loads (1 KB of LDS per wave and step) from the first
 * `window` bytes of `src` (16-byte aligned, at least 1 MiB, a multiple of
 * 16; unused otherwise).  Timing a mode against the readers alone and the
 * writers alone shows how much the two kinds of LDS write slow the reads.
 * `sink` as above. */
int blc_lds_mix(int mode, int it_r, int it_w, int blocks, const void *src, int64_t window,
                uint32_t *sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* BITLINEAR_CEILINGS_H */
