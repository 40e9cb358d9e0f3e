// Measured ceilings of the machine, for the benchmark only (not part of the
// BitLinear library): a plain streaming read of HBM with 16-byte loads, an
// int8 matrix-core loop with no memory traffic, and an empty kernel (the cost
// of one launch).  The benchmark reports each BitLinear kernel against these
// as well as against the vendor peaks.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/bitlinear_ceilings.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int READ_UNROLL = 4;

// Every thread reads READ_UNROLL 16-byte vectors per step, grid-stride over
// the buffer (consecutive lanes read consecutive 16-byte pieces), and folds
// them into a running XOR that is stored only when it equals `magic` (a
// run-time value the data never produces), so the loads stay live without
// writing anything.
__global__ __launch_bounds__(256) void read_stream_kernel(const u32x4 *__restrict__ src,
                                                          int64_t vecs, uint32_t *sink,
                                                          uint32_t magic)
{
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i + (READ_UNROLL - 1) * stride < vecs; i += READ_UNROLL * stride) {
        u32x4 v[READ_UNROLL];
#pragma unroll
        for (int u = 0; u < READ_UNROLL; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < READ_UNROLL; ++u) acc ^= v[u];
    }
    for (; i < vecs; i += stride) acc ^= __builtin_nontemporal_load(src + i);
    const uint32_t r = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (r == magic) sink[0] = r;
}

// CHAINS independent accumulators per wave, each advanced by
// v_mfma_i32_32x32x32_i8 `iters` times; operands stay in registers.
constexpr int CHAINS = 8;

__global__ __launch_bounds__(256) void mfma_i8_loop_kernel(int iters, int32_t *sink, int magic)
{
    const int lane = threadIdx.x & 63;
    const v4i a = {lane, lane * 3, lane ^ 5, 7};
    const v4i b = {lane * 5, 11, lane, lane ^ 9};
    v16i acc[CHAINS];
#pragma unroll
    for (int c = 0; c < CHAINS; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[c][r] = 0;
    for (int i = 0; i < iters; ++i)
#pragma unroll
        for (int c = 0; c < CHAINS; ++c)
            acc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[c], 0, 0, 0);
    int s = 0;
#pragma unroll
    for (int c = 0; c < CHAINS; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[c][r];
    if (s == magic) sink[0] = s;
}

__global__ void empty_kernel() {}

}  // namespace

extern "C" {

int blc_read_stream(const void *src, int64_t bytes, int blocks, uint32_t *sink, hipStream_t stream)
{
    if (!src || !sink || bytes < 16 || bytes % 16 != 0 || blocks < 1) return -1;
    if (((uintptr_t)src & 15u) != 0) return -1;
    hipLaunchKernelGGL(read_stream_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const u32x4 *)src, bytes / 16, sink, 0x9E3779B9u);
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

int64_t blc_mfma_i8_ops(int iters, int blocks)
{
    // 4 waves per block, CHAINS MFMAs per iteration, 2 * 32 * 32 * 32 ops each
    return (int64_t)blocks * 4 * CHAINS * iters * 2 * 32 * 32 * 32;
}

int blc_mfma_i8_loop(int iters, int blocks, int32_t *sink, hipStream_t stream)
{
    if (!sink || iters < 1 || blocks < 1) return -1;
    hipLaunchKernelGGL(mfma_i8_loop_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, iters,
                       sink, 0x7FFFFFF1);
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

int blc_empty(hipStream_t stream)
{
    hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, stream);
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // extern "C"
