// Measured ceilings of the machine, for the benchmark only (not part of the
// BitLinear library): a plain streaming read of HBM with 16-byte loads, an
// int8 matrix-core loop with no memory traffic, an empty kernel (the cost of
// one launch), and LDS traffic in the GEMM's patterns (fragment reads alone,
// and next to either ds_write_b128 stores or direct global-to-LDS loads from
// other waves of the block).  The benchmark reports each BitLinear kernel
// against these as well as against the vendor peaks.
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

// LDS traffic of a GEMM block (512 threads, two blocks per CU when launched
// with 2 x CUs blocks).  Waves 0-3 ("readers") issue `it_r` steps of four
// ds_read_b128 each, lane (l % 32, l / 32) reading row l % 32 of a padded
// [64][144-byte] tile (the fragment pattern, free of bank conflicts);
// waves 4-7 ("writers") issue `it_w` 16-byte stores each: mode 1 as
// ds_write_b128 (eight lanes per 128-byte row of the same padded tile layout),
// mode 2 as direct loads global_load_lds_dwordx4 from a window of `src` (each
// instruction fills 1 KB of LDS); mode 0: no writers.
constexpr int LDS_ROW = 144;
constexpr int LDS_TILE = 64 * LDS_ROW;
typedef __attribute__((address_space(3))) void lds_void_t;

__global__ __launch_bounds__(512) void lds_mix_kernel(int mode, int it_r, int it_w,
                                                      const uint8_t *__restrict__ src,
                                                      int64_t window, uint32_t *sink,
                                                      uint32_t magic)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[6 * LDS_TILE];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int i = tid; i < 3 * LDS_TILE / 4; i += 512) ((uint32_t *)lds)[i] = (uint32_t)i;
    __syncthreads();
    uint32_t acc = 0;
    if (wave < 4) {
        const int base = ((wave & 1) * 32 + (lane & 31)) * LDS_ROW + 64 * (lane >> 5);
        for (int i = 0; i < it_r; ++i) {
            const uint8_t *p = lds + (i % 3) * LDS_TILE + base;
            const u32x4 v0 = *(const u32x4 *)p, v1 = *(const u32x4 *)(p + 16);
            const u32x4 v2 = *(const u32x4 *)(p + 32), v3 = *(const u32x4 *)(p + 48);
            const u32x4 x = v0 ^ v1 ^ v2 ^ v3;
            acc ^= x.x ^ x.y ^ x.z ^ x.w;
            asm volatile("" ::: "memory");
        }
    } else if (mode == 1) {
        const int e = tid - 256;
        const int base = 3 * LDS_TILE + (e >> 3) * LDS_ROW + (e & 7) * 16;
        u32x4 v = {(uint32_t)e, 1u, 2u, 3u};
        for (int i = 0; i < it_w; ++i) {
            *(u32x4 *)(lds + base + (i % 2) * (32 * LDS_ROW)) = v;
            v.x += 1u;
            asm volatile("" ::: "memory");
        }
        acc = v.x;
    } else if (mode == 2) {
        // lane sources spread over the window less 16 steps of 32 KB, so
        // that every step stays inside it
        const int w4 = wave - 4;
        const int64_t lanes = (window - 16 * 32768) / 16;
        const uint8_t *s = src + (((int64_t)blockIdx.x * 256 + (tid - 256)) % lanes) * 16;
        for (int i = 0; i < it_w; ++i) {
            const uint8_t *g = s + (i & 15) * 32768;
            __builtin_amdgcn_global_load_lds((const void *)g,
                                             (lds_void_t *)(lds + 3 * LDS_TILE + (i % 6) * 4096 +
                                                            w4 * 1024),
                                             16, 0, 0);
            if ((i & 3) == 3) __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);
    }
    __syncthreads();
    acc ^= ((const uint32_t *)lds)[3 * LDS_TILE / 4 + tid];
    if (acc == magic) sink[0] = acc;
}

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

int blc_lds_mix(int mode, int it_r, int it_w, int blocks, const void *src, int64_t window,
                uint32_t *sink, hipStream_t stream)
{
    if (!sink || mode < 0 || mode > 2 || it_r < 0 || it_w < 0 || blocks < 1) return -1;
    if (mode == 2 && (!src || window < (1 << 20) || window % 16 != 0 || ((uintptr_t)src & 15u)))
        return -1;
    hipLaunchKernelGGL(lds_mix_kernel, dim3((unsigned)blocks), dim3(512), 0, stream, mode, it_r,
                       it_w, (const uint8_t *)src, window, sink, 0x9E3779B9u);
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // extern "C"
