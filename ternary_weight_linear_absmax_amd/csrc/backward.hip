// Backward through BitLinear for the input: grad_x = gamma * grad_y * t.
//
// Source: lumen-it.ai BitNet article (training paragraph: straight-through
// estimators keep the gradient flowing through the quantisers).  With both
// quantisers passed straight through, the layer acts on x as the matrix
// gamma * t, so the input gradient is a product with the same packed ternary
// matrix, transposed: grad_x[m, k] = gamma * sum_n grad_y[m, n] t[n, k].
// (The weight gradient passes straight through to the latent weights and is
// a dense product of grad_y and the activations, not a ternary one.)
//
// fp32 arithmetic (the gradient is a float; no quantisation of it is implied
// by the sources).  Block tile 64 (m) x 128 (k), 256 threads with 4 x 8
// outputs each; the reduction over n runs in stages of 32: the grad_y tile
// [64 m x 32 n] is staged transposed in LDS, the packed tile [32 n x 128 k]
// (32 bytes per row) is unpacked once into floats in LDS and then used by all
// 64 m rows; the next stage's global data is loaded into registers while the
// current one is computed (double-buffered LDS).
#include "internal.h"

namespace bl {
namespace {

constexpr int BW_BM = 64, BW_BK = 128, BW_BN = 32;

template <int DT, bool VEC>
__global__ __launch_bounds__(256) void backward_input_kernel(const void *__restrict__ grad_y,
                                                             int64_t m, int64_t n,
                                                             const uint8_t *__restrict__ packed,
                                                             int64_t pitch, int64_t k,
                                                             const float *__restrict__ gamma_p,
                                                             float *__restrict__ grad_x)
{
    __shared__ __attribute__((aligned(16))) float gs[2][BW_BN][BW_BM];
    __shared__ __attribute__((aligned(16))) float ts[2][BW_BN][BW_BK];
    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;           // 16 x 8 k, 16 x 4 m
    const int64_t m0 = (int64_t)blockIdx.y * BW_BM, k0 = (int64_t)blockIdx.x * BW_BK;
    const int nst = (int)((n + BW_BN - 1) / BW_BN);
    const int64_t words = pitch / 4;

    // staging roles: grad_y row gm = m0 + tid / 4, columns 8 (tid % 4) .. +7;
    // packed row tn = tid / 8, word k0 / 16 + tid % 8 (16 trits)
    const int gr = tid >> 2, gc = 8 * (tid & 3);
    const int tr = tid >> 3, tw = tid & 7;
    const int64_t gm = m0 + gr;
    const int64_t wk = k0 / 16 + tw;
    float gv[8];
    uint32_t tv = 0;

    auto load = [&](int st) __attribute__((always_inline)) {
        const int64_t nb = (int64_t)st * BW_BN;
        if (VEC && gm < m && nb + gc + 8 <= n) {
            if (DT == DT_BF16) {
                const uint4 v = load16((const uint16_t *)grad_y + gm * n + nb + gc);
                const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    gv[2 * e] = bf16_lo(u[e]);
                    gv[2 * e + 1] = bf16_hi(u[e]);
                }
            } else {
                const float *p = (const float *)grad_y + gm * n + nb + gc;
                const uint4 a = load16(p), b = load16(p + 4);
                gv[0] = __uint_as_float(a.x); gv[1] = __uint_as_float(a.y);
                gv[2] = __uint_as_float(a.z); gv[3] = __uint_as_float(a.w);
                gv[4] = __uint_as_float(b.x); gv[5] = __uint_as_float(b.y);
                gv[6] = __uint_as_float(b.z); gv[7] = __uint_as_float(b.w);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int64_t nn = nb + gc + e;
                float v = 0.0f;
                if (gm < m && nn < n) {
                    if (DT == DT_BF16)
                        v = __uint_as_float((uint32_t)((const uint16_t *)grad_y)[gm * n + nn] << 16);
                    else
                        v = ((const float *)grad_y)[gm * n + nn];
                }
                gv[e] = v;
            }
        }
        const int64_t tn = nb + tr;
        // rows past N and words past the row contribute nothing (code 1 = trit 0)
        tv = (tn < n && wk < words) ? ((const uint32_t *)(packed + tn * pitch))[wk] : 0x55555555u;
    };
    auto store = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int e = 0; e < 8; ++e) gs[buf][gc + e][gr] = gv[e];
        // word holds k = 16 tw + 4 i + j at byte j, bits 2 i (code t + 1)
        float f[16];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                f[4 * i + j] = (float)(int)((tv >> (8 * j + 2 * i)) & 3u) - 1.0f;
        float4 *dst = (float4 *)&ts[buf][tr][16 * tw];
#pragma unroll
        for (int q = 0; q < 4; ++q) dst[q] = make_float4(f[4 * q], f[4 * q + 1], f[4 * q + 2], f[4 * q + 3]);
    };

    float acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;

    load(0);
    store(0);
    __syncthreads();
    for (int st = 0; st < nst; ++st) {
        const int buf = st & 1;
        if (st + 1 < nst) load(st + 1);
#pragma unroll 4
        for (int nn = 0; nn < BW_BN; ++nn) {
            const float4 a = *(const float4 *)&gs[buf][nn][4 * ty];
            const float4 b0 = *(const float4 *)&ts[buf][nn][8 * tx];
            const float4 b1 = *(const float4 *)&ts[buf][nn][8 * tx + 4];
            const float av[4] = {a.x, a.y, a.z, a.w};
            const float bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
        }
        if (st + 1 < nst) store(buf ^ 1);
        __syncthreads();
    }

    const float gamma = gamma_p[0];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t row = m0 + 4 * ty + i;
        if (row >= m) continue;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int64_t col = k0 + 8 * tx + j;
            if (col < k) grad_x[row * k + col] = gamma * acc[i][j];
        }
    }
}

}  // namespace

hipError_t launch_backward_input(const void *grad_y, int dtype, int64_t m, int64_t n,
                                 const uint8_t *packed, int64_t k, const float *gamma,
                                 float *grad_x, hipStream_t s)
{
    const dim3 grid((unsigned)((k + BW_BK - 1) / BW_BK), (unsigned)((m + BW_BM - 1) / BW_BM));
    const int64_t pitch = pack2_pitch(k);
    // 16-byte loads need every grad_y row 16-byte aligned
    const bool vec = dtype == DT_BF16 ? n % 8 == 0 : n % 4 == 0;
    if (dtype == DT_BF16) {
        if (vec)
            hipLaunchKernelGGL((backward_input_kernel<DT_BF16, true>), grid, dim3(256), 0, s,
                               grad_y, m, n, packed, pitch, k, gamma, grad_x);
        else
            hipLaunchKernelGGL((backward_input_kernel<DT_BF16, false>), grid, dim3(256), 0, s,
                               grad_y, m, n, packed, pitch, k, gamma, grad_x);
    } else {
        if (vec)
            hipLaunchKernelGGL((backward_input_kernel<DT_F32, true>), grid, dim3(256), 0, s,
                               grad_y, m, n, packed, pitch, k, gamma, grad_x);
        else
            hipLaunchKernelGGL((backward_input_kernel<DT_F32, false>), grid, dim3(256), 0, s,
                               grad_y, m, n, packed, pitch, k, gamma, grad_x);
    }
    return hipGetLastError();
}

}  // namespace bl
