// Decoder-block glue around the BitLinear layers of the 2B-class layer stack:
// the input of every BitLinear is RMSNorm'ed and then quantised per token.
//
// Sources: asi.tokyo BitNet b1.58 2B4T article, stabiliser paragraph (a norm
// in front of the sub-layers, squared ReLU in the feed-forward block);
// cheatsheet.md summary of BitNet b1.58, "What is BitNet b1.58?" (RMSNorm, no
// bias; activations scaled per token).
//
// One 256-thread block per token row.  The row's pre-norm values are formed in
// registers (double precision), in one of three ways:
//   residual:  x += add (float, written back), value = x
//   gqa:       the value vectors of the first token's attention, each query
//              head reading key-value head h / (heads / kv_heads)
//   relu2:     value = relu(gate)^2 * up (double)
// then RMSNorm with unit gain in double precision (sum of squares reduced over
// the block), rounded to float, and the absmax quantiser with the same
// arithmetic as bitlinear_quantize_act (s = 127 / max|h|, q = rint(h * s)).
#include "internal.h"

namespace bl {
namespace {

__device__ inline float block_max(float v, float *red)
{
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    v = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    return v;
}

__device__ inline double block_sum_d(double v, double *red)
{
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    return (red[0] + red[1]) + (red[2] + red[3]);
}

__device__ inline int block_sum_i(int v, int *red)
{
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    return (red[0] + red[1]) + (red[2] + red[3]);
}

template <int MODE, int EPT>
__global__ __launch_bounds__(256) void glue_kernel(GlueArgs a, int64_t k, double eps,
                                                   int8_t *__restrict__ xq,
                                                   float *__restrict__ scale,
                                                   int32_t *__restrict__ rowsum)
{
    __shared__ double red_d[4];
    __shared__ float red_f[4];
    __shared__ int red_i[4];
    const int tid = threadIdx.x;
    const int64_t m = blockIdx.x;
    const int kk = (int)k;

    // All of the thread's loads first (indices clamped into the row, values
    // past K unused), so that they are in flight together.
    float f0[EPT], f1[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int i = tid + 256 * j;
        const int ic = i < kk ? i : kk - 1;
        if (MODE == GLUE_RESIDUAL) {
            f0[j] = a.x[m * k + ic];
            f1[j] = a.add ? a.add[m * k + ic] : 0.0f;
        } else if (MODE == GLUE_GQA) {
            const unsigned hd = (unsigned)a.head_dim, head = (unsigned)ic / hd;
            const unsigned d = (unsigned)ic - head * hd;
            f0[j] = a.src[m * a.ld + a.col + (int64_t)(head / (unsigned)a.group) * hd + d];
        } else {
            f0[j] = a.src[m * a.ld + ic];             // gate
            f1[j] = a.src[m * a.ld + a.col + ic];     // up
        }
    }

    double v[EPT];
    double ss = 0.0;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int i = tid + 256 * j;
        if (MODE == GLUE_RESIDUAL) {
            const float xv = a.add ? f0[j] + f1[j] : f0[j];
            if (a.add && i < kk) a.x[m * k + i] = xv;
            v[j] = (double)xv;
        } else if (MODE == GLUE_GQA) {
            v[j] = (double)f0[j];
        } else {
            const double gd = f0[j] > 0.0f ? (double)f0[j] : 0.0;
            v[j] = gd * gd * (double)f1[j];
        }
        if (i >= kk) v[j] = 0.0;
        ss += v[j] * v[j];
    }
    ss = block_sum_d(ss, red_d);
    const double inv = 1.0 / sqrt(ss / (double)k + eps);

    float h[EPT];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        h[j] = (float)(v[j] * inv);
        amax = fmaxf(amax, fabsf(h[j]));
    }
    amax = block_max(amax, red_f);
    const float s = act_scale(amax);

    int sum = 0;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int i = tid + 256 * j;
        if (i >= kk) continue;
        const int8_t q = quant1(h[j], s);
        sum += q;
        xq[m * k + i] = q;
    }
    sum = block_sum_i(sum, red_i);
    if (tid == 0) {
        scale[m] = s;
        rowsum[m] = sum;
    }
}

template <int MODE>
hipError_t launch_mode(const GlueArgs &a, int64_t m, int64_t k, double eps, int8_t *xq,
                       float *scale, int32_t *rowsum, hipStream_t s)
{
    const dim3 grid((unsigned)m), block(256);
    const int64_t per = (k + 255) / 256;
    if (per <= 4)
        hipLaunchKernelGGL((glue_kernel<MODE, 4>), grid, block, 0, s, a, k, eps, xq, scale, rowsum);
    else if (per <= 8)
        hipLaunchKernelGGL((glue_kernel<MODE, 8>), grid, block, 0, s, a, k, eps, xq, scale, rowsum);
    else if (per <= 16)
        hipLaunchKernelGGL((glue_kernel<MODE, 16>), grid, block, 0, s, a, k, eps, xq, scale, rowsum);
    else
        hipLaunchKernelGGL((glue_kernel<MODE, 32>), grid, block, 0, s, a, k, eps, xq, scale, rowsum);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_glue(int mode, const GlueArgs &a, int64_t m, int64_t k, double eps,
                       int8_t *xq, float *scale, int32_t *rowsum, hipStream_t s)
{
    switch (mode) {
    case GLUE_RESIDUAL: return launch_mode<GLUE_RESIDUAL>(a, m, k, eps, xq, scale, rowsum, s);
    case GLUE_GQA: return launch_mode<GLUE_GQA>(a, m, k, eps, xq, scale, rowsum, s);
    default: return launch_mode<GLUE_RELU2>(a, m, k, eps, xq, scale, rowsum, s);
    }
}

}  // namespace bl
