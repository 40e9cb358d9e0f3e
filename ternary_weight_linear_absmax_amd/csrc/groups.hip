// Group quantisation of the sign-binarised weights: one scale per group of
// consecutive output features.
//
// Source: lumen-it.ai article on the original 1-bit BitNet (group
// quantisation and normalisation, so that the layer can be split over devices
// with little communication).  Each of G equal groups of weight rows has its
// own scale beta_g = mean |W_g|; a BitLinear output column n takes the scale
// of its group, y[m, n] = acc[m, n] * beta_g / s[m].
//
// The product kernels write the exact int32 accumulators into the caller's y
// buffer (same size as the float output); this kernel then rescales them in
// place, one element per thread.
#include "internal.h"

namespace bl {
namespace {

__global__ __launch_bounds__(256) void group_rescale_kernel(float *__restrict__ y,
                                                            const float *__restrict__ scale,
                                                            const float *__restrict__ beta,
                                                            int64_t m, int64_t n,
                                                            int64_t rows_per_group)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= m * n) return;
    const int64_t gm = i / n, gn = i % n;
    const int32_t acc = __float_as_int(y[i]);          // the int32 accumulator's bits
    y[i] = epi_y(acc, epi_gs(beta[gn / rows_per_group], scale[gm]));
}

}  // namespace

hipError_t launch_group_rescale(float *y, const float *scale, const float *beta, int64_t m,
                                int64_t n, int64_t rows_per_group, hipStream_t s)
{
    const int64_t total = m * n;
    hipLaunchKernelGGL(group_rescale_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                       s, y, scale, beta, m, n, rows_per_group);
    return hipGetLastError();
}

}  // namespace bl
