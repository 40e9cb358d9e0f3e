// Per-token absmax quantisation of activations to int8.
//
// Sources: cheatsheet.md summary of BitNet b1.58, section "What is BitNet
// b1.58?", activation bullet (each token is scaled into a symmetric range);
// asi.tokyo BitNet b1.58 2B4T article (8-bit values travel between layers);
// lumen-it.ai BitNet article (absmax quantisation of activations).
//
// s = 127 / max|x| (IEEE float division), q = clamp(rint(x * s), -127, 127)
// with a float multiply and round-half-to-even; an all-zero token gets s = 1.
// Narrower activations (b bits, a future direction the cheatsheet.md summary
// names in its outlook) use Q = 2^(b-1) - 1 in place of 127.
// The row sum of q is emitted as well: the products use the 2-bit codes
// t + 1 and subtract it once per token.
//
// One 256-thread block per token: a max pass, a block reduction, then a
// quantise pass that re-reads the (cache-resident) row.
#include "internal.h"

namespace bl {
namespace {


// Vector path: 16-byte loads (8 bf16 or 4 fp32); requires K to be a multiple
// of the vector width so that every row stays 16-byte aligned.
template <int DT, bool VEC>
__global__ __launch_bounds__(256) void quant_act_kernel(const void *__restrict__ x, int64_t k,
                                                        int8_t *__restrict__ xq,
                                                        float *__restrict__ scale,
                                                        int32_t *__restrict__ rowsum,
                                                        float qmax)
{
    __shared__ float red_f[4];
    __shared__ int red_i[4];
    constexpr int E = DT == DT_BF16 ? 8 : 4;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t m = blockIdx.x;
    const uint8_t *row = (const uint8_t *)x + m * k * (DT == DT_BF16 ? 2 : 4);
    int8_t *qrow = xq + m * k;

    float amax = 0.0f;
    if (VEC) {
        const uint4 *v = (const uint4 *)row;
        for (int64_t i = tid; i < k / E; i += 256) {
            uint4 d = v[i];
            uint32_t w[4] = {d.x, d.y, d.z, d.w};
            if (DT == DT_BF16) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(w[e])), fabsf(bf16_hi(w[e]))));
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fabsf(__uint_as_float(w[e])));
            }
        }
    } else {
        for (int64_t i = tid; i < k; i += 256) {
            float f = DT == DT_BF16 ? __uint_as_float((uint32_t)((const uint16_t *)row)[i] << 16)
                                    : ((const float *)row)[i];
            amax = fmaxf(amax, fabsf(f));
        }
    }
    amax = wave_max_dpp(amax);
    if (lane == 63) red_f[wave] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red_f[0], red_f[1]), fmaxf(red_f[2], red_f[3]));
    const float s = act_scale_q(amax, qmax);

    int sum = 0;
    if (VEC) {
        const uint4 *v = (const uint4 *)row;
        for (int64_t i = tid; i < k / E; i += 256) {
            uint4 d = v[i];
            uint32_t w[4] = {d.x, d.y, d.z, d.w};
            if (DT == DT_BF16) {
                uint32_t out[2] = {0, 0};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    int8_t a = quant1q(bf16_lo(w[e]), s, qmax), b = quant1q(bf16_hi(w[e]), s, qmax);
                    sum += a + b;
                    uint32_t pair = ((uint32_t)(uint8_t)a) | ((uint32_t)(uint8_t)b << 8);
                    out[e >> 1] |= pair << (16 * (e & 1));
                }
                ((uint2 *)qrow)[i] = make_uint2(out[0], out[1]);
            } else {
                uint32_t out = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    int8_t a = quant1q(__uint_as_float(w[e]), s, qmax);
                    sum += a;
                    out |= (uint32_t)(uint8_t)a << (8 * e);
                }
                ((uint32_t *)qrow)[i] = out;
            }
        }
    } else {
        for (int64_t i = tid; i < k; i += 256) {
            float f = DT == DT_BF16 ? __uint_as_float((uint32_t)((const uint16_t *)row)[i] << 16)
                                    : ((const float *)row)[i];
            int8_t a = quant1q(f, s, qmax);
            sum += a;
            qrow[i] = a;
        }
    }
    sum = wave_sum_dpp(sum);
    if (lane == 63) red_i[wave] = sum;
    __syncthreads();
    if (tid == 0) {
        scale[m] = s;
        if (rowsum) rowsum[m] = red_i[0] + red_i[1] + red_i[2] + red_i[3];
    }
}

// Register-resident variant for rows of up to 256 * NV vectors: every load of
// the row is issued before the first use (clamped index, so unconditional),
// the row is read from memory once, and the max and the quantisation both work
// on the registers.  Same arithmetic and outputs as the kernel above.
template <int DT, int NV>
__global__ __launch_bounds__(256) void quant_act_reg_kernel(const void *__restrict__ x, int64_t k,
                                                            int8_t *__restrict__ xq,
                                                            float *__restrict__ scale,
                                                            int32_t *__restrict__ rowsum,
                                                        float qmax)
{
    __shared__ float red_f[4];
    __shared__ int red_i[4];
    constexpr int E = DT == DT_BF16 ? 8 : 4;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t m = blockIdx.x;
    const uint8_t *row = (const uint8_t *)x + m * k * (DT == DT_BF16 ? 2 : 4);
    int8_t *qrow = xq + m * k;
    const int nvec = (int)(k / E);

    uint4 v[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int i = tid + 256 * j;
        v[j] = load16(row + 16 * (int64_t)(i < nvec ? i : nvec - 1));
    }
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        if (tid + 256 * j >= nvec) continue;
        const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (DT == DT_BF16)
                amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(w[e])), fabsf(bf16_hi(w[e]))));
            else
                amax = fmaxf(amax, fabsf(__uint_as_float(w[e])));
        }
    }
    amax = wave_max_dpp(amax);
    if (lane == 63) red_f[wave] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red_f[0], red_f[1]), fmaxf(red_f[2], red_f[3]));
    const float s = act_scale_q(amax, qmax);

    int sum = 0;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int i = tid + 256 * j;
        if (i >= nvec) continue;
        const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
        if (DT == DT_BF16) {
            uint32_t out[2] = {0, 0};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                int8_t a = quant1q(bf16_lo(w[e]), s, qmax), b = quant1q(bf16_hi(w[e]), s, qmax);
                sum += a + b;
                uint32_t pair = ((uint32_t)(uint8_t)a) | ((uint32_t)(uint8_t)b << 8);
                out[e >> 1] |= pair << (16 * (e & 1));
            }
            ((uint2 *)qrow)[i] = make_uint2(out[0], out[1]);
        } else {
            uint32_t out = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                int8_t a = quant1q(__uint_as_float(w[e]), s, qmax);
                sum += a;
                out |= (uint32_t)(uint8_t)a << (8 * e);
            }
            ((uint32_t *)qrow)[i] = out;
        }
    }
    sum = wave_sum_dpp(sum);
    if (lane == 63) red_i[wave] = sum;
    __syncthreads();
    if (tid == 0) {
        scale[m] = s;
        if (rowsum) rowsum[m] = red_i[0] + red_i[1] + red_i[2] + red_i[3];
    }
}

template <int DT>
hipError_t launch_reg(int64_t nvec, const void *x, int64_t m, int64_t k, int8_t *xq, float *scale,
                      int32_t *rowsum, hipStream_t s, float qmax)
{
    const dim3 grid((unsigned)m), block(256);
    const int64_t per = (nvec + 255) / 256;
    if (per <= 1)
        hipLaunchKernelGGL((quant_act_reg_kernel<DT, 1>), grid, block, 0, s, x, k, xq, scale, rowsum, qmax);
    else if (per <= 2)
        hipLaunchKernelGGL((quant_act_reg_kernel<DT, 2>), grid, block, 0, s, x, k, xq, scale, rowsum, qmax);
    else if (per <= 4)
        hipLaunchKernelGGL((quant_act_reg_kernel<DT, 4>), grid, block, 0, s, x, k, xq, scale, rowsum, qmax);
    else if (per <= 8)
        hipLaunchKernelGGL((quant_act_reg_kernel<DT, 8>), grid, block, 0, s, x, k, xq, scale, rowsum, qmax);
    else
        hipLaunchKernelGGL((quant_act_reg_kernel<DT, 16>), grid, block, 0, s, x, k, xq, scale, rowsum, qmax);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_act(const void *x, int dtype, int64_t m, int64_t k, int8_t *xq,
                            float *scale, int32_t *rowsum, hipStream_t s, int qmax_i)
{
    const float qmax = (float)qmax_i;
    dim3 grid((unsigned)m), block(256);
    // rows of up to 256 * 16 vectors (32768 bf16 / 16384 fp32) stay in registers
    if (dtype == DT_BF16 && k % 8 == 0 && k / 8 <= 256 * 16)
        return launch_reg<DT_BF16>(k / 8, x, m, k, xq, scale, rowsum, s, qmax);
    if (dtype == DT_F32 && k % 4 == 0 && k / 4 <= 256 * 16)
        return launch_reg<DT_F32>(k / 4, x, m, k, xq, scale, rowsum, s, qmax);
    if (dtype == DT_BF16) {
        if (k % 8 == 0)
            hipLaunchKernelGGL((quant_act_kernel<DT_BF16, true>), grid, block, 0, s, x, k, xq,
                               scale, rowsum, qmax);
        else
            hipLaunchKernelGGL((quant_act_kernel<DT_BF16, false>), grid, block, 0, s, x, k, xq,
                               scale, rowsum, qmax);
    } else {
        if (k % 4 == 0)
            hipLaunchKernelGGL((quant_act_kernel<DT_F32, true>), grid, block, 0, s, x, k, xq,
                               scale, rowsum, qmax);
        else
            hipLaunchKernelGGL((quant_act_kernel<DT_F32, false>), grid, block, 0, s, x, k, xq,
                               scale, rowsum, qmax);
    }
    return hipGetLastError();
}

}  // namespace bl
