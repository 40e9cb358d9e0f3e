// Decoder-block glue around the BitLinear layers of the 2B-class layer stack:
// the input of every BitLinear is RMSNorm'ed and then quantised per token.
//
// Sources: asi.tokyo BitNet b1.58 2B4T article, stabiliser paragraph (a norm
// in front of the sub-layers, squared ReLU in the feed-forward block);
// cheatsheet.md summary of BitNet b1.58, "What is BitNet b1.58?" (RMSNorm, no
// bias; activations scaled per token).
//
// One 256-thread block per token row.  The BitLinear output it reads is either
// stored floats or, after a GEMM that split its k range, the int32 partial
// slices, which the block sums and scales itself (the split-k finish's
// arithmetic) in place of a separate finishing launch.  The row's pre-norm
// values are formed in registers (double precision), in one of three ways:
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

__device__ inline int block_sum_i(int v, int *red)
{
    v = wave_sum_dpp(v);
    if ((threadIdx.x & 63) == 63) red[threadIdx.x >> 6] = v;
    __syncthreads();
    return (red[0] + red[1]) + (red[2] + red[3]);
}

// Source columns of element i of the row: c0 (residual: the added product
// column; gqa: the value column; relu2: gate) and c1 (relu2: up).
template <int MODE>
__device__ inline void glue_cols(const GlueArgs &a, int i, int64_t &c0, int64_t &c1)
{
    if (MODE == GLUE_GQA) {
        const unsigned hd = (unsigned)a.head_dim, head = (unsigned)i / hd;
        const unsigned d = (unsigned)i - head * hd;
        c0 = a.col + (int64_t)(head / (unsigned)a.group) * hd + d;
    } else {
        c0 = i;
    }
    c1 = a.col + i;
}

// PART: the product's output arrives as split-k partial slices and is
// finished here (GlueArgs::part), so that the product needs no finish launch.
template <int MODE, int EPT, bool PART>
__global__ __launch_bounds__(256) void glue_kernel(GlueArgs a, int64_t k, double eps,
                                                   int8_t *__restrict__ xq,
                                                   float *__restrict__ scale,
                                                   int32_t *__restrict__ rowsum)
{
    __shared__ double red_d[4], red_vm[4];
    __shared__ int red_i[4];
    const int tid = threadIdx.x;
    const int64_t m = blockIdx.x;
    const int kk = (int)k;

    // All of the thread's loads first (indices clamped into the row, values
    // past K unused), so that they are in flight together.  The product's
    // row sum and scale are read before any write: the outputs may be the
    // same buffers (this block's row only).
    float f0[EPT], f1[EPT];
    if constexpr (PART) {
        // U slices' loads in flight at once (64 registers of loaded values);
        // slices past the last are loaded as slice s0 and masked out of the
        // sum, so that no load or wait sits behind a branch.  Column offsets
        // fit 32 bits: the GEMM leaves its slices unsummed only for products
        // it addresses in one block, whose N * pitch is below 2^31.
        constexpr int NSRC = MODE == GLUE_RELU2 ? 2 : 1;
        constexpr int U0 = 64 / (EPT * NSRC);
        constexpr int U = U0 < 1 ? 1 : U0 > 4 ? 4 : U0;
        const int32_t prs = a.p_rowsum[m];
        const double gs = epi_gs(a.p_gamma[0], a.p_scale[m]);
        const int32_t *row = a.part + m * a.ld;
        const int64_t slice = a.pm * a.ld;
        int col[NSRC][EPT];
        int32_t acc[NSRC][EPT];
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
            const int i = tid + 256 * j, ic = i < kk ? i : kk - 1;
            int64_t c0, c1;
            glue_cols<MODE>(a, ic, c0, c1);
            col[0][j] = (int)c0;
            if (NSRC == 2) col[NSRC - 1][j] = (int)c1;
#pragma unroll
            for (int q = 0; q < NSRC; ++q) acc[q][j] = 0;
            if (MODE == GLUE_RESIDUAL) f0[j] = a.x[m * k + ic];
        }
        for (int s0 = 0; s0 < a.splits; s0 += U) {
            int32_t t[U][NSRC][EPT];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t sp = s0 + u < a.splits ? s0 + u : s0;
                const int32_t *p = row + sp * slice;
#pragma unroll
                for (int q = 0; q < NSRC; ++q)
#pragma unroll
                    for (int j = 0; j < EPT; ++j) t[u][q][j] = p[col[q][j]];
            }
            __builtin_amdgcn_sched_barrier(0);   // every load issued before the first add
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int32_t keep = s0 + u < a.splits ? -1 : 0;   // no branch
#pragma unroll
                for (int q = 0; q < NSRC; ++q)
#pragma unroll
                    for (int j = 0; j < EPT; ++j) acc[q][j] += t[u][q][j] & keep;
            }
        }
        {
            // y rounded to float on its own, as the stored product output
            // is: the multiply must not fuse with the residual addition
#pragma clang fp contract(off)
#pragma unroll
            for (int j = 0; j < EPT; ++j) {
                const float y0 = epi_y(acc[0][j] - prs, gs);
                if (MODE == GLUE_RESIDUAL) f1[j] = y0;
                else f0[j] = y0;
                if (NSRC == 2) f1[j] = epi_y(acc[NSRC - 1][j] - prs, gs);
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
            const int i = tid + 256 * j;
            const int ic = i < kk ? i : kk - 1;
            int64_t c0, c1;
            glue_cols<MODE>(a, ic, c0, c1);
            if (MODE == GLUE_RESIDUAL) {
                f0[j] = a.x[m * k + ic];
                f1[j] = a.add ? a.add[m * k + ic] : 0.0f;
            } else if (MODE == GLUE_GQA) {
                f0[j] = a.src[m * a.ld + c0];
            } else {
                f0[j] = a.src[m * a.ld + c0];     // gate
                f1[j] = a.src[m * a.ld + c1];     // up
            }
        }
    }
    const bool has_add = PART || a.add;

    double v[EPT];
    double ss = 0.0, vm = 0.0;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int i = tid + 256 * j;
        if (MODE == GLUE_RESIDUAL) {
            const float xv = has_add ? f0[j] + f1[j] : f0[j];
            if (has_add && i < kk) a.x[m * k + i] = xv;
            v[j] = (double)xv;
        } else if (MODE == GLUE_GQA) {
            v[j] = (double)f0[j];
        } else {
            const double gd = f0[j] > 0.0f ? (double)f0[j] : 0.0;
            v[j] = gd * gd * (double)f1[j];
        }
        if (i >= kk) v[j] = 0.0;
        ss += v[j] * v[j];
        vm = fmax(vm, fabs(v[j]));
    }
    block_ss_vmax(ss, vm, red_d, red_vm, 4);
    const double inv = 1.0 / sqrt(ss / (double)k + eps);

    float h[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) h[j] = (float)(v[j] * inv);
    // max |h| from max |v| (see block_ss_vmax); an all-zero row gives 0
    const float amax = vm > 0.0 ? (float)(vm * inv) : 0.0f;
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

template <int MODE, bool PART>
hipError_t launch_mode(const GlueArgs &a, int64_t m, int64_t k, double eps, int8_t *xq,
                       float *scale, int32_t *rowsum, hipStream_t s)
{
    const dim3 grid((unsigned)m), block(256);
    const int64_t per = (k + 255) / 256;
#define GLUE_CASE(E_)                                                                           \
    if (per <= E_) {                                                                            \
        hipLaunchKernelGGL((glue_kernel<MODE, E_, PART>), grid, block, 0, s, a, k, eps, xq,     \
                           scale, rowsum);                                                      \
        return hipGetLastError();                                                               \
    }
    GLUE_CASE(4) GLUE_CASE(8) GLUE_CASE(12) GLUE_CASE(16) GLUE_CASE(28) GLUE_CASE(32)
#undef GLUE_CASE
    return hipErrorInvalidValue;
}

template <int MODE>
hipError_t launch_mode(const GlueArgs &a, int64_t m, int64_t k, double eps, int8_t *xq,
                       float *scale, int32_t *rowsum, hipStream_t s)
{
    if (a.part) return launch_mode<MODE, true>(a, m, k, eps, xq, scale, rowsum, s);
    return launch_mode<MODE, false>(a, m, k, eps, xq, scale, rowsum, s);
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
