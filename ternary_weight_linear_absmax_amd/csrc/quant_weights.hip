// Absmean weight quantiser and packers.
//
// Source: "1-bit LLM era: Microsoft introduces BitNet b1.58" (cheatsheet.md),
// section "What is BitNet b1.58?", weight bullet: scale the weights by their
// mean absolute value, round to the nearest integer, restrict to {-1, 0, 1}.
// Packing: the asi.tokyo BitNet b1.58 2B4T article (four trits per byte) and
// the news.hada.io topic 20406 comment on ternary packing (five per byte).
//
// gamma is computed in a fixed order so that it is reproducible bit for bit:
// each row's |w| are summed in double precision with k ascending, then the row
// sums are added in row order, divided by N*K and rounded once to float.
// The trit decision needs no division: round-half-even(|w| / gamma) >= 1
// exactly when 2|w| > gamma, and 2|w| is exact in float.
#include "internal.h"

namespace bl {
namespace {

__device__ inline float load_w(const void *p, int dtype, int64_t i)
{
    if (dtype == DT_BF16) {
        uint32_t u = (uint32_t)((const uint16_t *)p)[i] << 16;
        return __uint_as_float(u);
    }
    return ((const float *)p)[i];
}

// Trit code t+1 of one weight: 2 for +1, 0 for -1, 1 for 0.
__device__ inline uint32_t trit_code(float w, float gamma)
{
    float a2 = 2.0f * fabsf(w);
    if (!(a2 > gamma)) return 1u;
    return w > 0.0f ? 2u : 0u;
}

// Code of one weight under the sign binariser of the original 1-bit BitNet
// (lumen-it.ai article: weights to +1 or -1 with the signum function): -1
// for w < 0, +1 otherwise (zero, of either sign, maps to +1).
__device__ inline uint32_t sign_code(float w) { return w < 0.0f ? 0u : 2u; }

template <bool BIN>
__device__ inline uint32_t weight_code(float w, float gamma)
{
    return BIN ? sign_code(w) : trit_code(w, gamma);
}

// ---- row sums of |w| in double, k ascending -------------------------------
// A block owns 64 rows.  The tile [64 rows x 128 k] is staged through LDS with
// coalesced loads; then lane r of the first wave adds row r's 128 values in
// order, carrying its running sum from tile to tile.
constexpr int GR_ROWS = 64;
constexpr int GR_TK = 128;

__global__ __launch_bounds__(256) void gamma_rows_kernel(const void *__restrict__ w, int dtype,
                                                         int64_t n, int64_t k,
                                                         double *__restrict__ rowsums)
{
    __shared__ float tile[GR_ROWS][GR_TK + 1];
    const int tid = threadIdx.x;
    const int64_t row0 = (int64_t)blockIdx.x * GR_ROWS;
    double run = 0.0;
    for (int64_t k0 = 0; k0 < k; k0 += GR_TK) {
        const int kc = (int)((k - k0) < GR_TK ? (k - k0) : GR_TK);
        for (int e = tid; e < GR_ROWS * GR_TK; e += 256) {
            int r = e / GR_TK, c = e % GR_TK;
            int64_t row = row0 + r;
            float v = 0.0f;
            if (row < n && c < kc) v = fabsf(load_w(w, dtype, row * k + k0 + c));
            tile[r][c] = v;
        }
        __syncthreads();
        if (tid < GR_ROWS) {
            for (int c = 0; c < kc; ++c) run += (double)tile[tid][c];
        }
        __syncthreads();
    }
    if (tid < GR_ROWS && row0 + tid < n) rowsums[row0 + tid] = run;
}

// One thread adds the row sums in row order and forms gamma.
__global__ void gamma_final_kernel(const double *__restrict__ rowsums, int64_t n, int64_t k,
                                   float *__restrict__ gamma)
{
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    double total = 0.0;
    for (int64_t i = 0; i < n; ++i) total += rowsums[i];
    gamma[0] = (float)(total / ((double)n * (double)k));
}

// ---- 2-bit packing: one thread per 32-bit word (16 trits) ----------------------
// Word g of row r holds k = 16g + 4i + j at byte j, bits 2i..2i+1.
template <bool BIN>
__global__ __launch_bounds__(256) void pack2_kernel(const void *__restrict__ w, int dtype,
                                                    int64_t n, int64_t k,
                                                    const float *__restrict__ gamma_p,
                                                    uint32_t *__restrict__ packed)
{
    const int64_t words_per_row = pack2_pitch(k) / 4;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= n * words_per_row) return;
    const int64_t row = idx / words_per_row, g = idx % words_per_row;
    const float gamma = gamma_p[0];
    const int64_t base = row * k + 16 * g;
    uint32_t word = 0;
    for (int i = 0; i < 4; ++i) {
        for (int j = 0; j < 4; ++j) {
            int64_t kk = 16 * g + 4 * i + j;
            uint32_t code = 1u;
            if (kk < k) code = weight_code<BIN>(load_w(w, dtype, base + 4 * i + j), gamma);
            word |= code << (8 * j + 2 * i);
        }
    }
    packed[idx] = word;
}

// ---- base-3 packing: one thread per 32-bit word (4 bytes, 20 trits) ---------------
template <bool BIN>
__global__ __launch_bounds__(256) void pack3_kernel(const void *__restrict__ w, int dtype,
                                                    int64_t n, int64_t k,
                                                    const float *__restrict__ gamma_p,
                                                    uint32_t *__restrict__ packed)
{
    const int64_t words_per_row = pack3_pitch(k) / 4;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= n * words_per_row) return;
    const int64_t row = idx / words_per_row, g = idx % words_per_row;
    const float gamma = gamma_p[0];
    uint32_t word = 0;
    for (int b = 0; b < 4; ++b) {
        const int64_t byte_idx = 4 * g + b;
        uint32_t value = 0, weight = 1;
        for (int i = 0; i < 5; ++i) {
            int64_t kk = 5 * byte_idx + i;
            uint32_t code = 1u;
            if (kk < k) code = weight_code<BIN>(load_w(w, dtype, row * k + kk), gamma);
            value += code * weight;
            weight *= 3u;
        }
        word |= value << (8 * b);
    }
    packed[idx] = word;
}

// ---- decoders (parity and debugging) ------------------------------------------
__global__ __launch_bounds__(256) void unpack2_kernel(const uint32_t *__restrict__ packed,
                                                      int64_t n, int64_t k,
                                                      int8_t *__restrict__ trits)
{
    const int64_t words_per_row = pack2_pitch(k) / 4;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= n * words_per_row) return;
    const int64_t row = idx / words_per_row, g = idx % words_per_row;
    const uint32_t word = packed[idx];
    for (int i = 0; i < 4; ++i)
        for (int j = 0; j < 4; ++j) {
            int64_t kk = 16 * g + 4 * i + j;
            if (kk < k) trits[row * k + kk] = (int8_t)((int)((word >> (8 * j + 2 * i)) & 3u) - 1);
        }
}

__global__ __launch_bounds__(256) void unpack3_kernel(const uint8_t *__restrict__ packed,
                                                      int64_t n, int64_t k,
                                                      int8_t *__restrict__ trits)
{
    const int64_t pitch = pack3_pitch(k);
    const int64_t nbytes = (k + 4) / 5;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= n * nbytes) return;
    const int64_t row = idx / nbytes, b = idx % nbytes;
    uint32_t v = packed[row * pitch + b];
    for (int i = 0; i < 5; ++i) {
        int64_t kk = 5 * b + i;
        if (kk < k) trits[row * k + kk] = (int8_t)((int)(v % 3u) - 1);
        v /= 3u;
    }
}

inline unsigned blocks_for(int64_t items, int threads)
{
    return (unsigned)((items + threads - 1) / threads);
}

}  // namespace

hipError_t launch_gamma_rows(const void *w, int dtype, int64_t n, int64_t k, double *rowsums,
                             hipStream_t s)
{
    hipLaunchKernelGGL(gamma_rows_kernel, dim3(blocks_for(n, GR_ROWS)), dim3(256), 0, s, w,
                       dtype, n, k, rowsums);
    return hipGetLastError();
}

hipError_t launch_gamma_final(const double *rowsums, int64_t n, int64_t k, float *gamma,
                              hipStream_t s)
{
    hipLaunchKernelGGL(gamma_final_kernel, dim3(1), dim3(64), 0, s, rowsums, n, k, gamma);
    return hipGetLastError();
}

hipError_t launch_pack(const void *w, int dtype, int64_t n, int64_t k, int layout,
                       const float *gamma, uint8_t *packed, hipStream_t s, bool binary)
{
    if (layout == LAYOUT_PACK2) {
        int64_t words = n * (pack2_pitch(k) / 4);
        if (binary)
            hipLaunchKernelGGL(pack2_kernel<true>, dim3(blocks_for(words, 256)), dim3(256), 0, s,
                               w, dtype, n, k, gamma, (uint32_t *)packed);
        else
            hipLaunchKernelGGL(pack2_kernel<false>, dim3(blocks_for(words, 256)), dim3(256), 0, s,
                               w, dtype, n, k, gamma, (uint32_t *)packed);
    } else {
        int64_t words = n * (pack3_pitch(k) / 4);
        if (binary)
            hipLaunchKernelGGL(pack3_kernel<true>, dim3(blocks_for(words, 256)), dim3(256), 0, s,
                               w, dtype, n, k, gamma, (uint32_t *)packed);
        else
            hipLaunchKernelGGL(pack3_kernel<false>, dim3(blocks_for(words, 256)), dim3(256), 0, s,
                               w, dtype, n, k, gamma, (uint32_t *)packed);
    }
    return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t *packed, int layout, int64_t n, int64_t k, int8_t *trits,
                         hipStream_t s)
{
    if (layout == LAYOUT_PACK2) {
        int64_t words = n * (pack2_pitch(k) / 4);
        hipLaunchKernelGGL(unpack2_kernel, dim3(blocks_for(words, 256)), dim3(256), 0, s,
                           (const uint32_t *)packed, n, k, trits);
    } else {
        int64_t bytes = n * ((k + 4) / 5);
        hipLaunchKernelGGL(unpack3_kernel, dim3(blocks_for(bytes, 256)), dim3(256), 0, s, packed,
                           n, k, trits);
    }
    return hipGetLastError();
}

}  // namespace bl
