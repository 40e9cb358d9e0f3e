// Internal declarations shared by the HIP translation units of libbitlinear.
// Every launcher returns the hipError_t of its launch; shapes are validated by
// the C-ABI layer before any launcher runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <utility>

namespace bl {

enum : int { DT_F32 = 0, DT_BF16 = 1 };
enum : int { LAYOUT_PACK2 = 0, LAYOUT_PACK3 = 1 };

// Row pitch of the packed layouts (bytes); both are multiples of 16.
__host__ __device__ inline int64_t pack2_pitch(int64_t k) { return ((k + 63) / 64) * 16; }
__host__ __device__ inline int64_t pack3_pitch(int64_t k) { return (((k + 4) / 5 + 15) / 16) * 16; }

// Output of a forward kernel: either the rescaled float y or the raw int32
// accumulator (acc != nullptr selects the raw form).
struct Out {
    const float *scale;   // [M] per-token quantiser multiplier s
    const float *gamma;   // one float, absmean of the weights
    float *y;             // [M, N]
    int32_t *acc;         // [M, N] or nullptr
};

// ---- weights (quant_weights.hip) ----
// Exact absmean scale: gamma = float(round_to_double(sum |w|) / (N*K)).
// The workspace holds gamma_workspace_bytes(N*K) bytes of scratch.
int64_t gamma_workspace_bytes(int64_t count);
hipError_t launch_gamma(const void *w, int dtype, int64_t n, int64_t k, void *workspace,
                        float *gamma, hipStream_t s);
hipError_t launch_pack(const void *w, int dtype, int64_t n, int64_t k, int layout,
                       const float *gamma, uint8_t *packed, hipStream_t s, bool binary = false);
hipError_t launch_unpack(const uint8_t *packed, int layout, int64_t n, int64_t k,
                         int8_t *trits, hipStream_t s);

// ---- activations (quant_act.hip) ----
hipError_t launch_quant_act(const void *x, int dtype, int64_t m, int64_t k, int8_t *xq,
                            float *scale, int32_t *rowsum, hipStream_t s, int qmax = 127);

// ---- decoder-block glue (glue.hip) ----
enum : int { GLUE_RESIDUAL = 0, GLUE_GQA = 1, GLUE_RELU2 = 2 };
constexpr int64_t GLUE_MAX_K = 256 * 32;
struct GlueArgs {
    float *x;             // residual: [M, K] float, updated in place
    const float *add;     // residual: [M, K] float or nullptr
    const float *src;     // gqa / relu2: source rows
    int64_t ld;           // gqa / relu2: source row stride (floats)
    int64_t col;          // gqa: first value column; relu2: offset of "up" from "gate"
    int64_t group;        // gqa: query heads per key-value head
    int64_t head_dim;     // gqa
    // Product output as split-k partial slices instead of floats (add / src
    // unused): y[m, c] = (sum over slices of part[(s * pm + m) * ld + c]
    // - p_rowsum[m]) * (p_gamma[0] / p_scale[m]), the split-k finish's
    // arithmetic; for the residual form ld = K.
    const int32_t *part;
    int splits;
    int64_t pm;
    const int32_t *p_rowsum;
    const float *p_scale;
    const float *p_gamma;
};
hipError_t launch_glue(int mode, const GlueArgs &a, int64_t m, int64_t k, double eps,
                       int8_t *xq, float *scale, int32_t *rowsum, hipStream_t s);

// ---- products ----
// 2-bit layout, vector dot-product kernel; tokens handled in groups of up to 4.
hipError_t launch_gemv_pack2(const int8_t *xq, const int32_t *rowsum, int64_t m,
                             const uint8_t *packed, int64_t n, int64_t k, Out out,
                             hipStream_t s);
// One token (m = 1, k % 16 == 0, k <= 16384): the activation quantiser runs
// inside the 2-bit vector kernel, one launch; x is bf16 or fp32; xq, scale and
// rowsum are written as bitlinear_quantize_act would write them.
bool gemv_fused_supported(int64_t m, int64_t n, int64_t k, int dtype);
hipError_t launch_gemv_pack2_fused(const void *x, int dtype, int8_t *xq, float *scale,
                                   int32_t *rowsum, const uint8_t *packed, int64_t n, int64_t k,
                                   Out out, hipStream_t s);
// base-3 layout, vector kernel.
hipError_t launch_gemv_pack3(const int8_t *xq, const int32_t *rowsum, int64_t m,
                             const uint8_t *packed, int64_t n, int64_t k, Out out,
                             hipStream_t s);
// 2-bit layout, int8 matrix-core kernel.  ws: gemm_workspace_bytes(m, n, k)
// bytes of scratch, any contents (one int32 partial tile per split of k).
bool skinny_supported(int64_t m, int64_t n, int64_t k);
// Skinny path: k splits of the shared-activation kernel (1: unsplit, 0: the
// per-wave kernel instead) and the partial-sum workspace they need.
int skinny_splits(int64_t m, int64_t n, int64_t k);
int64_t skinny_workspace_bytes(int64_t m, int64_t n, int64_t k);
hipError_t launch_skinny_pack2(const int8_t *xq, const int32_t *rowsum, int64_t m,
                               const uint8_t *packed, int64_t n, int64_t k, Out out, void *ws,
                               hipStream_t s);
// Sums `splits` int32 [M, N] slices of ws in split order, then the epilogue.
hipError_t launch_splitk_finish(const int32_t *ws, const int32_t *rowsum, int64_t m, int64_t n,
                                int splits, Out out, int64_t ldy, hipStream_t s);
hipError_t launch_gemm_pack2(const int8_t *xq, const int32_t *rowsum, int64_t m,
                             const uint8_t *packed, int64_t n, int64_t k, Out out, void *ws,
                             hipStream_t s);
int64_t gemm_workspace_bytes(int64_t m, int64_t n, int64_t k);
// The same product with its k range split and the slices left unsummed:
// ws receives splits int32 [M, N] slices (row stride N), each the slice's sum
// of xq * (t + 1) without the row-sum term.  gemm_partial_splits gives the
// split count, or 0 where the product does not run that way (one split, or
// operands addressed in several blocks); the launch is valid only when it is
// at least 2.
int gemm_partial_splits(int64_t m, int64_t n, int64_t k);
int64_t gemm_partial_workspace_bytes(int64_t m, int64_t n, int64_t k);
hipError_t launch_gemm_pack2_partials(const int8_t *xq, const int32_t *rowsum, int64_t m,
                                      const uint8_t *packed, int64_t n, int64_t k, Out out,
                                      int32_t *ws, hipStream_t s);

// ---- backward (backward.hip) ----
// grad_x [m, k] fp32 = gamma * grad_y [m, n] (bf16 / fp32) * t [n, k] (2-bit layout).
hipError_t launch_backward_input(const void *grad_y, int dtype, int64_t m, int64_t n,
                                 const uint8_t *packed, int64_t k, const float *gamma,
                                 float *grad_x, hipStream_t s);

// 128-bit streaming load (the packed weights are read once per call).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ inline uint4 load_nt16(const void *p)
{
    u32x4 v = __builtin_nontemporal_load((const u32x4 *)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Plain 128-bit load through a native vector type (assigning a uint4 struct
// straight from memory can become a memcpy that keeps arrays out of registers).
__device__ inline uint4 load16(const void *p)
{
    const u32x4 v = *(const u32x4 *)p;
    return make_uint4(v.x, v.y, v.z, v.w);
}

// ---- per-token activation quantiser arithmetic, shared by the quantiser and
// the decoder-block glue so that both produce the same bytes ----
__device__ inline int8_t quant1(float x, float s)
{
    float r = rintf(x * s);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (int8_t)(int)r;
}
// The same with a narrower symmetric range [-qmax, qmax] (qmax = 2^(b-1) - 1
// for b-bit activations); qmax = 127 gives quant1.
__device__ inline int8_t quant1q(float x, float s, float qmax)
{
    float r = rintf(x * s);
    r = fminf(fmaxf(r, -qmax), qmax);
    return (int8_t)(int)r;
}
__device__ inline float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ inline float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }
// s = 127 / max|x|, or 1 for an all-zero token.
__device__ inline float act_scale(float amax) { return amax == 0.0f ? 1.0f : 127.0f / amax; }
__device__ inline float act_scale_q(float amax, float qmax) { return amax == 0.0f ? 1.0f : qmax / amax; }

constexpr int gcd_int(int a, int b) { return b == 0 ? a : gcd_int(b, a % b); }

template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>{}), ...);
}
// f(integral_constant<int, 0>) ... f(integral_constant<int, N - 1>), unrolled.
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f)
{
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Writes the output element (m, n) from the code-weighted sum sum_k (t+1) q
// and the token's rowsum: acc = codesum - rowsum.
__device__ inline void store_out(const Out &o, int64_t ldy, int64_t m, int64_t n,
                                 int32_t codesum, int32_t rowsum)
{
    int32_t acc = codesum - rowsum;
    if (o.acc) {
        o.acc[m * ldy + n] = acc;
    } else {
        float gs = o.gamma[0] / o.scale[m];
        o.y[m * ldy + n] = (float)acc * gs;
    }
}

}  // namespace bl
