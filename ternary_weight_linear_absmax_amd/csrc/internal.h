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

// ---- one token with the decoder block's glue around the product (gemv.hip) ----
enum : int { NORM_RESIDUAL = 0, NORM_GQA = 1, NORM_F64 = 2 };
constexpr int64_t NORM_MAX_K = 16384;
struct NormArgs {
    int pro;              // NORM_RESIDUAL / NORM_GQA / NORM_F64
    const void *src;      // residual: float [K]; gqa: float row (the QKV output); f64: double [K]
    const float *add;     // residual: float [K] added to src, or nullptr
    float *x_out;         // residual with add: src + add, stored by block 0 (not src)
    int64_t col;          // gqa: first value column
    int64_t group;        // gqa: query heads per key-value head
    int64_t head_dim;     // gqa
    double eps;
    int8_t *xq;           // optional: the quantised token [K]
    float *scale;         // optional: its scale [1]
    int32_t *rowsum;      // optional: its row sum [1]
    int64_t f;            // relu2: gate rows [0, F), up rows [F, 2F) of the packed matrix
    double *v;            // relu2: output [F]
};
bool gemv_norm_supported(int64_t n, int64_t k);
// n: logical rows (2F with relu2)
hipError_t launch_gemv_norm(const NormArgs &a, int64_t n, int64_t k, const uint8_t *packed,
                            Out out, bool relu2, hipStream_t s);

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
// base-3 layout, vector kernels.  ws: gemv3_workspace_bytes(m, n, k) bytes of
// scratch, any contents (the partial sums of the k slices of the one-token
// table kernel).
int64_t gemv3_workspace_bytes(int64_t m, int64_t n, int64_t k);
hipError_t launch_gemv_pack3(const int8_t *xq, const int32_t *rowsum, int64_t m,
                             const uint8_t *packed, int64_t n, int64_t k, Out out, void *ws,
                             hipStream_t s);
// one token, digit table (K a multiple of 16)
bool gemv3lut_supported(int64_t m, int64_t k);
hipError_t launch_gemv3lut(const int8_t *xq, const int32_t *rowsum, const uint8_t *packed,
                           int64_t n, int64_t k, Out out, hipStream_t s);
// one token, partial-sum tables (gemv3sum.hip); 0 slices: not this shape
int gemv3sum_slices(int64_t m, int64_t n, int64_t k);
int64_t gemv3sum_workspace_bytes(int64_t m, int64_t n, int64_t k);
hipError_t launch_gemv3sum(const int8_t *xq, const int32_t *rowsum, const uint8_t *packed,
                           int64_t n, int64_t k, Out out, int32_t *ws, hipStream_t s);
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
// Tiled int8 GEMM.  variant: GEMM_TILED (square-ish block tiles, any K) or
// GEMM_WIDE (64 x 512 block tiles, K a multiple of 16).
enum : int { GEMM_TILED = 0, GEMM_WIDE = 1 };
// The variant AUTO takes for this shape.
int gemm_preferred_variant(int64_t m, int64_t n, int64_t k);
hipError_t launch_gemm_pack2(const int8_t *xq, const int32_t *rowsum, int64_t m,
                             const uint8_t *packed, int64_t n, int64_t k, Out out, void *ws,
                             hipStream_t s, int variant = GEMM_TILED);
int64_t gemm_workspace_bytes(int64_t m, int64_t n, int64_t k, int variant = GEMM_TILED);
// wide-tile kernel (gemm_wide.hip): columns per wave (32-column blocks, 2 or
// 4) and k split for a shape, and one launch (plus the split-k finish when
// finish is set and it splits)
struct GemmWide { int wn, splits, kg; };   // kg: k-groups per block (2: eight waves)
GemmWide gemm_wide_config(int64_t m, int64_t n, int64_t k);
int gemm_wide_splits(int64_t m, int64_t n, int64_t k);
hipError_t launch_gemm_wide_cfg(const int8_t *xq, const int32_t *rowsum, int64_t m,
                                const uint8_t *packed, int64_t n, int64_t k, Out out,
                                GemmWide c, int32_t *ws, hipStream_t s, int64_t ldy, bool finish);
hipError_t launch_gemm_wide(const int8_t *xq, const int32_t *rowsum, int64_t m,
                            const uint8_t *packed, int64_t n, int64_t k, Out out, int splits,
                            int32_t *ws, hipStream_t s, int64_t ldy, bool finish);
// The same product with its k range split and the slices left unsummed:
// ws receives splits int32 [M, N] slices (row stride N), each the slice's sum
// of xq * (t + 1) without the row-sum term.  gemm_partial_splits gives the
// split count, or 0 where the product does not run that way (one split, or
// operands addressed in several blocks); the launch is valid only when it is
// at least 2.
int gemm_partial_splits(int64_t m, int64_t n, int64_t k, int variant);
int64_t gemm_partial_workspace_bytes(int64_t m, int64_t n, int64_t k, int variant);
hipError_t launch_gemm_pack2_partials(const int8_t *xq, const int32_t *rowsum, int64_t m,
                                      const uint8_t *packed, int64_t n, int64_t k, Out out,
                                      int32_t *ws, hipStream_t s, int variant);

// ---- group scales (groups.hip) ----
// y [m, n] holds int32 accumulators (as bits); rescaled in place with the scale
// of each column's group of rows_per_group output features.
hipError_t launch_group_rescale(float *y, const float *scale, const float *beta, int64_t m,
                                int64_t n, int64_t rows_per_group, hipStream_t s);

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
// s = 127 / max|x|, or 1 for an all-zero token; where the division overflows
// (max|x| below about 3.7e-37) s is the largest finite float, so that the
// codes stay defined and gamma / s stays finite.
__device__ inline float act_scale(float amax)
{
    return amax == 0.0f ? 1.0f : fminf(127.0f / amax, __FLT_MAX__);
}
__device__ inline float act_scale_q(float amax, float qmax)
{
    return amax == 0.0f ? 1.0f : fminf(qmax / amax, __FLT_MAX__);
}

constexpr int gcd_int(int a, int b) { return b == 0 ? a : gcd_int(b, a % b); }

// ---- vector-kernel helpers shared by the one-token kernels ----
__device__ inline uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

// Four values quantised with the activation quantiser's arithmetic
// (rint(x s) clamped to +-127, as quant1) and packed into the bytes of one
// word, value a in the lowest byte.
__device__ inline uint32_t quant4(float a, float b, float c, float d, float s)
{
    auto q = [&](float x) __attribute__((always_inline)) {
        return (uint32_t)(int)__builtin_amdgcn_fmed3f(rintf(x * s), -127.0f, 127.0f);
    };
    const uint32_t ab = __builtin_amdgcn_perm(q(b), q(a), 0x0c0c0400u);   // a, b in bytes 0, 1
    const uint32_t cd = __builtin_amdgcn_perm(q(d), q(c), 0x0c0c0400u);
    return __builtin_amdgcn_perm(cd, ab, 0x05040100u);
}

// Nibble form of 16 activation bytes for the 4-bit dot products: x = 16 hi + lo
// with lo = x & 15 (unsigned) and hi = x >> 4 (signed).  Byte j of l02 holds
// lo(x[j]) | lo(x[8 + j]) << 4, of h02 the two hi nibbles, and l13 / h13 the
// same for x[4 + j] and x[12 + j]: the nibble order of a packed word masked
// with 0x33333333 (codes of k = j and 8 + j) or shifted by 2 first (4 + j,
// 12 + j).
__device__ inline uint4 nibble_split(uint4 x)
{
    uint4 r;
    r.x = (x.x & 0x0F0F0F0Fu) | ((x.z & 0x0F0F0F0Fu) << 4);          // l02
    r.y = ((x.x >> 4) & 0x0F0F0F0Fu) | (x.z & 0xF0F0F0F0u);          // h02
    r.z = (x.y & 0x0F0F0F0Fu) | ((x.w & 0x0F0F0F0Fu) << 4);          // l13
    r.w = ((x.y >> 4) & 0x0F0F0F0Fu) | (x.w & 0xF0F0F0F0u);          // h13
    return r;
}

// One packed word (16 trits) against 16 activation bytes in nibble form:
// 4-bit dot products of the codes with the signed high nibbles (ah) and the
// unsigned low nibbles (al); the word's sum is 16 ah + al.  7 ALU operations.
__device__ inline void dot8_word(uint32_t w, uint4 xs, int &ah, uint32_t &al)
{
    const uint32_t c02 = w & 0x33333333u, c13 = (w >> 2) & 0x33333333u;
    ah = __builtin_amdgcn_sdot8((int)c02, (int)xs.y, ah, false);
    ah = __builtin_amdgcn_sdot8((int)c13, (int)xs.w, ah, false);
    al = __builtin_amdgcn_udot8(c02, xs.x, al, false);
    al = __builtin_amdgcn_udot8(c13, xs.z, al, false);
}

// Sum over the 64 lanes of a wave with DPP row operations; lane 63 holds the
// result.
__device__ inline int wave_sum_dpp(int v)
{
    v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
    v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
    v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);  // row_half_mirror
    v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);  // row_mirror
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31
    return v;
}

// Maximum of non-negative floats over the wave, same DPP pattern (disabled
// lanes contribute 0, the identity here); lane 63 holds the result.
template <int CTRL, int ROWS>
__device__ inline float max_dpp_step(float v)
{
    const int t = __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xF, false);
    return fmaxf(v, __int_as_float(t));
}

__device__ inline float wave_max_dpp(float v)
{
    v = max_dpp_step<0xB1, 0xF>(v);    // quad_perm [1,0,3,2]
    v = max_dpp_step<0x4E, 0xF>(v);    // quad_perm [2,3,0,1]
    v = max_dpp_step<0x141, 0xF>(v);   // row_half_mirror
    v = max_dpp_step<0x140, 0xF>(v);   // row_mirror
    v = max_dpp_step<0x142, 0xA>(v);   // row_bcast:15
    v = max_dpp_step<0x143, 0xC>(v);   // row_bcast:31
    return v;
}


// The same patterns on doubles (two 32-bit DPP moves per step; disabled lanes
// contribute 0.0): the sum, and the maximum of non-negative values, over the
// wave, in lane 63.
template <int CTRL, int ROWS>
__device__ inline double dpp_d(double v)
{
    const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, ROWS, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, ROWS, 0xF, false);
    return __hiloint2double(hi, lo);
}

__device__ inline double wave_sum_dpp_d(double v)
{
    v += dpp_d<0xB1, 0xF>(v);
    v += dpp_d<0x4E, 0xF>(v);
    v += dpp_d<0x141, 0xF>(v);
    v += dpp_d<0x140, 0xF>(v);
    v += dpp_d<0x142, 0xA>(v);
    v += dpp_d<0x143, 0xC>(v);
    return v;
}

__device__ inline double wave_max_dpp_d(double v)
{
    v = fmax(v, dpp_d<0xB1, 0xF>(v));
    v = fmax(v, dpp_d<0x4E, 0xF>(v));
    v = fmax(v, dpp_d<0x141, 0xF>(v));
    v = fmax(v, dpp_d<0x140, 0xF>(v));
    v = fmax(v, dpp_d<0x142, 0xA>(v));
    v = fmax(v, dpp_d<0x143, 0xC>(v));
    return v;
}

// RMSNorm's two reductions in one pass: the sum of squares of v and max |v|
// over the block (nw waves; red_ss and red_vm hold one entry per wave).  The
// quantiser's max |h| with h = (float)(v * inv) is then (float)(max|v| * inv)
// exactly, since v -> (float)(|v| * inv) is non-decreasing for inv > 0.
__device__ inline void block_ss_vmax(double &ss, double &vm, double *red_ss, double *red_vm,
                                     int nw)
{
    ss = wave_sum_dpp_d(ss);
    vm = wave_max_dpp_d(vm);
    if ((threadIdx.x & 63) == 63) {
        red_ss[threadIdx.x >> 6] = ss;
        red_vm[threadIdx.x >> 6] = vm;
    }
    __syncthreads();
    ss = 0.0;
    vm = 0.0;
    for (int q = 0; q < nw; ++q) {
        ss += red_ss[q];
        vm = fmax(vm, red_vm[q]);
    }
}

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

// Epilogue: y = acc * gamma / s.  The row factor gamma / s is formed in double
// precision (for float gamma and s it stays far inside the double range, so
// no token, however small its scale, loses precision there) and each output
// is the double product rounded once to float.
__device__ inline double epi_gs(float gamma, float s) { return (double)gamma / (double)s; }
__device__ inline float epi_y(int32_t acc, double gs) { return (float)((double)acc * gs); }

// Writes the output element (m, n) from the code-weighted sum sum_k (t+1) q
// and the token's rowsum: acc = codesum - rowsum.
__device__ inline void store_out(const Out &o, int64_t ldy, int64_t m, int64_t n,
                                 int32_t codesum, int32_t rowsum)
{
    int32_t acc = codesum - rowsum;
    if (o.acc) {
        o.acc[m * ldy + n] = acc;
    } else {
        o.y[m * ldy + n] = epi_y(acc, epi_gs(o.gamma[0], o.scale[m]));
    }
}

}  // namespace bl
