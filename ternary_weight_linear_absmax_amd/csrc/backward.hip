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
// The gradient stays a float (no quantisation of it is implied by the
// sources): every product g * t is exact and the sums are accumulated in fp32.
// A plain fp32-FMA version of the same tiling measured 2.7-3x slower.

#include "internal.h"

namespace bl {
namespace {

// ---- matrix-core kernel -----------------------------------------------------------
// The product on v_mfma_f32_32x32x16_bf16: each fp32 gradient is split
// into three bf16 parts hi + mid + lo (a bf16 gradient is its own hi part,
// so it needs one product instead of three; round to nearest at each step; the
// parts carry 8 significant bits each, so for normal values their sum is the
// gradient exactly), the trits are exact in bf16, and the matrix cores
// accumulate the three products in fp32.  Block tile 64 (m) x 128 (k), four
// waves of 32 x 64; per stage of 32 n the block writes the three gradient
// parts [m][n] and the raw packed bytes into LDS, unpacks the trits into a
// [k][n] bf16 tile (n contiguous: one 16-byte operand per lane), then runs
// 2 (n steps) x 2 (k tiles) x 3 (parts) MFMAs per wave; the next stage's
// global data is loaded during the MFMAs.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM2 = 64, BK2 = 128, BN2 = 32;
constexpr int LDAB = BN2 * 2 + 16;   // bytes per LDS row of 32 bf16 (+16 pad)
constexpr int TRS = BN2 + 4;         // words per LDS row of raw packed words [word][n]

__device__ inline uint32_t bf16_pair(__bf16 a, __bf16 b)
{
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

template <int DT, bool VEC, int G>
__global__ __launch_bounds__(256 * G) void backward_mfma_kernel(const void *__restrict__ grad_y,
                                                            int64_t m, int64_t n,
                                                            const uint8_t *__restrict__ packed,
                                                            int64_t pitch, int64_t k,
                                                            const float *__restrict__ gamma_p,
                                                            float *__restrict__ grad_x)
{
    // G groups of four waves share the block's tile; group g takes the
    // n stages g, g + G, ... with its own LDS buffers, and the groups' sums
    // are added at the end (G = 2 for matrices with few tiles: half the
    // serial chain of stages per block)
    __shared__ __attribute__((aligned(16))) uint8_t as_all[G][2][3][BM2 * LDAB];
    __shared__ __attribute__((aligned(16))) uint8_t bs_all[G][2][BK2 * LDAB];
    __shared__ __attribute__((aligned(16))) uint32_t traw_all[G][BK2 / 16][TRS];
    // bf16 gradients are their own first part (the other two are zero), so
    // one product per fragment gives the same sums
    constexpr int NPART = DT == DT_BF16 ? 1 : 3;
    const int grp = (int)(threadIdx.x >> 8);
    auto &as = as_all[grp];
    auto &bs = bs_all[grp];
    auto &traw = traw_all[grp];
    const int tid = threadIdx.x & 255, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wk = wave >> 1;
    const int h = lane >> 5, l32 = lane & 31;
    const int64_t m0 = (int64_t)blockIdx.y * BM2, k0 = (int64_t)blockIdx.x * BK2;
    const int nst_all = (int)((n + BN2 - 1) / BN2);
    const int nst = (nst_all + G - 1) / G;   // iterations; stage of iteration j: G j + grp
    const int64_t words = pitch / 4;

    // staging roles: gradient row m0 + tid / 4, columns 8 (tid % 4) .. +7;
    // raw packed word tid % 8 of row tid / 8 (threads 0..255: 32 rows x 8 words)
    const int gr = tid >> 2, gc = 8 * (tid & 3);
    const int64_t gm = m0 + gr;
    const int tr = tid >> 3, tw = tid & 7;
    const int64_t wkk = k0 / 16 + tw;
    float gv[8];
    uint32_t tv = 0;

    auto load = [&](int it) __attribute__((always_inline)) {
        const int64_t nb = (int64_t)(G * it + grp) * BN2;   // past N: zeros
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
        tv = (tn < n && wkk < words) ? ((const uint32_t *)(packed + tn * pitch))[wkk] : 0x55555555u;
    };
    // three bf16 parts of the 8 gradient values, and the raw packed word
    auto store = [&](int buf) __attribute__((always_inline)) {
        uint32_t part[3][4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float a = gv[2 * e], b = gv[2 * e + 1];
            const __bf16 ah = (__bf16)a, bh = (__bf16)b;
            const float ar = a - (float)ah, br = b - (float)bh;
            const __bf16 am = (__bf16)ar, bm = (__bf16)br;
            const __bf16 al = (__bf16)(ar - (float)am), bl2 = (__bf16)(br - (float)bm);
            part[0][e] = bf16_pair(ah, bh);
            part[1][e] = bf16_pair(am, bm);
            part[2][e] = bf16_pair(al, bl2);
        }
#pragma unroll
        for (int q = 0; q < NPART; ++q)
            *(uint4 *)(&as[buf][q][gr * LDAB + 2 * gc]) =
                make_uint4(part[q][0], part[q][1], part[q][2], part[q][3]);
        traw[tw][tr] = tv;
    };
    // trits of the stage into bs[buf][k][n]: thread -> n octet tid % 4 and k
    // pair tid / 4; the octet's eight raw words come in two 16-byte LDS reads
    // ([word][n] layout), and each pair of codes (n even, n odd) becomes a
    // pair of bf16 trits with one byte permute: code c selects the bytes of
    // -1 (0xBF80), 0 or +1 (0x3F80) from a table held in two constants
    auto unpack = [&](int buf) __attribute__((always_inline)) {
        const int o = tid & 3, kp = tid >> 2;
        const int g = kp >> 3, q = (2 * kp) & 15;   // word, first k within it (even)
        // k q of a word sits at bits 8 (q % 4) + 2 (q / 4); k q + 1 one byte up
        const int sh = 8 * (q & 3) + 2 * (q >> 2);
        const uint4 wa = *(const uint4 *)&traw[g][8 * o];
        const uint4 wb = *(const uint4 *)&traw[g][8 * o + 4];
        const uint32_t w[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
        uint32_t v0[4], v1[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            // selector bytes (c0 + 4, c0, c1 + 4, c1): low byte then high byte
            // of each bf16, table bytes 0..3 = BF 00 3F 00, 4..7 = 80 00 80 00
            const uint32_t x0 = ((w[2 * e] >> sh) & 3u) | (((w[2 * e + 1] >> sh) & 3u) << 16);
            const uint32_t x1 =
                ((w[2 * e] >> (sh + 8)) & 3u) | (((w[2 * e + 1] >> (sh + 8)) & 3u) << 16);
            v0[e] = __builtin_amdgcn_perm(0x00800080u, 0x003F00BFu, x0 * 0x101u + 0x00040004u);
            v1[e] = __builtin_amdgcn_perm(0x00800080u, 0x003F00BFu, x1 * 0x101u + 0x00040004u);
        }
        *(uint4 *)(&bs[buf][(2 * kp) * LDAB + 16 * o]) = make_uint4(v0[0], v0[1], v0[2], v0[3]);
        *(uint4 *)(&bs[buf][(2 * kp + 1) * LDAB + 16 * o]) = make_uint4(v1[0], v1[1], v1[2], v1[3]);
    };

    f32x16 acc[2];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;

    load(0);
    store(0);
    __syncthreads();
    unpack(0);
    __syncthreads();
    for (int st = 0; st < nst; ++st) {
        const int buf = st & 1;
        if (st + 1 < nst) load(st + 1);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            bf16x8 b[2];
#pragma unroll
            for (int c = 0; c < 2; ++c)
                b[c] = *(const bf16x8 *)(&bs[buf][(64 * wk + 32 * c + l32) * LDAB + 32 * s + 16 * h]);
#pragma unroll
            for (int q = 0; q < NPART; ++q) {
                const bf16x8 a =
                    *(const bf16x8 *)(&as[buf][q][(32 * wm + l32) * LDAB + 32 * s + 16 * h]);
#pragma unroll
                for (int c = 0; c < 2; ++c)
                    acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b[c], acc[c], 0, 0, 0);
            }
        }
        if (st + 1 < nst) {
            store(buf ^ 1);
            __syncthreads();
            unpack(buf ^ 1);
        }
        __syncthreads();
    }

    if constexpr (G == 2) {
        // group 1's sums into LDS (free after the loop's last barrier), then
        // group 0 adds them: a fixed order, group 0 + group 1
        float *tile = (float *)&as_all[0][0][0][0];   // [64][128 + 4]
        static_assert(64 * 132 * 4 <= (int)sizeof(as_all), "tile fits");
        if (grp == 1)
#pragma unroll
            for (int r = 0; r < 16; ++r)
#pragma unroll
                for (int c = 0; c < 2; ++c)
                    tile[(32 * wm + 8 * (r / 4) + 4 * h + (r % 4)) * 132 + 64 * wk + 32 * c + l32] =
                        acc[c][r];
        __syncthreads();
        if (grp == 1) return;
#pragma unroll
        for (int r = 0; r < 16; ++r)
#pragma unroll
            for (int c = 0; c < 2; ++c)
                acc[c][r] += tile[(32 * wm + 8 * (r / 4) + 4 * h + (r % 4)) * 132 + 64 * wk + 32 * c + l32];
    }
    // lane (l32, h), register r: row 8 (r / 4) + 4 h + r % 4 of the wave's 32
    // m rows, column l32 of k tile c
    const float gamma = gamma_p[0];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + 32 * wm + 8 * (r / 4) + 4 * h + (r % 4);
        if (row >= m) continue;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int64_t col = k0 + 64 * wk + 32 * c + l32;
            if (col < k) grad_x[row * k + col] = gamma * acc[c][r];
        }
    }
}

}  // namespace

namespace {
template <int G>
void launch_g(const void *grad_y, int dtype, bool vec, int64_t m, int64_t n, const uint8_t *packed,
              int64_t pitch, int64_t k, const float *gamma, float *grad_x, hipStream_t s)
{
    const dim3 grid((unsigned)((k + BK2 - 1) / BK2), (unsigned)((m + BM2 - 1) / BM2));
    const dim3 block(256 * G);
    if (dtype == DT_BF16) {
        if (vec)
            hipLaunchKernelGGL((backward_mfma_kernel<DT_BF16, true, G>), grid, block, 0, s, grad_y, m,
                               n, packed, pitch, k, gamma, grad_x);
        else
            hipLaunchKernelGGL((backward_mfma_kernel<DT_BF16, false, G>), grid, block, 0, s, grad_y,
                               m, n, packed, pitch, k, gamma, grad_x);
    } else {
        if (vec)
            hipLaunchKernelGGL((backward_mfma_kernel<DT_F32, true, G>), grid, block, 0, s, grad_y, m,
                               n, packed, pitch, k, gamma, grad_x);
        else
            hipLaunchKernelGGL((backward_mfma_kernel<DT_F32, false, G>), grid, block, 0, s, grad_y, m,
                               n, packed, pitch, k, gamma, grad_x);
    }
}
}  // namespace

hipError_t launch_backward_input(const void *grad_y, int dtype, int64_t m, int64_t n,
                                 const uint8_t *packed, int64_t k, const float *gamma,
                                 float *grad_x, hipStream_t s)
{
    const int64_t pitch = pack2_pitch(k);
    // 16-byte loads need every grad_y row 16-byte aligned
    const bool vec = dtype == DT_BF16 ? n % 8 == 0 : n % 4 == 0;
    // two wave groups per block when the tiles do not fill the CUs
    const int64_t tiles = ((k + BK2 - 1) / BK2) * ((m + BM2 - 1) / BM2);
    if (tiles < 256 && n >= 2 * BN2)
        launch_g<2>(grad_y, dtype, vec, m, n, packed, pitch, k, gamma, grad_x, s);
    else
        launch_g<1>(grad_y, dtype, vec, m, n, packed, pitch, k, gamma, grad_x, s);
    return hipGetLastError();
}

}  // namespace bl
