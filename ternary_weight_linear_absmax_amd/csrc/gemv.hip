// Ternary GEMV kernels for small token counts (decode): y[m, n] for M <= 4 per
// pass, streaming the packed weights from HBM once.
//
// Source: asi.tokyo BitNet b1.58 2B4T article, packing paragraph: the trits
// travel packed (four per byte) and are unpacked right next to the arithmetic
// units, where they are multiplied with the 8-bit activations.  On gfx950 the
// "arithmetic unit" is v_dot4_i32_i8: the 2-bit layout is chosen so that
// (word >> 2i) & 0x03030303 gives four consecutive k as int8 codes t + 1, which
// dot4 multiplies with four consecutive int8 activations in one instruction.
// The codes are offset by one, so sum_k (t+1) q = acc + rowsum(q); the row sum
// from the activation quantiser is subtracted once per output.
//
// Two masks avoid two of the four shifts: word & 0x0C0C0C0C is 4x the codes of
// the second quarter, whose dot products are collected in a separate
// accumulator and divided by 4 (exactly) at the end.
//
// Work split: lanes run along k in groups of LG lanes (one packed row per
// group); each lane loads 16 bytes (64 trits) per step with a 128-bit load and
// the matching 64 activation bytes per token; a lane group owns R consecutive
// rows, so every activation load is reused R times.  Partial sums are reduced
// across the LG lanes with xor shuffles.
#include "internal.h"

namespace bl {
namespace {

__device__ inline uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

// 64 activation bytes k = 64c .. 64c+63 of one token, zero past K.
template <bool AL>
__device__ inline void load_x64(const int8_t *__restrict__ xrow, int64_t k, int64_t c, uint4 xv[4])
{
    const int64_t k0 = 64 * c;
    if (AL) {
#pragma unroll
        for (int d = 0; d < 4; ++d)
            xv[d] = (k0 + 16 * d < k) ? *(const uint4 *)(xrow + k0 + 16 * d) : zero4();
    } else {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            uint32_t e[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint32_t v = 0;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    int64_t kk = k0 + 16 * d + 4 * q + b;
                    if (kk < k) v |= (uint32_t)(uint8_t)xrow[kk] << (8 * b);
                }
                e[q] = v;
            }
            xv[d] = make_uint4(e[0], e[1], e[2], e[3]);
        }
    }
}

// One packed word (16 trits) against the 16 matching activation bytes.
__device__ inline void dot_word(uint32_t w, uint4 x, int &lo, int &hi)
{
    const int u0 = (int)(w & 0x03030303u);
    const int u1 = (int)(w & 0x0C0C0C0Cu);
    const uint32_t w4 = w >> 4;
    const int u2 = (int)(w4 & 0x03030303u);
    const int u3 = (int)(w4 & 0x0C0C0C0Cu);
    lo = __builtin_amdgcn_sdot4(u0, (int)x.x, lo, false);
    hi = __builtin_amdgcn_sdot4(u1, (int)x.y, hi, false);
    lo = __builtin_amdgcn_sdot4(u2, (int)x.z, lo, false);
    hi = __builtin_amdgcn_sdot4(u3, (int)x.w, hi, false);
}

template <int LG>
__device__ inline int group_sum(int v)
{
#pragma unroll
    for (int off = LG / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

template <int MT, int LG, int R, bool AL>
__global__ __launch_bounds__(256) void gemv2_kernel(const int8_t *__restrict__ xq,
                                                    const int32_t *__restrict__ rowsum,
                                                    int64_t k, const uint4 *__restrict__ packed,
                                                    int64_t n, int64_t chunks, Out out,
                                                    int64_t ldy, int64_t m0)
{
    constexpr int RPW = 64 / LG;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int grp = lane / LG, li = lane % LG;
    const int64_t row0 = (((int64_t)blockIdx.x * 4 + wave) * RPW + grp) * R;
    if (row0 >= n) return;

    int lo[R][MT], hi[R][MT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t) lo[r][t] = hi[r][t] = 0;

    for (int64_t c = li; c < chunks; c += LG) {
        uint4 w[R];
#pragma unroll
        for (int r = 0; r < R; ++r)
            w[r] = (row0 + r < n) ? load_nt16(packed + (row0 + r) * chunks + c)
                                  : zero4();
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            uint4 xv[4];
            load_x64<AL>(xq + (m0 + t) * k, k, c, xv);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                dot_word(w[r].x, xv[0], lo[r][t], hi[r][t]);
                dot_word(w[r].y, xv[1], lo[r][t], hi[r][t]);
                dot_word(w[r].z, xv[2], lo[r][t], hi[r][t]);
                dot_word(w[r].w, xv[3], lo[r][t], hi[r][t]);
            }
        }
    }

#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            int v = lo[r][t] + (hi[r][t] >> 2);
            v = group_sum<LG>(v);
            if (li == 0 && row0 + r < n) store_out(out, ldy, m0 + t, row0 + r, v, rowsum[m0 + t]);
        }
}

// ---- base-3 layout --------------------------------------------------------------
// A lane takes 16 packed bytes (80 trits) per step; each byte is split into
// its five base-3 digits (the codes t + 1) with the exact identity
// floor(b / 3) = (b * 171) >> 9 for 0 <= b < 256.

__device__ inline int x_byte(const uint32_t *xw, int idx)
{
    return (int)(int8_t)(uint8_t)(xw[idx >> 2] >> (8 * (idx & 3)));
}

template <int MT, bool AL>
__global__ __launch_bounds__(256) void gemv3_kernel(const int8_t *__restrict__ xq,
                                                    const int32_t *__restrict__ rowsum,
                                                    int64_t k, const uint4 *__restrict__ packed,
                                                    int64_t n, int64_t chunks, Out out,
                                                    int64_t ldy, int64_t m0)
{
    constexpr int LG = 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t row = (int64_t)blockIdx.x * 4 + wave;
    if (row >= n) return;
    int acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = 0;

    for (int64_t c = lane; c < chunks; c += LG) {
        const uint4 wv = load_nt16(packed + row * chunks + c);
        const uint32_t wb[4] = {wv.x, wv.y, wv.z, wv.w};
        const int64_t k0 = 80 * c;
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            uint32_t xw[20];
            const int8_t *xrow = xq + (m0 + t) * k;
            if (AL && k0 + 80 <= k) {
#pragma unroll
                for (int d = 0; d < 5; ++d) {
                    uint4 v = *(const uint4 *)(xrow + k0 + 16 * d);
                    xw[4 * d] = v.x; xw[4 * d + 1] = v.y; xw[4 * d + 2] = v.z; xw[4 * d + 3] = v.w;
                }
            } else {
#pragma unroll
                for (int q = 0; q < 20; ++q) {
                    uint32_t v = 0;
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        int64_t kk = k0 + 4 * q + b;
                        if (kk < k) v |= (uint32_t)(uint8_t)xrow[kk] << (8 * b);
                    }
                    xw[q] = v;
                }
            }
            int a = acc[t];
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                uint32_t b = (wb[j >> 2] >> (8 * (j & 3))) & 0xFFu;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    uint32_t q3 = (b * 171u) >> 9;
                    int digit = (int)(b - 3u * q3);
                    a += digit * x_byte(xw, 5 * j + i);
                    b = q3;
                }
                a += (int)b * x_byte(xw, 5 * j + 4);
            }
            acc[t] = a;
        }
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        int v = group_sum<64>(acc[t]);
        if (lane == 0) store_out(out, ldy, m0 + t, row, v, rowsum[m0 + t]);
    }
}

// Lanes per row: the largest group whose last step wastes at most 1/8 of the
// row's 16-byte chunks (all lanes of a group step together).
int pick_lanes(int64_t chunks)
{
    const int cands[4] = {64, 32, 16, 8};
    for (int i = 0; i < 4; ++i) {
        int lg = cands[i];
        int64_t waste = ((chunks + lg - 1) / lg) * lg - chunks;
        if (waste * 8 <= chunks) return lg;
    }
    return 8;
}

template <int MT, int LG, int R>
hipError_t launch2(bool al, const int8_t *xq, const int32_t *rowsum, int64_t n, int64_t k,
                   const uint8_t *packed, Out out, int64_t m0, hipStream_t s)
{
    const int64_t chunks = pack2_pitch(k) / 16;
    const int64_t tasks = (n + R - 1) / R;
    const int64_t waves = (tasks + (64 / LG) - 1) / (64 / LG);
    const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
    if (al)
        hipLaunchKernelGGL((gemv2_kernel<MT, LG, R, true>), grid, block, 0, s, xq, rowsum, k,
                           (const uint4 *)packed, n, chunks, out, n, m0);
    else
        hipLaunchKernelGGL((gemv2_kernel<MT, LG, R, false>), grid, block, 0, s, xq, rowsum, k,
                           (const uint4 *)packed, n, chunks, out, n, m0);
    return hipGetLastError();
}

template <int MT, int R>
hipError_t launch2_lg(int lg, bool al, const int8_t *xq, const int32_t *rowsum, int64_t n,
                      int64_t k, const uint8_t *packed, Out out, int64_t m0, hipStream_t s)
{
    switch (lg) {
    case 64: return launch2<MT, 64, R>(al, xq, rowsum, n, k, packed, out, m0, s);
    case 32: return launch2<MT, 32, R>(al, xq, rowsum, n, k, packed, out, m0, s);
    case 16: return launch2<MT, 16, R>(al, xq, rowsum, n, k, packed, out, m0, s);
    default: return launch2<MT, 8, R>(al, xq, rowsum, n, k, packed, out, m0, s);
    }
}

template <int MT>
hipError_t launch3(bool al, const int8_t *xq, const int32_t *rowsum, int64_t n, int64_t k,
                   const uint8_t *packed, Out out, int64_t m0, hipStream_t s)
{
    const int64_t chunks = pack3_pitch(k) / 16;
    const dim3 grid((unsigned)((n + 3) / 4)), block(256);
    if (al)
        hipLaunchKernelGGL((gemv3_kernel<MT, true>), grid, block, 0, s, xq, rowsum, k,
                           (const uint4 *)packed, n, chunks, out, n, m0);
    else
        hipLaunchKernelGGL((gemv3_kernel<MT, false>), grid, block, 0, s, xq, rowsum, k,
                           (const uint4 *)packed, n, chunks, out, n, m0);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_pack2(const int8_t *xq, const int32_t *rowsum, int64_t m,
                             const uint8_t *packed, int64_t n, int64_t k, Out out, hipStream_t s)
{
    const bool al = (k % 16) == 0;
    const int lg = pick_lanes(pack2_pitch(k) / 16);
    for (int64_t m0 = 0; m0 < m; m0 += 4) {
        const int64_t mt = (m - m0) < 4 ? (m - m0) : 4;
        hipError_t e;
        switch (mt) {
        case 1: e = launch2_lg<1, 4>(lg, al, xq, rowsum, n, k, packed, out, m0, s); break;
        case 2: e = launch2_lg<2, 4>(lg, al, xq, rowsum, n, k, packed, out, m0, s); break;
        case 3: e = launch2_lg<3, 2>(lg, al, xq, rowsum, n, k, packed, out, m0, s); break;
        default: e = launch2_lg<4, 2>(lg, al, xq, rowsum, n, k, packed, out, m0, s); break;
        }
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_gemv_pack3(const int8_t *xq, const int32_t *rowsum, int64_t m,
                             const uint8_t *packed, int64_t n, int64_t k, Out out, hipStream_t s)
{
    const bool al = (k % 16) == 0;
    for (int64_t m0 = 0; m0 < m; m0 += 4) {
        const int64_t mt = (m - m0) < 4 ? (m - m0) : 4;
        hipError_t e;
        switch (mt) {
        case 1: e = launch3<1>(al, xq, rowsum, n, k, packed, out, m0, s); break;
        case 2: e = launch3<2>(al, xq, rowsum, n, k, packed, out, m0, s); break;
        case 3: e = launch3<3>(al, xq, rowsum, n, k, packed, out, m0, s); break;
        default: e = launch3<4>(al, xq, rowsum, n, k, packed, out, m0, s); break;
        }
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace bl
