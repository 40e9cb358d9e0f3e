// Ternary x int8 GEMM on the gfx950 matrix cores (prefill and batched decode).
//
// Source: asi.tokyo BitNet b1.58 2B4T article, packing paragraph (trits packed
// four per byte, unpacked beside the arithmetic units, multiplied with 8-bit
// activations) and its closing remark that today's hardware treats ternary
// weights as int8.  Here the int8 unit is v_mfma_i32_32x32x32_i8: a 32x32
// int32 tile += A[32 x 32 int8] * B[32 x 32 int8] per wave.
//
// Operand layout of v_mfma_i32_32x32x32_i8 (lane l, h = l / 32):
//   A: 16 bytes = A[i = l % 32][k = 16h .. 16h+15]
//   B: 16 bytes = B[k = 16h .. 16h+15][j = l % 32]
//   D: register r = D[i = 8(r/4) + 4h + r%4][j = l % 32]
// One packed 2-bit word holds 16 consecutive k of one weight row, and
// (word >> 2i) & 0x03030303 (i = 0..3) are exactly the four B registers of
// one lane, in k order: the weights go from global memory straight into
// registers, 4x smaller than int8, and are unpacked there with 7 ALU ops per
// MFMA.  The activations (A) are staged through LDS, shared by the two waves
// of a block that cover the same tokens.
//
// The B operand carries the codes t + 1; the epilogue subtracts the token's
// row sum of q (exact integer arithmetic), then rescales by gamma / s.
//
// Block tile: 128 tokens x 128 weight rows, k in steps of 128; four waves in a
// 2 x 2 arrangement, each owning a 64 x 64 output tile (2 x 2 MFMA tiles).
// The k loop is double-buffered: the next stage's global loads are issued
// before the current stage's MFMAs.
#include "internal.h"

namespace bl {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int LDA = BK + 16;            // padded LDS row (bytes)

__device__ inline uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

// Global -> register load of this thread's four 16-byte pieces of the A tile.
template <bool AL>
__device__ inline void load_a(const int8_t *__restrict__ xq, int64_t m, int64_t k, int64_t m0,
                              int64_t k0, uint4 regs[4])
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = threadIdx.x + 256 * i;
        const int row = e >> 3, col = (e & 7) * 16;
        const int64_t gm = m0 + row, gk = k0 + col;
        uint4 v = zero4();
        if (gm < m) {
            const int8_t *p = xq + gm * k + gk;
            if (AL) {
                if (gk < k) v = *(const uint4 *)p;
            } else {
                uint32_t wds[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    uint32_t acc = 0;
#pragma unroll
                    for (int b = 0; b < 4; ++b)
                        if (gk + 4 * q + b < k) acc |= (uint32_t)(uint8_t)p[4 * q + b] << (8 * b);
                    wds[q] = acc;
                }
                v = make_uint4(wds[0], wds[1], wds[2], wds[3]);
            }
        }
        regs[i] = v;
    }
}

__device__ inline void store_a(uint8_t *lds, const uint4 regs[4])
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = threadIdx.x + 256 * i;
        const int row = e >> 3, col = (e & 7) * 16;
        *(uint4 *)(lds + row * LDA + col) = regs[i];
    }
}

// This lane's 16 packed bytes (64 trits) of weight row n for the stage at k0.
__device__ inline uint4 load_b(const uint8_t *__restrict__ packed, int64_t pitch, int64_t n,
                               int64_t nrow, int64_t k0, int h)
{
    const int64_t byte = (k0 / 4) + 16 * h;   // 4 trits per byte
    if (nrow >= n || byte >= pitch) return zero4();
    return load_nt16(packed + nrow * pitch + byte);
}

__device__ inline v4i unpack_word(uint32_t w)
{
    v4i r;
    r[0] = (int)(w & 0x03030303u);
    r[1] = (int)((w >> 2) & 0x03030303u);
    r[2] = (int)((w >> 4) & 0x03030303u);
    r[3] = (int)((w >> 6) & 0x03030303u);
    return r;
}

__device__ inline uint32_t word_of(const uint4 &v, int p)
{
    return p == 0 ? v.x : p == 1 ? v.y : p == 2 ? v.z : v.w;
}

template <bool AL>
__global__ __launch_bounds__(256) void gemm2_kernel(const int8_t *__restrict__ xq,
                                                    const int32_t *__restrict__ rowsum,
                                                    int64_t m, int64_t k,
                                                    const uint8_t *__restrict__ packed, int64_t n,
                                                    int64_t pitch, int tiles_m, Out out)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][BM * LDA];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int h = lane >> 5, l32 = lane & 31;
    const int tm = blockIdx.x % tiles_m, tn = blockIdx.x / tiles_m;
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const int nk = (int)((k + BK - 1) / BK);

    v16i acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][s][r] = 0;

    const int64_t nrow[2] = {n0 + wn * 64 + l32, n0 + wn * 64 + 32 + l32};

    uint4 areg[4];
    uint4 breg[2], bnext[2];
    load_a<AL>(xq, m, k, m0, 0, areg);
    store_a(lds[0], areg);
    breg[0] = load_b(packed, pitch, n, nrow[0], 0, h);
    breg[1] = load_b(packed, pitch, n, nrow[1], 0, h);
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) {
            const int64_t k1 = (int64_t)(kt + 1) * BK;
            load_a<AL>(xq, m, k, m0, k1, areg);
            bnext[0] = load_b(packed, pitch, n, nrow[0], k1, h);
            bnext[1] = load_b(packed, pitch, n, nrow[1], k1, h);
        }
        const uint8_t *la = lds[cur];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            v4i af[2], bf[2];
#pragma unroll
            for (int a = 0; a < 2; ++a) {
                const int row = wm * 64 + 32 * a + l32;
                uint4 v = *(const uint4 *)(la + row * LDA + 64 * h + 16 * p);
                af[a] = v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
            }
#pragma unroll
            for (int s = 0; s < 2; ++s) bf[s] = unpack_word(word_of(breg[s], p));
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int s = 0; s < 2; ++s)
                    acc[a][s] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[a], bf[s], acc[a][s], 0,
                                                                      0, 0);
        }
        if (more) store_a(lds[cur ^ 1], areg);
        __syncthreads();
        if (more) {
            breg[0] = bnext[0];
            breg[1] = bnext[1];
        }
    }

#pragma unroll
    for (int a = 0; a < 2; ++a) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t gm = m0 + wm * 64 + 32 * a + 8 * (r / 4) + 4 * h + (r % 4);
            if (gm >= m) continue;
            const int32_t rs = rowsum[gm];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int64_t gn = nrow[s];
                if (gn < n) store_out(out, n, gm, gn, acc[a][s][r], rs);
            }
        }
    }
}

}  // namespace

hipError_t launch_gemm_pack2(const int8_t *xq, const int32_t *rowsum, int64_t m,
                             const uint8_t *packed, int64_t n, int64_t k, Out out, hipStream_t s)
{
    const int tiles_m = (int)((m + BM - 1) / BM);
    const int64_t tiles_n = (n + BN - 1) / BN;
    const dim3 grid((unsigned)(tiles_m * tiles_n)), block(256);
    const int64_t pitch = pack2_pitch(k);
    if (k % 16 == 0)
        hipLaunchKernelGGL((gemm2_kernel<true>), grid, block, 0, s, xq, rowsum, m, k, packed, n,
                           pitch, tiles_m, out);
    else
        hipLaunchKernelGGL((gemm2_kernel<false>), grid, block, 0, s, xq, rowsum, m, k, packed, n,
                           pitch, tiles_m, out);
    return hipGetLastError();
}

}  // namespace bl
