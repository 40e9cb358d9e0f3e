// Ternary x int8 product for a few tokens (up to 16): weight-streaming kernel
// on the 16x16x64 int8 matrix cores.
//
// Source: asi.tokyo BitNet b1.58 2B4T article, packing paragraph (trits packed
// four per byte, unpacked beside the arithmetic units, multiplied with 8-bit
// activations).  With a handful of tokens the product is bound by streaming
// the packed weights from HBM, so every packed byte is read exactly once and
// the matrix core only replaces the dot-product ALU work of the vector kernel.
//
// v_mfma_i32_16x16x64_i8: D[16 x 16] += A[16 x 64] * B[64 x 16], per wave.
// Lane l (r = l % 16, b = l / 16) supplies 16 bytes of row r of A and 16 bytes
// of column r of B, both for k-block b; D lane l holds D[4b + q][r], q = 0..3.
// Which physical k a k-block stands for is free, as long as A and B agree.
// Here A = weight rows (16 per MFMA), B = tokens (the 16 token slots).
//
// k mapping: a wave walks K in chunks of 256.  In chunk c, lane (r, b) loads
// the 16 packed bytes 64c + 16b .. +15 of its weight row (the four k-block
// lanes of a row read 64 contiguous bytes) and the 64 bytes of activations
// 256c + 64b .. +63 of its token.  Step u = 0..3 of the chunk multiplies packed
// word u of the 16 bytes (k = 256c + 64b + 16u .. +15, codes unpacked with
// (w >> 2i) & 0x03030303) with activation bytes 16u .. 16u+15: the same 16 k.
//
// The B operand carries codes t + 1; the epilogue subtracts the token's row
// sum, then rescales by gamma / s.
//
// Block: KS waves on the same 16 RB weight rows, splitting the chunks
// round-robin; each wave keeps RB accumulators (RB row blocks share one
// activation fragment) and prefetches the next chunk while computing the
// current one.  The waves' partial sums meet in LDS at the end.
#include "internal.h"

namespace bl {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int SK_CHUNK = 256;   // k per chunk
constexpr int SK_MAX_KS = 8;

__device__ inline v4i unpack_word16(uint32_t w)
{
    v4i r;
    r[0] = (int)(w & 0x03030303u);
    r[1] = (int)((w >> 2) & 0x03030303u);
    r[2] = (int)((w >> 4) & 0x03030303u);
    r[3] = (int)((w >> 6) & 0x03030303u);
    return r;
}

__device__ inline uint32_t word_at(const uint4 &v, int u)
{
    return u == 0 ? v.x : u == 1 ? v.y : u == 2 ? v.z : v.w;
}

template <int RB>
struct SkinnyLoads {
    uint4 w[RB];      // 16 packed bytes per row block
    uint4 x[4];       // 64 activation bytes
};

template <int RB, int KS>
__global__ __launch_bounds__(64 * KS) void skinny_kernel(const int8_t *__restrict__ xq,
                                                         const int32_t *__restrict__ rowsum,
                                                         int64_t m, int64_t k,
                                                         const uint8_t *__restrict__ packed,
                                                         int64_t n, int64_t pitch, Out out,
                                                         int64_t ldy)
{
    __shared__ v4i red[KS][RB][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, b = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * 16 * RB;
    const int nchunks = (int)(k / SK_CHUNK);

    // Per-lane base addresses (rows and tokens clamped into the matrices:
    // clamped lanes only feed outputs that are never stored).
    const uint8_t *wrow[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        int64_t row = n0 + 16 * rb + r;
        row = row < n ? row : n - 1;
        wrow[rb] = packed + row * pitch + 16 * b;
    }
    const int64_t tok = r < m ? r : m - 1;
    const int8_t *xrow = xq + tok * k + 64 * b;

    auto load = [&](SkinnyLoads<RB> &L, int c) __attribute__((always_inline)) {
        const int cc = c < nchunks ? c : nchunks - 1;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) L.w[rb] = load_nt16(wrow[rb] + (int64_t)cc * 64);
#pragma unroll
        for (int q = 0; q < 4; ++q) L.x[q] = load16(xrow + (int64_t)cc * SK_CHUNK + 16 * q);
    };

    v4i acc[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) acc[rb] = v4i{0, 0, 0, 0};

    // Epilogue operands of this lane's token, loaded now (their latency
    // overlaps the weight stream).
    const int32_t e_rs = rowsum[tok];
    const float e_g = out.acc ? 0.0f : out.gamma[0] / out.scale[tok];

    auto compute = [&](const SkinnyLoads<RB> &L) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const v4i xb = v4i{(int)L.x[u].x, (int)L.x[u].y, (int)L.x[u].z, (int)L.x[u].w};
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                acc[rb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(unpack_word16(word_at(L.w[rb], u)),
                                                                xb, acc[rb], 0, 0, 0);
        }
    };

    // Chunks wave, wave + KS, ...: one chunk of loads in flight ahead of the
    // compute.  Loads are unconditional (clamped chunk index), so the waits
    // are exact; a step past the end computes nothing.
    const int steps = (nchunks - wave + KS - 1) / KS;
    SkinnyLoads<RB> cur, nxt;
    load(cur, wave);
    for (int s = 0; s < steps; ++s) {
        load(nxt, wave + KS * (s + 1));
        __builtin_amdgcn_sched_barrier(0);
        compute(cur);
        __builtin_amdgcn_sched_barrier(0);
        cur = nxt;
    }

    // Combine the waves' partial sums, then the epilogue on wave 0: lane
    // (r, b) holds rows n0 + 16 rb + 4b + q of token r.
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) red[wave][rb][lane] = acc[rb];
    __syncthreads();
    if (wave != 0 || r >= m) return;
    const int32_t rs = e_rs;
    const float g = e_g;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        v4i t = red[0][rb][lane];
#pragma unroll
        for (int w = 1; w < KS; ++w) t += red[w][rb][lane];
        const int64_t row0 = n0 + 16 * rb + 4 * b;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (row0 + q >= n) break;
            const int32_t v = t[q] - rs;
            if (out.acc)
                out.acc[r * ldy + row0 + q] = v;
            else
                out.y[r * ldy + row0 + q] = (float)v * g;
        }
    }
}

template <int RB, int KS>
hipError_t launch_rb_ks(const int8_t *xq, const int32_t *rowsum, int64_t m,
                        const uint8_t *packed, int64_t n, int64_t k, Out out, hipStream_t s)
{
    const int64_t blocks = (n + 16 * RB - 1) / (16 * RB);
    hipLaunchKernelGGL((skinny_kernel<RB, KS>), dim3((unsigned)blocks), dim3(64 * KS), 0, s, xq,
                       rowsum, m, k, packed, n, pack2_pitch(k), out, (int64_t)n);
    return hipGetLastError();
}

}  // namespace

bool skinny_supported(int64_t m, int64_t n, int64_t k)
{
    return m >= 1 && m <= 16 && k % SK_CHUNK == 0 && n >= 1 && n <= ((int64_t)1 << 31) / 64;
}

// Rows per wave (16 RB) and waves per block (KS): keep about 2048 waves in
// flight, with RB as large as that allows (RB row blocks share one activation
// fragment).
hipError_t launch_skinny_pack2(const int8_t *xq, const int32_t *rowsum, int64_t m,
                               const uint8_t *packed, int64_t n, int64_t k, Out out,
                               hipStream_t s)
{
    const int64_t chunks = k / SK_CHUNK;
    const int64_t target = 2048;
    int rb = 4;
    while (rb > 1 && ((n + 16 * rb - 1) / (16 * rb)) * (chunks < SK_MAX_KS ? chunks : SK_MAX_KS) < target)
        rb /= 2;
    const int64_t blocks = (n + 16 * rb - 1) / (16 * rb);
    int64_t ks = (target + blocks - 1) / blocks;
    if (ks > chunks) ks = chunks;
    const int ksel = ks <= 1 ? 1 : ks <= 2 ? 2 : ks <= 4 ? 4 : 8;
#define SK_CASE(RB_, KS_) \
    if (rb == RB_ && ksel == KS_) return launch_rb_ks<RB_, KS_>(xq, rowsum, m, packed, n, k, out, s);
    SK_CASE(4, 1) SK_CASE(4, 2) SK_CASE(4, 4) SK_CASE(4, 8)
    SK_CASE(2, 1) SK_CASE(2, 2) SK_CASE(2, 4) SK_CASE(2, 8)
    SK_CASE(1, 1) SK_CASE(1, 2) SK_CASE(1, 4) SK_CASE(1, 8)
#undef SK_CASE
    return hipErrorInvalidValue;
}

}  // namespace bl
