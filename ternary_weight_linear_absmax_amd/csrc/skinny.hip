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
constexpr int64_t SK_MAX_M = 64;   // four groups of 16 token slots
#ifndef SKINNY_CH
#define SKINNY_CH 1                   // chunks per step (2 and 4 measured slower)
#endif

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

template <int RB, int TG, int CH>
struct SkinnyLoads {
    uint4 w[CH][RB];      // 16 packed bytes per chunk and row block
    uint4 x[CH][TG][4];   // 64 activation bytes per chunk and token group
};

// TG groups of 16 token slots (M <= 16 TG); every unpacked weight operand
// feeds TG MFMAs.
template <int RB, int KS, int TG, int CH>
__global__ __launch_bounds__(64 * KS) void skinny_kernel(const int8_t *__restrict__ xq,
                                                         const int32_t *__restrict__ rowsum,
                                                         int64_t m, int64_t k,
                                                         const uint8_t *__restrict__ packed,
                                                         int64_t n, int64_t pitch, Out out,
                                                         int64_t ldy)
{
    static_assert(KS * RB * TG <= 64, "partial sums must fit in 64 KB of LDS");
    __shared__ v4i red[KS][RB * TG][64];
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
    const int8_t *xrow[TG];
    int32_t e_rs[TG];
    float e_g[TG];
#pragma unroll
    for (int g = 0; g < TG; ++g) {
        const int64_t tok = 16 * g + r < m ? 16 * g + r : m - 1;
        xrow[g] = xq + tok * k + 64 * b;
        // epilogue operands of this lane's tokens, loaded before the stream
        e_rs[g] = rowsum[tok];
        e_g[g] = out.acc ? 0.0f : out.gamma[0] / out.scale[tok];
    }

    // Step c covers chunks CH c .. CH c + CH - 1, so the four k-block lanes of
    // a row read 64 CH contiguous packed bytes per step.  Chunks past the end
    // load a clamped (valid) address and get zero activations.
    const int ngroups = (nchunks + CH - 1) / CH;
    auto load = [&](SkinnyLoads<RB, TG, CH> &L, int c) __attribute__((always_inline)) {
        const int cg = c < ngroups ? c : ngroups - 1;
#pragma unroll
        for (int h = 0; h < CH; ++h) {
            const int ch = CH * cg + h;
            const int cc = ch < nchunks ? ch : nchunks - 1;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) L.w[h][rb] = load_nt16(wrow[rb] + (int64_t)cc * 64);
#pragma unroll
            for (int g = 0; g < TG; ++g)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint4 v = load16(xrow[g] + (int64_t)cc * SK_CHUNK + 16 * q);
                    L.x[h][g][q] = ch < nchunks ? v : make_uint4(0u, 0u, 0u, 0u);
                }
        }
    };

    v4i acc[RB][TG];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int g = 0; g < TG; ++g) acc[rb][g] = v4i{0, 0, 0, 0};

    auto compute = [&](const SkinnyLoads<RB, TG, CH> &L) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < CH; ++h)
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    const v4i a = unpack_word16(word_at(L.w[h][rb], u));
#pragma unroll
                    for (int g = 0; g < TG; ++g) {
                        const uint4 &xv = L.x[h][g][u];
                        const v4i xb = v4i{(int)xv.x, (int)xv.y, (int)xv.z, (int)xv.w};
                        acc[rb][g] =
                            __builtin_amdgcn_mfma_i32_16x16x64_i8(a, xb, acc[rb][g], 0, 0, 0);
                    }
                }
    };

    // Steps wave, wave + KS, ...: one step of loads in flight ahead of the
    // compute.  Loads are unconditional (clamped step index), so the waits
    // are exact; a step past the end computes nothing.
    const int steps = (ngroups - wave + KS - 1) / KS;
    SkinnyLoads<RB, TG, CH> cur, nxt;
    load(cur, wave);
    for (int s = 0; s < steps; ++s) {
        load(nxt, wave + KS * (s + 1));
        __builtin_amdgcn_sched_barrier(0);
        compute(cur);
        __builtin_amdgcn_sched_barrier(0);
        cur = nxt;
    }

    // Combine the waves' partial sums, then the epilogue on wave 0: lane
    // (r, b) holds rows n0 + 16 rb + 4b + q of tokens 16 g + r.
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int g = 0; g < TG; ++g) red[wave][rb * TG + g][lane] = acc[rb][g];
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int g = 0; g < TG; ++g) {
        const int64_t tok = 16 * g + r;
        if (tok >= m) continue;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            v4i t = red[0][rb * TG + g][lane];
#pragma unroll
            for (int w = 1; w < KS; ++w) t += red[w][rb * TG + g][lane];
            const int64_t row0 = n0 + 16 * rb + 4 * b;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (row0 + q >= n) break;
                const int32_t v = t[q] - e_rs[g];
                if (out.acc)
                    out.acc[tok * ldy + row0 + q] = v;
                else
                    out.y[tok * ldy + row0 + q] = (float)v * e_g[g];
            }
        }
    }
}

template <int RB, int KS, int TG>
hipError_t launch_rb_ks(const int8_t *xq, const int32_t *rowsum, int64_t m,
                        const uint8_t *packed, int64_t n, int64_t k, Out out, hipStream_t s)
{
    const int64_t blocks = (n + 16 * RB - 1) / (16 * RB);
    hipLaunchKernelGGL((skinny_kernel<RB, KS, TG, SKINNY_CH>), dim3((unsigned)blocks),
                       dim3(64 * KS), 0, s, xq, rowsum, m, k, packed, n, pack2_pitch(k), out,
                       (int64_t)n);
    return hipGetLastError();
}

template <int TG>
hipError_t launch_tg(const int8_t *xq, const int32_t *rowsum, int64_t m, const uint8_t *packed,
                     int64_t n, int64_t k, Out out, hipStream_t s)
{
    // Rows per wave (16 RB) and waves per block (KS): keep about 2048 waves
    // in flight, with RB as large as that allows (RB row blocks share one
    // activation fragment), and the partial sums within 64 KB of LDS.
    const int64_t chunks = (k / SK_CHUNK + SKINNY_CH - 1) / SKINNY_CH;   // steps along K
    const int64_t target = 2048;
    const int rb_max = TG >= 4 ? 2 : 4;
    int rb = rb_max;
    while (rb > 1 &&
           ((n + 16 * rb - 1) / (16 * rb)) * (chunks < SK_MAX_KS ? chunks : SK_MAX_KS) < target)
        rb /= 2;
    const int64_t blocks = (n + 16 * rb - 1) / (16 * rb);
    int64_t ks = (target + blocks - 1) / blocks;
    if (ks > chunks) ks = chunks;
    const int ksel = ks <= 1 ? 1 : ks <= 2 ? 2 : ks <= 4 ? 4 : 8;
#define SK_CASE(RB_, KS_)                                                                      \
    if (rb == RB_ && ksel == KS_)                                                              \
        return launch_rb_ks<RB_, KS_, TG>(xq, rowsum, m, packed, n, k, out, s);
    if constexpr (TG <= 2) { SK_CASE(4, 1) SK_CASE(4, 2) SK_CASE(4, 4) SK_CASE(4, 8) }
    SK_CASE(2, 1) SK_CASE(2, 2) SK_CASE(2, 4) SK_CASE(2, 8)
    SK_CASE(1, 1) SK_CASE(1, 2) SK_CASE(1, 4) SK_CASE(1, 8)
#undef SK_CASE
    return hipErrorInvalidValue;
}

}  // namespace

bool skinny_supported(int64_t m, int64_t n, int64_t k)
{
    return m >= 1 && m <= SK_MAX_M && k % SK_CHUNK == 0 && n >= 1 && n <= ((int64_t)1 << 31) / 64;
}


// ---- shared-activation variant ------------------------------------------------
// Block: 4 waves on BN = 64 RB weight rows and all M (<= 16 TG) tokens, over
// all k stages of 256; used when the row blocks alone fill the CUs.  Per
// stage the block copies the
// activations [16 TG tokens][256 bytes] into an LDS ring with contiguous
// 16-byte loads (each wave instruction reads whole token rows); each wave
// streams the packed bytes of its RB row blocks of 16 rows straight from HBM
// into registers, several stages ahead, and reads every token's activation
// fragments from LDS.  Same k mapping as above: lane (r, b), word u of its 16
// packed bytes <-> activation bytes 64 b + 16 u .. +15 of the stage.
// gridDim.y > 1 splits the stages over blocks: each split stores its raw code
// sums into its own slice of a partial buffer, which a finish kernel adds in
// split order (device-scope atomics with a last-block finish instead measured
// several times slower: the atomics dominate).
namespace {

constexpr int SK2_LDA = 256 + 16;   // LDS row of one token's stage (bytes)
constexpr int SK2_NS = 3;           // LDS ring
constexpr int SK2_DA = 2;   // activation stages in flight ahead (registers; deeper: slower)
constexpr int SK2_PW = 4;   // weight stages in flight ahead (registers; deeper: slower)

template <int TG, int RB>
__global__ __launch_bounds__(256) void skinny2_kernel(const int8_t *__restrict__ xq,
                                                      const int32_t *__restrict__ rowsum,
                                                      int64_t m, int64_t k,
                                                      const uint8_t *__restrict__ packed,
                                                      int64_t n, int64_t pitch, Out out,
                                                      int64_t ldy, int32_t *__restrict__ part)
{
    constexpr int MT = 16 * TG, BN = 64 * RB;
    constexpr int SLOT = MT * SK2_LDA;
    __shared__ __attribute__((aligned(16))) uint8_t lds[SK2_NS * SLOT];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, b = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * BN;
    // split y of gridDim.y takes stages [s0, s1) of the k range (>= 1 each)
    const int ns_all = (int)(k / SK_CHUNK);
    const int s0 = (int)((int64_t)blockIdx.y * ns_all / gridDim.y);
    const int s1 = (int)((int64_t)(blockIdx.y + 1) * ns_all / gridDim.y);
    const int ns = s1 - s0;

    // activation pieces of this thread: piece p = tid + 256 i of the stage,
    // token p / 16, bytes 16 (p % 16) .. +15 (tokens past M clamped: they
    // only feed outputs that are never stored)
    const int8_t *asrc[TG];
    uint32_t adst[TG];
#pragma unroll
    for (int i = 0; i < TG; ++i) {
        const int p = tid + 256 * i;
        int64_t tok = p >> 4;
        tok = tok < m ? tok : m - 1;
        asrc[i] = xq + tok * k + (int64_t)s0 * SK_CHUNK + 16 * (p & 15);
        adst[i] = (uint32_t)((p >> 4) * SK2_LDA + 16 * (p & 15));
    }
    // weight rows of this lane (clamped into the matrix)
    const uint8_t *wsrc[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        int64_t row = n0 + 16 * (wave * RB + rb) + r;
        row = row < n ? row : n - 1;
        wsrc[rb] = packed + row * pitch + (int64_t)s0 * (SK_CHUNK / 4) + 16 * b;
    }

    auto aload = [&](uint4 (&a)[TG], int st) __attribute__((always_inline)) {
        const int sc = st < ns ? st : ns - 1;
        const int64_t k0 = (int64_t)sc * SK_CHUNK;
#pragma unroll
        for (int i = 0; i < TG; ++i) a[i] = load16(asrc[i] + k0);
    };
    auto astore = [&](const uint4 (&a)[TG], int st) __attribute__((always_inline)) {
        uint8_t *slot = lds + (st % SK2_NS) * SLOT;
#pragma unroll
        for (int i = 0; i < TG; ++i) *(uint4 *)(slot + adst[i]) = a[i];
    };
    auto wload = [&](uint4 (&w)[RB], int st) __attribute__((always_inline)) {
        const int sc = st < ns ? st : ns - 1;
        const int64_t off = (int64_t)sc * (SK_CHUNK / 4);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) w[rb] = load_nt16(wsrc[rb] + off);
    };

    v4i acc[RB][TG];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int g = 0; g < TG; ++g) acc[rb][g] = v4i{0, 0, 0, 0};

    // prologue: stage 0 into LDS; activations of stages 1 .. DA and weights
    // of stages 0 .. PW-1 in flight
    uint4 ra[SK2_DA][TG], rw[SK2_PW][RB];
    {
        uint4 a0[TG];
        aload(a0, 0);
#pragma unroll
        for (int d = 0; d < SK2_DA; ++d) aload(ra[d], 1 + d);
#pragma unroll
        for (int q = 0; q < SK2_PW; ++q) wload(rw[q], q);
        astore(a0, 0);
    }
    __syncthreads();

    // Iteration j: store the activations of stage j+1 (loaded DA iterations
    // ago) into slot (j+1) % 3, issue the loads of stage j+1+DA (activations)
    // and j+PW (weights), then the MFMAs of stage j from slot j % 3; one
    // barrier.  Slot (j+1) % 3 was last read in iteration j-2.
    constexpr int UR = SK2_DA * SK2_PW / gcd_int(SK2_DA, SK2_PW);
    constexpr int U = UR * SK2_NS / gcd_int(UR, SK2_NS);
    auto iter = [&](auto jc, int j) __attribute__((always_inline)) {
        constexpr int J = decltype(jc)::value;
        constexpr int AS = J % SK2_DA, WS = J % SK2_PW;
        if (j + 1 < ns) astore(ra[AS], j + 1);
        aload(ra[AS], j + 1 + SK2_DA);
        uint4 wcur[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) wcur[rb] = rw[WS][rb];
        wload(rw[WS], j + SK2_PW);
        __builtin_amdgcn_sched_barrier(0);
        const uint8_t *slot = lds + (J % SK2_NS) * SLOT;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            v4i xb[TG];
#pragma unroll
            for (int g = 0; g < TG; ++g) {
                const uint4 v = load16(slot + (16 * g + r) * SK2_LDA + 64 * b + 16 * u);
                xb[g] = v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
            }
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const v4i a = unpack_word16(word_at(wcur[rb], u));
#pragma unroll
                for (int g = 0; g < TG; ++g)
                    acc[rb][g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, xb[g], acc[rb][g], 0, 0, 0);
            }
        }
        __syncthreads();
    };
    const int nu = ns - ns % U;
    for (int j = 0; j < nu; j += U)
        static_for<U>([&](auto jc) __attribute__((always_inline)) { iter(jc, j + jc); });
    static_for<U - 1>([&](auto jc) __attribute__((always_inline)) {
        if (nu + jc < ns) iter(jc, nu + jc);
    });

    // Epilogue: lane (r, b) holds rows 16 (wave RB + rb) + 4 b + q of token
    // 16 g + r.  The block's [MT tokens][BN rows] tile is transposed through
    // LDS (the ring is free after the last barrier) so that every thread then
    // writes four consecutive rows of one token: stores are contiguous along
    // the output rows.  Split k range: the raw code sums go to this split's
    // slice of the partial buffer, the finish kernel adds the slices in order.
    static_assert(MT * (BN + 4) * 4 <= SK2_NS * SLOT, "epilogue tile fits the ring");
    int32_t *tile = (int32_t *)lds;   // [MT][BN + 4]
#pragma unroll
    for (int g = 0; g < TG; ++g)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
            *(v4i *)(tile + (16 * g + r) * (BN + 4) + 16 * (wave * RB + rb) + 4 * b) = acc[rb][g];
    __syncthreads();
    // 16-byte stores where rows of four stay 16-byte aligned (the partial
    // buffer always is)
    const uintptr_t base = part ? 0 : out.acc ? (uintptr_t)out.acc : (uintptr_t)out.y;
    const bool vec = (n % 4) == 0 && (part || ((ldy % 4) == 0 && (base & 15) == 0));
    for (int e = tid; e < MT * (BN / 4); e += 256) {
        const int tok = e / (BN / 4), c4 = 4 * (e % (BN / 4));
        if (tok >= m) continue;
        const int64_t row = n0 + c4;
        if (row >= n) continue;
        const v4i v = *(const v4i *)(tile + tok * (BN + 4) + c4);
        if (part) {
            int32_t *dst = part + ((int64_t)blockIdx.y * m + tok) * n + row;
            if (vec && row + 3 < n) {
                *(v4i *)dst = v;
            } else {
                for (int j = 0; j < 4 && row + j < n; ++j) dst[j] = v[j];
            }
            continue;
        }
        const int32_t rs = rowsum[tok];
        if (out.acc) {
            int32_t *dst = out.acc + tok * ldy + row;
            const v4i a = v - rs;
            if (vec && row + 3 < n) *(v4i *)dst = a;
            else
                for (int j = 0; j < 4 && row + j < n; ++j) dst[j] = a[j];
        } else {
            const float gs = out.gamma[0] / out.scale[tok];
            float *dst = out.y + tok * ldy + row;
            float4 f;
            f.x = (float)(v[0] - rs) * gs;
            f.y = (float)(v[1] - rs) * gs;
            f.z = (float)(v[2] - rs) * gs;
            f.w = (float)(v[3] - rs) * gs;
            if (vec && row + 3 < n) *(float4 *)dst = f;
            else {
                const float fa[4] = {f.x, f.y, f.z, f.w};
                for (int j = 0; j < 4 && row + j < n; ++j) dst[j] = fa[j];
            }
        }
    }
}

}  // namespace

namespace {

template <int TG>
hipError_t launch_sk2(const int8_t *xq, const int32_t *rowsum, int64_t m, const uint8_t *packed,
                      int64_t n, int64_t k, Out out, int splits, int32_t *part, hipStream_t s)
{
    hipLaunchKernelGGL((skinny2_kernel<TG, 1>), dim3((unsigned)((n + 63) / 64), (unsigned)splits),
                       dim3(256), 0, s, xq, rowsum, m, k, packed, n, pack2_pitch(k), out,
                       (int64_t)n, splits > 1 ? part : (int32_t *)nullptr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits == 1) return e;
    return launch_splitk_finish(part, rowsum, m, n, splits, out, n, s);
}

}  // namespace

int skinny_splits(int64_t m, int64_t n, int64_t k)
{
    if (m > 16 || k % SK_CHUNK != 0) return 0;   // 0: the per-wave kernel
    // Measured on the 2B- and 70B-class shapes at M = 16: with >= 192 blocks of
    // 64 rows the unsplit kernel is fastest; with 96..191 blocks and long rows
    // (>= 32 stages of 256 k) splitting k up to about 512 blocks pays for the
    // extra finish launch (70B-class K = 28672, N = 8192: 26.1 -> 22.3 us);
    // smaller matrices run faster on the per-wave kernel.
    const int64_t blocks = (n + 63) / 64, stages = k / SK_CHUNK;
    if (blocks >= 192) return 1;
    if (blocks < 96 || stages < 32) return 0;
    int64_t sp = (512 + blocks - 1) / blocks;
    if (sp > stages / 8) sp = stages / 8;
    return (int)sp;
}

int64_t skinny_workspace_bytes(int64_t m, int64_t n, int64_t k)
{
    if (!skinny_supported(m, n, k)) return 0;
    const int sp = skinny_splits(m, n, k);
    return sp > 1 ? 4 * (int64_t)sp * m * n : 0;
}

hipError_t launch_skinny_pack2(const int8_t *xq, const int32_t *rowsum, int64_t m,
                               const uint8_t *packed, int64_t n, int64_t k, Out out, void *ws,
                               hipStream_t s)
{
    // up to 16 tokens: the shared-activation kernel, its k range split over
    // blocks when the matrix has too few 64-row blocks to keep enough bytes in
    // flight; otherwise the per-wave kernel, which splits k over the waves of
    // a block
    const int sp = skinny_splits(m, n, k);
    if (sp >= 1) return launch_sk2<1>(xq, rowsum, m, packed, n, k, out, sp, (int32_t *)ws, s);
    if (m <= 16) return launch_tg<1>(xq, rowsum, m, packed, n, k, out, s);
    if (m <= 32) return launch_tg<2>(xq, rowsum, m, packed, n, k, out, s);
    return launch_tg<4>(xq, rowsum, m, packed, n, k, out, s);
}

}  // namespace bl
