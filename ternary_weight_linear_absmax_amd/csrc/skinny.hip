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
#include "dma.h"
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
    double e_g[TG];
#pragma unroll
    for (int g = 0; g < TG; ++g) {
        const int64_t tok = 16 * g + r < m ? 16 * g + r : m - 1;
        xrow[g] = xq + tok * k + 64 * b;
        // epilogue operands of this lane's tokens, loaded before the stream
        e_rs[g] = rowsum[tok];
        e_g[g] = out.acc ? 0.0 : epi_gs(out.gamma[0], out.scale[tok]);
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
                    out.y[tok * ldy + row0 + q] = epi_y(v, e_g[g]);
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


namespace {

// ---- shared-activation variant -------------------------------------------------
// Block: 64 RB weight rows and all M (<= 16) tokens, over all k stages of KS;
// used when the row blocks fill the CUs.  Four producer waves move both
// operands of each stage straight into an LDS ring of NS stages (direct
// loads: RB KS / 16 bytes of weights and 16 KS of activations per stage),
// so that NS - 2 stages of weights are in flight per block without holding
// them in registers; four math waves read both from LDS, each on 16 RB of
// the rows (one activation fragment feeds RB MFMAs).  (A predecessor
// streamed the weights into registers, four stages ahead, and copied the
// activations through registers into a padded LDS ring: 20.0 / 22.3 us on
// the 70B-class matrices at M = 16, against 17.1 / 19.3 us.)
// RB = 1 on the 2B-class matrices: KS = 512 in four stages (64 KB, two
// blocks per CU) where K % 512 = 0 (up/gate, K = 2560, at M = 4 / 8 / 16:
// 5.43 / 5.53 / 5.58 -> 5.12 / 5.23 / 5.31 us; six such stages 5.37-5.69 us),
// else KS = 256 in six stages (48 KB).
// RB = 2 on the 70B-class matrices: each activation stage then serves twice
// the weight bytes (M = 16, rotating weights, paired timing: 19.0 -> 17.7 us
// with K = 8192, 21.8 -> 20.0 us with K = 28672 split four ways instead of
// two; rings of 10 or 12 stages 18.9 / 21.1 and 19.4 / 21.8 us; eight splits
// 21.8 us); and there KS = 512 in a four-stage ring (96 KB: half the
// barriers per k) runs 15.9 -> 13.9 us and 18.8 -> 16.9 us (five or six
// stages 14.3-15.0 / 17.3-17.8 us, three 14.2 / 17.0; KS = 1024 in three
// stages 14.7 / 18.7 us).
// Ring layout without padding, 16-byte chunks permuted so that a fragment
// read of consecutive rows hits distinct bank groups: weights [BN rows][KS/4
// bytes], chunk c of row r at c ^ wswz(r); activations [16 tokens][KS
// bytes], chunk c of token t at c ^ t.  Stage j + 1 is published at the
// barrier that ends stage j (producers wait on their own load counter; no
// fence on either side: a math wave's reads of stage j are consumed by its
// MFMAs before it reaches the barrier).  k mapping: lane (r, b) takes the
// stage's k range [KS/4 b, KS/4 (b + 1)); word u of its packed bytes <->
// activation bytes KS/4 b + 16 u .. +15 of the stage; K % KS = 0.
// gridDim.y > 1 splits the stages over blocks: each split stores its raw
// code sums into its own slice of a partial buffer, which a finish kernel
// adds in split order (device-scope atomics with a last-block finish instead
// measured several times slower: the atomics dominate).
// Ring depth with KS = 256: six stages (48 KB with RB = 1, four stages of
// weights in flight per block); timed on the 70B-class matrices at M = 16
// with rotating weights and RB = 1: four stages 18.8 us, six 17.1, eight
// 17.4, nine 17.7 (K = 8192).
constexpr int SK3_NS = 6;

// LDS position of a weight row's 16-byte chunks: chunk c of row r at
// c ^ wswz(r), so that eight consecutive rows' chunks of one fragment read
// fall in distinct bank groups (rows of 64 bytes: four rows share a bank
// group pattern, hence r >> 2; rows of 128 bytes and more: r itself)
template <int KS>
__device__ inline int wswz(int r) { return KS == 256 ? (r >> 2) & 3 : r & 7; }

template <int NS, int RB, int KS = 256>
__global__ __launch_bounds__(512) void skinny3_kernel(const int8_t *__restrict__ xq,
                                                      const int32_t *__restrict__ rowsum,
                                                      int64_t m, int64_t k,
                                                      const uint8_t *__restrict__ packed,
                                                      int64_t n, int64_t pitch, Out out,
                                                      int64_t ldy, int32_t *__restrict__ part)
{
    static_assert(NS >= 3, "two stages in flight");
    constexpr int MT = 16, BN = 64 * RB;
    constexpr int SW = BN * (KS / 4), SX = MT * KS, SS = SW + SX;
    constexpr int CW = KS / 64;             // 16-byte chunks of a weight row per stage
    constexpr int WT = SW / 1024 / 4;       // weight transfers per producer wave
    constexpr int XT = SX / 1024 / 4;       // activation transfers per producer wave
    constexpr int PT = WT + XT;             // direct loads per producer wave and stage
    __shared__ __attribute__((aligned(16))) uint8_t lds[NS * SS];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t n0 = (int64_t)blockIdx.x * BN;
    const int ns_all = (int)(k / KS);
    const int s0 = (int)((int64_t)blockIdx.y * ns_all / gridDim.y);
    const int s1 = (int)((int64_t)(blockIdx.y + 1) * ns_all / gridDim.y);
    const int ns = s1 - s0;
    v4i acc[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) acc[i] = v4i{0, 0, 0, 0};
    const int r = lane & 15, b = lane >> 4;

    if (wave >= 4) {
        // producer wave pw fills weight rows 16 (pw RB + q) .. + 15 (q < RB)
        // and tokens 4 pw .. 4 pw + 3 of every stage (1 KB each); rows and
        // tokens past the matrices are clamped (they feed outputs that are
        // never stored)
        const int pw = wave - 4;
        const uint8_t *wsrc[WT];
#pragma unroll
        for (int q = 0; q < WT; ++q) {
            const int wr = (1024 / (KS / 4)) * (pw * WT + q) + lane / CW;
            int64_t row = n0 + wr;
            row = row < n ? row : n - 1;
            wsrc[q] = packed + row * pitch + (int64_t)s0 * (KS / 4) +
                      16 * ((lane % CW) ^ wswz<KS>(wr));
        }
        const int8_t *xsrc[XT];
#pragma unroll
        for (int q = 0; q < XT; ++q) {
            const int xt = (1024 / KS) * (pw * XT + q) + lane / (KS / 16);
            int64_t tok = xt;
            tok = tok < m ? tok : m - 1;
            xsrc[q] = xq + tok * k + (int64_t)s0 * KS + 16 * ((lane % (KS / 16)) ^ xt);
        }
        auto issue = [&](int st) __attribute__((always_inline)) {
            uint8_t *slot = lds + (st % NS) * SS;
#pragma unroll
            for (int q = 0; q < WT; ++q)
                dl_load16(wsrc[q] + (int64_t)st * (KS / 4), slot + 1024 * (pw * WT + q));
#pragma unroll
            for (int q = 0; q < XT; ++q)
                dl_load16(xsrc[q] + (int64_t)st * KS, slot + SW + 1024 * (pw * XT + q));
        };
        static_for<NS - 1>([&](auto sc) __attribute__((always_inline)) {
            if (decltype(sc)::value < ns) issue(decltype(sc)::value);
        });
        if (ns >= NS - 1) __builtin_amdgcn_s_waitcnt(dl_vmcnt((NS - 2) * PT));
        else __builtin_amdgcn_s_waitcnt(dl_vmcnt(0));
        dl_barrier();
        for (int j = 0; j < ns; ++j) {
            if (j + NS - 1 < ns) {
                issue(j + NS - 1);
                __builtin_amdgcn_s_waitcnt(dl_vmcnt((NS - 2) * PT));   // stage j + 1 landed
            } else {
                __builtin_amdgcn_s_waitcnt(dl_vmcnt(0));
            }
            dl_barrier();
        }
    } else {
        // math wave: weight rows 16 (RB wave + i) + r (A operands), tokens r (B)
        // lane (r, b) takes the stage's k range [KS/4 b, KS/4 (b + 1)): packed
        // chunks CW/4 b .. of its weight rows, activation chunks of token r
        constexpr int CL = CW / 4;          // weight chunks per lane and stage
        int woff[RB][CL];
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            const int wr = 16 * (RB * wave + i) + r;
#pragma unroll
            for (int c = 0; c < CL; ++c)
                woff[i][c] = wr * (KS / 4) + 16 * ((CL * b + c) ^ wswz<KS>(wr));
        }
        dl_barrier();
        for (int j = 0; j < ns; ++j) {
            const uint8_t *slot = lds + (j % NS) * SS;
            uint4 wv[RB][CL];
#pragma unroll
            for (int i = 0; i < RB; ++i)
#pragma unroll
                for (int c = 0; c < CL; ++c) wv[i][c] = load16(slot + woff[i][c]);
            v4i xb[4 * CL];
#pragma unroll
            for (int u = 0; u < 4 * CL; ++u) {
                const uint4 v = load16(slot + SW + r * KS + 16 * ((4 * CL * b + u) ^ r));
                xb[u] = v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
            }
#pragma unroll
            for (int u = 0; u < 4 * CL; ++u)
#pragma unroll
                for (int i = 0; i < RB; ++i)
                    acc[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                        unpack_word16(word_at(wv[i][u / 4], u % 4)), xb[u], acc[i], 0, 0, 0);
            dl_barrier();
        }
    }
    __syncthreads();   // every load has landed and every read is done

    // Epilogue (math lanes hold D[4 b + q][r] of row tile i = weight row
    // 16 (RB wave + i) + 4 b + q, token r): the [16 tokens][BN rows] tile
    // transposed through LDS, then four consecutive rows of one token per
    // thread, as in the shared-activation kernel.
    int32_t *tile = (int32_t *)lds;   // [MT][BN + 4]
    if (wave < 4)
#pragma unroll
        for (int i = 0; i < RB; ++i)
            *(v4i *)(tile + r * (BN + 4) + 16 * (RB * wave + i) + 4 * b) = acc[i];
    __syncthreads();
    const uintptr_t base = part ? 0 : out.acc ? (uintptr_t)out.acc : (uintptr_t)out.y;
    const bool vec = (n % 4) == 0 && (part || ((ldy % 4) == 0 && (base & 15) == 0));
    for (int e = tid; e < MT * (BN / 4); e += 512) {
        const int t = e / (BN / 4), c4 = 4 * (e % (BN / 4));
        if (t >= m) continue;
        const int64_t row = n0 + c4;
        if (row >= n) continue;
        const v4i v = *(const v4i *)(tile + t * (BN + 4) + c4);
        if (part) {
            int32_t *dst = part + ((int64_t)blockIdx.y * m + t) * n + row;
            if (vec && row + 3 < n) {
                *(v4i *)dst = v;
            } else {
                for (int q = 0; q < 4 && row + q < n; ++q) dst[q] = v[q];
            }
            continue;
        }
        const int32_t rs = rowsum[t];
        if (out.acc) {
            int32_t *dst = out.acc + t * ldy + row;
            const v4i a = v - rs;
            if (vec && row + 3 < n) *(v4i *)dst = a;
            else
                for (int q = 0; q < 4 && row + q < n; ++q) dst[q] = a[q];
        } else {
            const double gs = epi_gs(out.gamma[0], out.scale[t]);
            float *dst = out.y + t * ldy + row;
            float4 f;
            f.x = epi_y(v[0] - rs, gs);
            f.y = epi_y(v[1] - rs, gs);
            f.z = epi_y(v[2] - rs, gs);
            f.w = epi_y(v[3] - rs, gs);
            if (vec && row + 3 < n) *(float4 *)dst = f;
            else {
                const float fa[4] = {f.x, f.y, f.z, f.w};
                for (int q = 0; q < 4 && row + q < n; ++q) dst[q] = fa[q];
            }
        }
    }
}

}  // namespace

namespace {

// 128-row blocks (RB = 2) for matrices with at least 160 of them, or at least
// 32 with rows of at least 64 stages (split over blocks); K of at least 16
// stages.  The 2B-class matrices keep 64-row blocks.
bool wide_rows(int64_t n, int64_t k)
{
    const int64_t b128 = (n + 127) / 128, stages = k / SK_CHUNK;
    return stages >= 16 && (b128 >= 160 || (b128 >= 32 && stages >= 64));
}

hipError_t launch_shared(const int8_t *xq, const int32_t *rowsum, int64_t m,
                         const uint8_t *packed, int64_t n, int64_t k, Out out, int splits,
                         int32_t *part, hipStream_t s)
{
    int32_t *pp = splits > 1 ? part : (int32_t *)nullptr;
    if (wide_rows(n, k))
        if (k % 512 == 0)
            hipLaunchKernelGGL((skinny3_kernel<4, 2, 512>),
                               dim3((unsigned)((n + 127) / 128), (unsigned)splits), dim3(512), 0,
                               s, xq, rowsum, m, k, packed, n, pack2_pitch(k), out, (int64_t)n, pp);
        else
            hipLaunchKernelGGL((skinny3_kernel<SK3_NS, 2, 256>),
                               dim3((unsigned)((n + 127) / 128), (unsigned)splits), dim3(512), 0,
                               s, xq, rowsum, m, k, packed, n, pack2_pitch(k), out, (int64_t)n, pp);
    else if (k % 512 == 0)
        hipLaunchKernelGGL((skinny3_kernel<4, 1, 512>),
                           dim3((unsigned)((n + 63) / 64), (unsigned)splits), dim3(512), 0, s,
                           xq, rowsum, m, k, packed, n, pack2_pitch(k), out, (int64_t)n, pp);
    else
        hipLaunchKernelGGL((skinny3_kernel<SK3_NS, 1>),
                           dim3((unsigned)((n + 63) / 64), (unsigned)splits), dim3(512), 0, s,
                           xq, rowsum, m, k, packed, n, pack2_pitch(k), out, (int64_t)n, pp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits == 1) return e;
    return launch_splitk_finish(part, rowsum, m, n, splits, out, n, s);
}

}  // namespace

int skinny_splits(int64_t m, int64_t n, int64_t k)
{
    if (m > 16 || k % SK_CHUNK != 0) return 0;   // 0: the per-wave kernel
    if (wide_rows(n, k)) {
        // about one 128-row block per CU, at least eight stages (of 512 k,
        // or 256 when K % 512 != 0) per split (70B-class: K = 8192 unsplit,
        // K = 28672 four ways)
        const int64_t b128 = (n + 127) / 128, stages = k / (k % 512 == 0 ? 512 : 256);
        int sp = (int)(256 / b128);
        sp = sp < 1 ? 1 : sp;
        while (sp > 1 && stages / sp < 8) --sp;
        return sp;
    }
    // Measured on the 2B- and 70B-class shapes at M = 16: with >= 192 blocks of
    // 64 rows the unsplit kernel is fastest; with 96..191 blocks and long rows
    // (>= 32 stages of 256 k) the k range split in two (about one block per
    // CU) pays for the extra finish launch (70B-class K = 28672, N = 8192 with
    // the direct-load kernel: 19.3 us split two ways, 22.6 three, 19.9 four);
    // smaller matrices run faster on the per-wave kernel.
    const int64_t blocks = (n + 63) / 64, stages = k / SK_CHUNK;
    if (blocks >= 192) return 1;
    if (blocks < 96 || stages < 32) return 0;
    return 2;
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
    if (sp >= 1) return launch_shared(xq, rowsum, m, packed, n, k, out, sp, (int32_t *)ws, s);
    if (m <= 16) return launch_tg<1>(xq, rowsum, m, packed, n, k, out, s);
    if (m <= 32) return launch_tg<2>(xq, rowsum, m, packed, n, k, out, s);
    return launch_tg<4>(xq, rowsum, m, packed, n, k, out, s);
}

}  // namespace bl
