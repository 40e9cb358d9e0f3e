// Absmean weight quantiser and packers.
//
// Source: "1-bit LLM era: Microsoft introduces BitNet b1.58" (cheatsheet.md),
// section "What is BitNet b1.58?", weight bullet: scale the weights by their
// mean absolute value, round to the nearest integer, restrict to {-1, 0, 1}.
// Packing: the asi.tokyo BitNet b1.58 2B4T article (four trits per byte) and
// the news.hada.io topic 20406 comment on ternary packing (five per byte).
//
// gamma is the exact sum of |w| rounded once to double, divided by N*K in
// double precision and rounded to float; it does not depend on the order in
// which elements are added, so the sum is split over the whole chip.
// The trit decision needs no division: round-half-even(|w| / gamma) >= 1
// exactly when 2|w| > gamma, and 2|w| is exact in float.
//
// Exact sum.  A finite float magnitude is m * 2^(e - 150), m < 2^24 an integer,
// e = max(biased exponent, 1).  Each lane keeps two double accumulators that
// only ever receive magnitudes from a window of exponents [elo, ehi]: such
// values are integer multiples of u = 2^(elo - 150 + LS) (LS = 16 for bf16,
// whose low 16 significand bits are zero, else 0) and smaller than
// 2^(ehi - 126), so C of them sum below C * 2^(ehi - elo + 24 - LS) * u; with
// ehi - elo <= 29 + LS - log2(C) that stays within 2^53 * u and every addition
// is exact.  A lane sets its window from the first non-zero vector it reads
// (top four binades above that vector's largest exponent); magnitudes outside
// it (rare for weight matrices) are added exactly as integers m into per-block
// LDS bins indexed by e.  At the end a lane's accumulators, divided by u, are
// integers below 2^53 and join the bins too.  A block turns its bins into a
// 32-bit-limb integer B = sum * 2^150 (limbs kept as unnormalised 64-bit sums)
// and writes it to the workspace; a one-block kernel adds the blocks' limbs,
// propagates carries and rounds B * 2^-150 to the nearest double.
#include "internal.h"

namespace bl {
namespace {

typedef unsigned long long ull;
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int GAMMA_THREADS = 256;
constexpr int GAMMA_MAX_BLOCKS = 2048;
constexpr int64_t GAMMA_ELEMS_PER_BLOCK = 8192;
constexpr int GAMMA_BINS = 272;      // bin i: integer weight 2^i in B (i <= 254 + 16)
constexpr int GAMMA_LIMBS = 12;      // B < 2^(271 + 64 + 11): 11 limbs, one spare
constexpr int GAMMA_SLOT = 16;       // workspace words per block: limbs, then flags
constexpr int GAMMA_FLAG = GAMMA_LIMBS;
constexpr int GAMMA_MARGIN = 4;      // window top: binades above the first vector's max

__device__ inline float load_w(const void *p, int dtype, int64_t i)
{
    if (dtype == DT_BF16) {
        uint32_t u = (uint32_t)((const uint16_t *)p)[i] << 16;
        return __uint_as_float(u);
    }
    return ((const float *)p)[i];
}

// One lane's accumulation state.  The window is held as bounds on float
// magnitude bits: in window iff lo_m1 <= mag - 1 and mag < hi (mag >= 1).
// Unset: lo_m1 = 0xffffffff, hi = 1, so only zeros pass.
struct GammaLane {
    double acc0 = 0.0, acc1 = 0.0;
    uint32_t lo_m1 = 0xffffffffu, hi = 1u;
    uint32_t lo16_m1 = 0xffffu;   // the low bound for bf16 magnitudes, 16-bit
    int elo = 0;
    uint32_t flags = 0;   // bit 0: an infinity, bit 1: a NaN
};

// Exact handling of one float magnitude outside the fast test: opens the
// window if it is unset, then adds the value to an accumulator or to a bin.
__device__ inline void gamma_slow(GammaLane &L, uint32_t mag, ull *bins)
{
    if (mag == 0u) return;
    const uint32_t e = mag >> 23;
    if (e == 255u) {
        L.flags |= (mag & 0x7fffffu) ? 2u : 1u;
        return;
    }
    if (mag - 1u >= L.lo_m1 && mag < L.hi) {
        L.acc0 += (double)__uint_as_float(mag);
        return;
    }
    const uint32_t m = e ? ((mag & 0x7fffffu) | 0x800000u) : mag;
    atomicAdd(&bins[e ? e : 1u], (ull)m);
}

__device__ inline void gamma_open_window(GammaLane &L, uint32_t max_mag, int width)
{
    if (L.hi != 1u || max_mag == 0u) return;
    const int emax = (int)(max_mag >> 23);
    if (emax >= 255) return;   // only non-finite values so far
    int ehi = emax + GAMMA_MARGIN;
    if (ehi > 254) ehi = 254;
    int elo = ehi - width;
    if (elo < 1) elo = 1;
    L.elo = elo;
    L.lo_m1 = ((uint32_t)elo << 23) - 1u;
    L.lo16_m1 = ((uint32_t)elo << 7) - 1u;
    L.hi = (uint32_t)(ehi + 1) << 23;
}

template <int DT>
__device__ inline void gamma_vector(GammaLane &L, uint4 q, int width, ull *bins)
{
    uint32_t w[4] = {q.x, q.y, q.z, q.w};
    if (DT == DT_BF16) {
        // eight bf16 magnitudes; batch test on packed 16-bit lanes
        u16x2 mx = {0, 0}, mn = {0xffff, 0xffff};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            w[e] &= 0x7fff7fffu;
            u16x2 h = __builtin_bit_cast(u16x2, w[e]);
            mx = __builtin_elementwise_max(mx, h);
            mn = __builtin_elementwise_min(mn, h - (u16x2){1, 1});
        }
        const uint32_t vmax = (uint32_t)(mx.x > mx.y ? mx.x : mx.y) << 16;
        const uint32_t vmin_m1 = mn.x < mn.y ? mn.x : mn.y;   // 0xffff: all zero
        const bool ok = vmax < L.hi && vmin_m1 >= L.lo16_m1;
        if (ok) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                L.acc0 += (double)__uint_as_float(w[e] << 16);
                L.acc1 += (double)__uint_as_float(w[e] & 0xffff0000u);
            }
        } else {
            gamma_open_window(L, vmax, width);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                gamma_slow(L, w[e] << 16, bins);
                gamma_slow(L, w[e] & 0xffff0000u, bins);
            }
        }
    } else {
        uint32_t vmax = 0, vmin_m1 = 0xffffffffu;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            w[e] &= 0x7fffffffu;
            vmax = w[e] > vmax ? w[e] : vmax;
            vmin_m1 = (w[e] - 1u) < vmin_m1 ? (w[e] - 1u) : vmin_m1;
        }
        const bool ok = vmax < L.hi && vmin_m1 >= L.lo_m1;
        if (ok) {
            L.acc0 += (double)__uint_as_float(w[0]);
            L.acc1 += (double)__uint_as_float(w[1]);
            L.acc0 += (double)__uint_as_float(w[2]);
            L.acc1 += (double)__uint_as_float(w[3]);
        } else {
            gamma_open_window(L, vmax, width);
#pragma unroll
            for (int e = 0; e < 4; ++e) gamma_slow(L, w[e], bins);
        }
    }
}

// nvec: whole 16-byte vectors of W; the count - nvec * E tail elements are
// binned by block 0.  width: ehi - elo bound for this launch.
template <int DT>
__global__ __launch_bounds__(GAMMA_THREADS) void gamma_partial_kernel(
    const void *__restrict__ w, int64_t nvec, int64_t count, int width, ull *__restrict__ ws)
{
    __shared__ ull bins[GAMMA_BINS];
    __shared__ ull limbs[GAMMA_LIMBS];
    __shared__ uint32_t block_flags;
    constexpr int E = DT == DT_BF16 ? 8 : 4;
    const int tid = threadIdx.x;
    for (int i = tid; i < GAMMA_BINS; i += GAMMA_THREADS) bins[i] = 0;
    if (tid < GAMMA_LIMBS) limbs[tid] = 0;
    if (tid == 0) block_flags = 0;
    __syncthreads();

    GammaLane L;
    // Block b streams the contiguous vectors [b nvec / G, (b + 1) nvec / G),
    // four per thread and step (16 KB per block and step), the next step's
    // loads issued before this step's arithmetic.  Indices past the range load
    // a clamped (valid) address and are replaced by zero vectors, which add
    // nothing.
    const uint4 *v = (const uint4 *)w;
    const int64_t vbeg = (int64_t)blockIdx.x * nvec / gridDim.x;
    const int64_t vend = (int64_t)(blockIdx.x + 1) * nvec / gridDim.x;
    constexpr int64_t stride = GAMMA_THREADS;
    constexpr int U = 4;
    auto fetch = [&](uint4 (&buf)[U], int64_t base) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            // the load is unconditional and its value always used (masked),
            // so no branch separates it from the others
            const int64_t idx = base + u * stride;
            const uint4 q = v[idx < vend ? idx : vend - 1];
            const uint32_t msk = idx < vend ? 0xffffffffu : 0u;
            buf[u] = make_uint4(q.x & msk, q.y & msk, q.z & msk, q.w & msk);
        }
    };
    int64_t i = vbeg + tid;
    if (vend > vbeg) {
        uint4 cur[U];
        fetch(cur, i);
        for (; i < vend; i += U * stride) {
            uint4 nxt[U];
            fetch(nxt, i + U * stride);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < U; ++u) gamma_vector<DT>(L, cur[u], width, bins);
#pragma unroll
            for (int u = 0; u < U; ++u) cur[u] = nxt[u];
        }
    }
    if (blockIdx.x == 0 && tid == 0) {
        for (int64_t t = nvec * E; t < count; ++t) {
            const float f = load_w(w, DT, t);
            const uint32_t mag = __float_as_uint(f) & 0x7fffffffu;
            if ((mag >> 23) == 255u) L.flags |= (mag & 0x7fffffu) ? 2u : 1u;
            else if (mag) {
                const uint32_t e = mag >> 23;
                atomicAdd(&bins[e ? e : 1u], (ull)(e ? ((mag & 0x7fffffu) | 0x800000u) : mag));
            }
        }
    }
    // the accumulators are integer multiples of u = 2^(elo - 150 + LS), below 2^53 u
    const double acc = L.acc0 + L.acc1;
    if (acc != 0.0) {
        const int ls = DT == DT_BF16 ? 16 : 0;
        const int g = L.elo - 150 + ls;
        atomicAdd(&bins[L.elo + ls], (ull)ldexp(acc, -g));
    }
    if (L.flags) atomicOr(&block_flags, L.flags);
    __syncthreads();
    for (int b = tid; b < GAMMA_BINS; b += GAMMA_THREADS) {
        const ull x = bins[b];
        if (!x) continue;
        const int l = b >> 5, sh = b & 31;
        const uint32_t p0 = (uint32_t)(x << sh);
        const uint32_t p1 = (uint32_t)(sh ? (x >> (32 - sh)) : (x >> 32));
        const uint32_t p2 = (uint32_t)(sh ? (x >> (64 - sh)) : 0ull);
        atomicAdd(&limbs[l], (ull)p0);
        if (p1) atomicAdd(&limbs[l + 1], (ull)p1);
        if (p2) atomicAdd(&limbs[l + 2], (ull)p2);
    }
    __syncthreads();
    ull *slot = ws + (int64_t)blockIdx.x * GAMMA_SLOT;
    if (tid < GAMMA_LIMBS) slot[tid] = limbs[tid];
    if (tid == GAMMA_FLAG) slot[GAMMA_FLAG] = block_flags;
}

// Adds the blocks' limbs, normalises the carries and rounds B * 2^-150 to the
// nearest double (ties to even); gamma = float(sum / (N*K)).  1024 threads:
// thread t adds entry t % 16 of blocks t / 16, t / 16 + 64, ... (coalesced,
// eight loads in flight), then two levels of LDS sums.
constexpr int GAMMA_FIN_THREADS = 1024;
constexpr int GAMMA_FIN_J = GAMMA_FIN_THREADS / GAMMA_SLOT;   // partials per entry

__global__ __launch_bounds__(GAMMA_FIN_THREADS) void gamma_finish_kernel(
    const ull *__restrict__ ws, int nblocks, int64_t n, int64_t k, float *__restrict__ gamma)
{
    __shared__ ull part[GAMMA_SLOT][GAMMA_FIN_J + 1];
    __shared__ ull part2[GAMMA_SLOT][8];
    const int tid = threadIdx.x, e = tid % GAMMA_SLOT, j = tid / GAMMA_SLOT;
    ull s = 0;
    if (e <= GAMMA_FLAG) {
#pragma unroll 8
        for (int b = j; b < nblocks; b += GAMMA_FIN_J) {
            const ull x = ws[(int64_t)b * GAMMA_SLOT + e];
            s = e == GAMMA_FLAG ? (s | x) : s + x;
        }
    }
    part[e][j] = s;
    __syncthreads();
    if (tid < GAMMA_SLOT * 8) {
        const int e2 = tid / 8, q = tid % 8;
        ull t = 0;
        for (int r = 0; r < GAMMA_FIN_J / 8; ++r) {
            const ull x = part[e2][8 * q + r];
            t = e2 == GAMMA_FLAG ? (t | x) : t + x;
        }
        part2[e2][q] = t;
    }
    __syncthreads();
    if (tid != 0) return;
    uint32_t d[GAMMA_LIMBS + 3] = {};
    ull carry = 0, flags = 0;
    for (int l = 0; l < GAMMA_LIMBS; ++l) {
        ull t = carry;
        for (int q = 0; q < 8; ++q) t += part2[l][q];
        d[l] = (uint32_t)t;
        carry = t >> 32;
    }
    for (int q = 0; q < 8; ++q) flags |= part2[GAMMA_FLAG][q];
    if (flags & 2u) {
        gamma[0] = __uint_as_float(0x7fc00000u);
        return;
    }
    if (flags & 1u) {
        gamma[0] = __uint_as_float(0x7f800000u);
        return;
    }
    int top = -1;
    for (int l = GAMMA_LIMBS - 1; l >= 0; --l)
        if (d[l]) {
            top = 32 * l + 31 - __clz(d[l]);
            break;
        }
    double sum = 0.0;
    if (top >= 0) {
        const int low = top > 52 ? top - 52 : 0;     // lowest kept bit
        const int li = low >> 5, sh = low & 31;
        const ull w0 = (ull)d[li] | ((ull)d[li + 1] << 32);
        ull mant = (w0 >> sh) | (sh ? ((ull)d[li + 2] << (64 - sh)) : 0ull);
        mant &= (1ull << 53) - 1ull;
        if (low > 0) {
            const int hb = low - 1;                  // the first dropped bit
            const bool half = (d[hb >> 5] >> (hb & 31)) & 1u;
            bool sticky = (d[hb >> 5] & ((1u << (hb & 31)) - 1u)) != 0u;
            for (int l = 0; l < (hb >> 5); ++l) sticky |= d[l] != 0u;
            if (half && (sticky || (mant & 1ull))) mant += 1ull;
        }
        sum = ldexp((double)mant, low - 150);
    }
    gamma[0] = (float)(sum / ((double)n * (double)k));
}

// ---- trit codes ---------------------------------------------------------------------

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

// Element e of a run of 32-bit words holding bf16 pairs or floats.
template <int DT>
__device__ inline float elem_of(const uint32_t *words, int e)
{
    if (DT == DT_BF16)
        return __uint_as_float((e & 1) ? (words[e >> 1] & 0xffff0000u) : (words[e >> 1] << 16));
    return __uint_as_float(words[e]);
}

// ---- 2-bit packing: one thread per 32-bit word (16 trits) ----------------------
// Word g of row r holds k = 16g + 4i + j at byte j, bits 2i..2i+1.
// VEC: K * sizeof(element) is a multiple of 16, so a whole word's 16 elements
// are 32 (bf16) or 64 (fp32) aligned bytes, read with 16-byte loads.
template <int DT, bool BIN, bool VEC>
__global__ __launch_bounds__(256) void pack2_kernel(const void *__restrict__ w, int64_t n,
                                                    int64_t k, const float *__restrict__ gamma_p,
                                                    uint32_t *__restrict__ packed)
{
    const int64_t words_per_row = pack2_pitch(k) / 4;
    // blocks walk W from its end: the tail that the gamma pass read last is
    // still in the last-level cache when the first blocks run
    const int64_t idx =
        (int64_t)(gridDim.x - 1 - blockIdx.x) * blockDim.x + threadIdx.x;
    if (idx >= n * words_per_row) return;
    const int64_t row = idx / words_per_row, g = idx % words_per_row;
    const float gamma = gamma_p[0];
    const int64_t base = row * k + 16 * g;
    uint32_t word = 0;
    if (VEC && 16 * g + 16 <= k) {
        constexpr int NV = DT == DT_BF16 ? 2 : 4;
        uint32_t raw[4 * NV];
        const uint8_t *src = (const uint8_t *)w + base * (DT == DT_BF16 ? 2 : 4);
#pragma unroll
        for (int c = 0; c < NV; ++c) {
            const uint4 q = load16(src + 16 * c);
            raw[4 * c] = q.x, raw[4 * c + 1] = q.y, raw[4 * c + 2] = q.z, raw[4 * c + 3] = q.w;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                word |= weight_code<BIN>(elem_of<DT>(raw, 4 * i + j), gamma) << (8 * j + 2 * i);
    } else {
        for (int i = 0; i < 4; ++i) {
            for (int j = 0; j < 4; ++j) {
                int64_t kk = 16 * g + 4 * i + j;
                uint32_t code = 1u;
                if (kk < k) code = weight_code<BIN>(load_w(w, DT, base + 4 * i + j), gamma);
                word |= code << (8 * j + 2 * i);
            }
        }
    }
    packed[idx] = word;
}

// ---- base-3 packing: one thread per 32-bit word (4 bytes, 20 trits) ---------------
// VEC: K is a multiple of 4, so the word's 20 elements start 8-byte aligned
// (bf16, five 8-byte loads) or 16-byte aligned (fp32, five 16-byte loads).
template <int DT, bool BIN, bool VEC>
__global__ __launch_bounds__(256) void pack3_kernel(const void *__restrict__ w, int64_t n,
                                                    int64_t k, const float *__restrict__ gamma_p,
                                                    uint32_t *__restrict__ packed)
{
    const int64_t words_per_row = pack3_pitch(k) / 4;
    // blocks walk W from its end: the tail that the gamma pass read last is
    // still in the last-level cache when the first blocks run
    const int64_t idx =
        (int64_t)(gridDim.x - 1 - blockIdx.x) * blockDim.x + threadIdx.x;
    if (idx >= n * words_per_row) return;
    const int64_t row = idx / words_per_row, g = idx % words_per_row;
    const float gamma = gamma_p[0];
    uint32_t word = 0;
    if (VEC && 20 * g + 20 <= k) {
        const int64_t first = row * k + 20 * g;
        uint32_t raw[DT == DT_BF16 ? 10 : 20];
        if (DT == DT_BF16) {
            const uint2 *src = (const uint2 *)((const uint16_t *)w + first);
#pragma unroll
            for (int c = 0; c < 5; ++c) {
                const uint2 q = src[c];
                raw[2 * c] = q.x, raw[2 * c + 1] = q.y;
            }
        } else {
            const uint8_t *src = (const uint8_t *)((const float *)w + first);
#pragma unroll
            for (int c = 0; c < 5; ++c) {
                const uint4 q = load16(src + 16 * c);
                raw[4 * c] = q.x, raw[4 * c + 1] = q.y, raw[4 * c + 2] = q.z, raw[4 * c + 3] = q.w;
            }
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            uint32_t value = 0;
#pragma unroll
            for (int i = 4; i >= 0; --i)
                value = 3u * value + weight_code<BIN>(elem_of<DT>(raw, 5 * b + i), gamma);
            word |= value << (8 * b);
        }
    } else {
        for (int b = 0; b < 4; ++b) {
            const int64_t byte_idx = 4 * g + b;
            uint32_t value = 0, weight = 1;
            for (int i = 0; i < 5; ++i) {
                int64_t kk = 5 * byte_idx + i;
                uint32_t code = 1u;
                if (kk < k) code = weight_code<BIN>(load_w(w, DT, row * k + kk), gamma);
                value += code * weight;
                weight *= 3u;
            }
            word |= value << (8 * b);
        }
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

int gamma_blocks(int64_t count)
{
    int64_t b = (count + GAMMA_ELEMS_PER_BLOCK - 1) / GAMMA_ELEMS_PER_BLOCK;
    if (b < 1) b = 1;
    if (b > GAMMA_MAX_BLOCKS) b = GAMMA_MAX_BLOCKS;
    return (int)b;
}

int64_t gamma_workspace_bytes(int64_t count)
{
    return (int64_t)gamma_blocks(count) * GAMMA_SLOT * (int64_t)sizeof(ull);
}

hipError_t launch_gamma(const void *w, int dtype, int64_t n, int64_t k, void *workspace,
                        float *gamma, hipStream_t s)
{
    const int64_t count = n * k;
    const int esz = dtype == DT_BF16 ? 2 : 4, per_vec = 16 / esz;
    const int64_t nvec = count / per_vec;
    const int blocks = gamma_blocks(count);
    // the most elements one lane adds to its accumulators, as a power of two
    // (a block's range holds at most ceil(nvec / blocks) vectors)
    const int64_t per_block = (nvec + blocks - 1) / blocks;
    const int64_t per_lane = ((per_block + GAMMA_THREADS - 1) / GAMMA_THREADS) * per_vec;
    int p = 0;
    while (((int64_t)1 << p) < per_lane) ++p;
    const int width = 29 + (dtype == DT_BF16 ? 16 : 0) - p;
    if (width < 1) return hipErrorInvalidValue;   // beyond 2^40 elements
    ull *ws = (ull *)workspace;
    if (dtype == DT_BF16)
        hipLaunchKernelGGL(gamma_partial_kernel<DT_BF16>, dim3(blocks), dim3(GAMMA_THREADS), 0, s,
                           w, nvec, count, width, ws);
    else
        hipLaunchKernelGGL(gamma_partial_kernel<DT_F32>, dim3(blocks), dim3(GAMMA_THREADS), 0, s, w,
                           nvec, count, width, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gamma_finish_kernel, dim3(1), dim3(GAMMA_FIN_THREADS), 0, s,
                       (const ull *)ws, blocks, n, k, gamma);
    return hipGetLastError();
}

namespace {
template <int DT, bool BIN>
void pack_launch(const void *w, int64_t n, int64_t k, int layout, const float *gamma,
                 uint8_t *packed, hipStream_t s)
{
    if (layout == LAYOUT_PACK2) {
        const int64_t words = n * (pack2_pitch(k) / 4);
        const bool vec = (k * (DT == DT_BF16 ? 2 : 4)) % 16 == 0;
        if (vec)
            hipLaunchKernelGGL((pack2_kernel<DT, BIN, true>), dim3(blocks_for(words, 256)),
                               dim3(256), 0, s, w, n, k, gamma, (uint32_t *)packed);
        else
            hipLaunchKernelGGL((pack2_kernel<DT, BIN, false>), dim3(blocks_for(words, 256)),
                               dim3(256), 0, s, w, n, k, gamma, (uint32_t *)packed);
    } else {
        const int64_t words = n * (pack3_pitch(k) / 4);
        if (k % 4 == 0)
            hipLaunchKernelGGL((pack3_kernel<DT, BIN, true>), dim3(blocks_for(words, 256)),
                               dim3(256), 0, s, w, n, k, gamma, (uint32_t *)packed);
        else
            hipLaunchKernelGGL((pack3_kernel<DT, BIN, false>), dim3(blocks_for(words, 256)),
                               dim3(256), 0, s, w, n, k, gamma, (uint32_t *)packed);
    }
}
}  // namespace

hipError_t launch_pack(const void *w, int dtype, int64_t n, int64_t k, int layout,
                       const float *gamma, uint8_t *packed, hipStream_t s, bool binary)
{
    if (dtype == DT_BF16) {
        if (binary) pack_launch<DT_BF16, true>(w, n, k, layout, gamma, packed, s);
        else pack_launch<DT_BF16, false>(w, n, k, layout, gamma, packed, s);
    } else {
        if (binary) pack_launch<DT_F32, true>(w, n, k, layout, gamma, packed, s);
        else pack_launch<DT_F32, false>(w, n, k, layout, gamma, packed, s);
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
