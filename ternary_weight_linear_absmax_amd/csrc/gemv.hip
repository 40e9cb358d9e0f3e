// Ternary GEMV kernels for small token counts (decode): y[m, n] for M <= 4 per
// pass, streaming the packed weights from HBM once.
//
// Source: asi.tokyo BitNet b1.58 2B4T article, packing paragraph: the trits
// travel packed (four per byte) and are unpacked right next to the arithmetic
// units, where they are multiplied with the 8-bit activations.  The codes are
// offset by one, so sum_k (t+1) q = acc + rowsum(q); the row sum from the
// activation quantiser is subtracted once per output.
//
// Arithmetic of the 2-bit kernel: a packed word masked with 0x33333333 holds
// eight 2-bit codes in eight nibbles (k = j and 8 + j of its 16 trits), and
// shifted right by 2 first, the other eight (4 + j, 12 + j).  The activations
// are split once per block into their low (unsigned) and high (signed) nibbles
// in the same order, so that v_dot8 (4-bit dot products of eight) gives
// sum c x = 16 sum c hi + sum c lo: 7 ALU operations per 16 trits.  Kernels
// that read the activations with the weights use v_dot4 on
// (word >> 2i) & 0x03030303 (four consecutive k as int8 codes) instead, with
// two of the four shifts replaced by a second mask whose products are 4x
// too large and collected apart: 9 operations per 16 trits.
#include "internal.h"

namespace bl {
namespace {

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

// 64 activation bytes k = 64c .. 64c+63 of one token; zero past K.  AL: K is a
// multiple of 16, so every 16-byte piece is wholly inside or outside the row.
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

// A 4-byte load that always takes the vector memory path (a raw buffer load
// of a 4-byte range; a uniform address would otherwise become a scalar load).
// Vector loads return in issue order, so one issued just ahead of a kernel's
// weight loads has arrived by the time the first weights have; a scalar load
// in flight instead holds up every later kernel-argument load (whose wait
// drains the scalar counter to zero), and one left to the compiler tends to
// sink to its first use in the epilogue, adding a memory latency there.
__device__ inline uint32_t vload_u32(const void *p)
{
    // 0x00020000: the gfx9 raw-buffer descriptor word (untyped 32-bit data)
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void *)p, 0, 4, 0x00020000);
    return __builtin_amdgcn_raw_buffer_load_b32(r, 0, 0, 0);
}

// ---- 2-bit layout ------------------------------------------------------------
// A block is KS waves.  It owns RB = R * ST consecutive weight rows; wave w
// takes the w-th share of every row's 16-byte chunks, and lane l of the wave
// takes chunks l and l + 64 of that share (CPL <= 2), so a lane holds at most
// 2 x 64 activation bytes per token in registers.  The block walks its rows in
// ST steps of R rows; the weights of steps s+1 and s+2 are issued before the
// arithmetic of step s (a scheduling barrier keeps them there), so every wave
// always has loads in flight, and a kernel that quantises its token first has
// the first two steps' weights on the way meanwhile (two steps ahead measured
// 3.2% faster per decode launch than one, and faster than all steps at once).
// Row indices past N are clamped: the loads stay in bounds and
// those rows are not stored.  Per-wave partial sums go through LDS and are
// combined once at the end.
constexpr int GEMV_R = 2;
constexpr int GEMV_KS_MAX = 8;
constexpr int GEMV_WAVES = 4;   // waves per block when K is short
#ifndef GEMV_PF
#define GEMV_PF 2               // steps of weight loads in flight ahead
#endif

// One token quantised inside the product (QDT = input type, VPT = 16-byte
// input vectors per thread): the block's threads split the token, reduce
// max |x| over the block, quantise their vectors with the same arithmetic as
// the activation quantiser (s = 127 / max|x|, q = rint(x s) clamped) into an
// LDS copy of the int8 token, and sum the bytes for the row sum; every lane
// then reads its chunks' activations from LDS.  Block 0 also writes xq, s and
// the row sum.
constexpr int GEMV_X_LDS = -2;   // QDT value: int8 token staged in LDS
constexpr int64_t GEMV_X_LDS_MAX_K = 32768;

struct FuseQ {
    const void *x;        // [K] input token (bf16 or fp32)
    int8_t *xq;           // [K]
    float *scale;         // [1]
    int32_t *rowsum;      // [1]
};

template <int MT, int CPL, int ST, bool AL, int QDT = -1, int VPT = 0>
__global__ __launch_bounds__(GEMV_KS_MAX * 64) void gemv2_kernel(
    const int8_t *__restrict__ xq, const int32_t *__restrict__ rowsum, int64_t k,
    const uint4 *__restrict__ packed, int64_t n, int64_t chunks, int64_t share, Out out,
    int64_t ldy, int64_t m0, int ks, FuseQ fq)
{
    constexpr int R = GEMV_R, RB = GEMV_R * ST;
    constexpr bool FUSED = QDT >= 0;
    constexpr bool XLDS = QDT == GEMV_X_LDS;   // int8 token staged once per block in LDS
    static_assert(!(FUSED || XLDS) || (MT == 1 && AL), "one token, K % 16 == 0");
    // A block is ks x wr waves: wave w takes k-share w % ks of the rows of
    // row group w / ks; the block's wr * RB rows are contiguous, and their
    // outputs are written together at the end.
    __shared__ int part[GEMV_KS_MAX][GEMV_KS_MAX * RB][MT];
    __shared__ float q_max[GEMV_KS_MAX];
    __shared__ int q_sum[GEMV_KS_MAX];
    extern __shared__ uint4 q_lds[];   // fused: the int8 token, K bytes
    const int wr = (int)(blockDim.x >> 6) / ks;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kw = wave % ks, rw = wave / ks;
    const int64_t blk0 = (int64_t)blockIdx.x * wr * RB;
    const int64_t row0 = blk0 + (int64_t)rw * RB;

    int64_t coff[CPL];
    bool ok[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int64_t c = kw * share + lane + 64 * j;
        ok[j] = (lane + 64 * j < share) && c < chunks;
        coff[j] = ok[j] ? c : 0;
    }

    // One token read once per block (fused quantisation, or the int8 token
    // staged in LDS): its 16-byte vectors are loaded before the weights, so
    // that the first use waits only for them while the weight loads stay in
    // flight.
    constexpr int QE = QDT == DT_BF16 ? 8 : QDT == DT_F32 ? 4 : 16;   // values per vector
    uint4 raw[(FUSED || XLDS) ? VPT : 1];
    if constexpr (FUSED || XLDS) {
        const int nvec = (int)(k / QE);
        const uint8_t *src = FUSED ? (const uint8_t *)fq.x : (const uint8_t *)(xq + m0 * k);
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            const int i = threadIdx.x + (int)blockDim.x * v;
            raw[v] = i < nvec ? load16(src + 16 * (int64_t)i) : zero4();
        }
        __builtin_amdgcn_sched_barrier(0);
    }

    // Activations read straight from global memory (neither fused nor staged
    // in LDS): every lane's activation loads and the epilogue operands go out
    // before the weights, with no branch or use between them (the operands'
    // loads read the row sums in place of gamma and s for an int32 output),
    // so that nothing waits for one of them before the weight loads are out.
    uint4 xv[MT][CPL][4];
    int32_t g_rs = 0;
    float g_g = 0.0f, g_sc = 1.0f;
    if constexpr (!FUSED && !XLDS) {
        const int g_t = threadIdx.x % MT;
        const float *gp = out.acc ? (const float *)rowsum : out.gamma;
        const float *sp = out.acc ? (const float *)rowsum + m0 : out.scale + m0;
        g_rs = rowsum[m0 + g_t];
        g_g = __uint_as_float(vload_u32(gp));
        g_sc = sp[g_t];
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                if constexpr (AL) {
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        const int64_t e0 = 64 * coff[j] + 16 * d;
                        xv[t][j][d] = load16(xq + (m0 + t) * k + (e0 < k ? e0 : 0));
                    }
                } else {
                    load_x64<AL>(xq + (m0 + t) * k, k, coff[j], xv[t][j]);
                }
            }
        __builtin_amdgcn_sched_barrier(0);
    }

    // weight ring: GEMV_PF steps of loads in flight ahead of the arithmetic
    constexpr int PF = GEMV_PF < ST ? GEMV_PF : ST;
    uint4 w[PF + 1][R][CPL];
    auto load = [&](uint4(&wb)[R][CPL], int s) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            int64_t row = row0 + s * R + r;
            row = row < n ? row : n - 1;
#pragma unroll
            for (int j = 0; j < CPL; ++j) wb[r][j] = load_nt16(packed + row * chunks + coff[j]);
        }
    };
#pragma unroll
    for (int q = 0; q < PF; ++q) load(w[q], q);
    __builtin_amdgcn_sched_barrier(0);

    // Epilogue operands (row sum, gamma / s) of the output this thread writes
    // at the end (wr * RB * MT <= blockDim outputs, one per thread), loaded
    // now so that their latency overlaps the weight stream.
    const int nout = wr * RB * MT;
    const int e_rr = threadIdx.x / MT, e_t = threadIdx.x % MT;
    int32_t e_rs = 0;
    double e_gs = 0.0;
    if (XLDS && threadIdx.x < nout) {
        e_rs = rowsum[m0 + e_t];
        if (!out.acc) e_gs = epi_gs(out.gamma[0], out.scale[m0 + e_t]);
    }
    if constexpr (!FUSED && !XLDS) {
        e_rs = g_rs;
        if (!out.acc) e_gs = epi_gs(g_g, g_sc);
    }

    float q_s = 0.0f;
    if constexpr (XLDS) {
        const int nvec = (int)(k / 16);
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            const int i = threadIdx.x + (int)blockDim.x * v;
            if (i < nvec) q_lds[i] = raw[v];
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < CPL; ++j)
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const int64_t e0 = 64 * coff[j] + 16 * d;   // K % 16 == 0: pieces are whole
                xv[0][j][d] = (ok[j] && e0 < k) ? q_lds[e0 / 16] : zero4();
            }
    } else if constexpr (!FUSED) {
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int j = 0; j < CPL; ++j)
#pragma unroll
                for (int d = 0; d < 4; ++d)
                    if (!ok[j] || (AL && 64 * coff[j] + 16 * d >= k)) xv[t][j][d] = zero4();
    } else {
        const int nvec = (int)(k / QE), nthr = (int)blockDim.x;
        const float gamma = out.gamma[0];
        float amax = 0.0f;
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            const uint32_t u[4] = {raw[v].x, raw[v].y, raw[v].z, raw[v].w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
                amax = QDT == DT_BF16
                           ? fmaxf(amax, fmaxf(fabsf(bf16_lo(u[i])), fabsf(bf16_hi(u[i]))))
                           : fmaxf(amax, fabsf(__uint_as_float(u[i])));
        }
        amax = wave_max_dpp(amax);
        if (lane == 63) q_max[wave] = amax;
        __syncthreads();
        amax = 0.0f;
        for (int q = 0; q < nthr / 64; ++q) amax = fmaxf(amax, q_max[q]);
        q_s = act_scale(amax);

        int sum = 0;
        uint8_t *ql = (uint8_t *)q_lds;
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            const int i = threadIdx.x + nthr * v;
            if (i >= nvec) continue;
            const uint32_t u[4] = {raw[v].x, raw[v].y, raw[v].z, raw[v].w};
            if (QDT == DT_BF16) {
                uint32_t d[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    d[h] = quant4(bf16_lo(u[2 * h]), bf16_hi(u[2 * h]), bf16_lo(u[2 * h + 1]),
                                  bf16_hi(u[2 * h + 1]), q_s);
                    sum = __builtin_amdgcn_sdot4((int)d[h], 0x01010101, sum, false);
                }
                const uint2 qv = make_uint2(d[0], d[1]);
                *(uint2 *)(ql + 8 * i) = qv;
                if (blockIdx.x == 0) *(uint2 *)(fq.xq + 8 * (int64_t)i) = qv;
            } else {
                const uint32_t d = quant4(__uint_as_float(u[0]), __uint_as_float(u[1]),
                                          __uint_as_float(u[2]), __uint_as_float(u[3]), q_s);
                sum = __builtin_amdgcn_sdot4((int)d, 0x01010101, sum, false);
                *(uint32_t *)(ql + 4 * i) = d;
                if (blockIdx.x == 0) *(uint32_t *)(fq.xq + 4 * (int64_t)i) = d;
            }
        }
        sum = wave_sum_dpp(sum);
        if (lane == 63) q_sum[wave] = sum;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < CPL; ++j)
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const int64_t e0 = 64 * coff[j] + 16 * d;   // K % 16 == 0: pieces are whole
                xv[0][j][d] = (ok[j] && e0 < k) ? q_lds[e0 / 16] : zero4();
            }
        if (!out.acc) e_gs = epi_gs(gamma, q_s);
    }
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int j = 0; j < CPL; ++j)
#pragma unroll
            for (int d = 0; d < 4; ++d) xv[t][j][d] = nibble_split(xv[t][j][d]);

#pragma unroll
    for (int s = 0; s < ST; ++s) {
        if (s + PF < ST) load(w[(s + PF) % (PF + 1)], s + PF);
        __builtin_amdgcn_sched_barrier(0);
        const int b = s % (PF + 1);
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                int ah = 0;
                uint32_t al = 0;
#pragma unroll
                for (int j = 0; j < CPL; ++j) {
                    dot8_word(w[b][r][j].x, xv[t][j][0], ah, al);
                    dot8_word(w[b][r][j].y, xv[t][j][1], ah, al);
                    dot8_word(w[b][r][j].z, xv[t][j][2], ah, al);
                    dot8_word(w[b][r][j].w, xv[t][j][3], ah, al);
                }
                const int v = wave_sum_dpp(16 * ah + (int)al);
                if (lane == 63) part[kw][rw * RB + s * R + r][t] = v;
            }
        }
    }
    __syncthreads();
    if (FUSED) {
        for (int q = 0; q < (int)(blockDim.x >> 6); ++q) e_rs += q_sum[q];
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            fq.scale[0] = q_s;
            fq.rowsum[0] = e_rs;
        }
    }
    if (threadIdx.x < nout && blk0 + e_rr < n) {
        int sum = 0;
        for (int q = 0; q < ks; ++q) sum += part[q][e_rr][e_t];
        const int32_t acc = sum - e_rs;
        const int64_t idx = (m0 + e_t) * ldy + blk0 + e_rr;
        if (out.acc)
            out.acc[idx] = acc;
        else
            out.y[idx] = epi_y(acc, e_gs);
    }
}

// Rows longer than GEMV_KS_MAX * 128 chunks (K > 65536): one wave per row,
// lanes stride over the chunks, activations loaded with each chunk.
template <bool AL>
__global__ __launch_bounds__(256) void gemv2_long_kernel(const int8_t *__restrict__ xq,
                                                         const int32_t *__restrict__ rowsum,
                                                         int64_t k, const uint4 *__restrict__ packed,
                                                         int64_t n, int64_t chunks, Out out,
                                                         int64_t ldy, int64_t m)
{
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= n) return;
    for (int64_t t = 0; t < m; ++t) {
        int lo = 0, hi = 0;
        for (int64_t c = lane; c < chunks; c += 64) {
            const uint4 w = load_nt16(packed + row * chunks + c);
            uint4 xv[4];
            load_x64<AL>(xq + t * k, k, c, xv);
            dot_word(w.x, xv[0], lo, hi);
            dot_word(w.y, xv[1], lo, hi);
            dot_word(w.z, xv[2], lo, hi);
            dot_word(w.w, xv[3], lo, hi);
        }
        const int v = wave_sum_dpp(lo + (hi >> 2));
        if (lane == 63) store_out(out, ldy, t, row, v, rowsum[t]);
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
    int32_t e_rs[MT];
    double e_gs[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        acc[t] = 0;
        // epilogue operands, loaded before the weight stream starts
        e_rs[t] = rowsum[m0 + t];
        e_gs[t] = out.acc ? 0.0 : epi_gs(out.gamma[0], out.scale[m0 + t]);
    }

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
        if (lane != 0) continue;
        const int32_t a = v - e_rs[t];
        if (out.acc)
            out.acc[(m0 + t) * ldy + row] = a;
        else
            out.y[(m0 + t) * ldy + row] = epi_y(a, e_gs[t]);
    }
}

// ---- base-3 layout, one token: table decode ----------------------------------
// A 243-entry table in LDS maps a packed byte to its five codes (digits) in
// byte lanes (entry.x = digits 0..3, entry.y = digit 4).  Four packed bytes
// (20 trits) are decoded by four table reads and a 4 x 4 byte transpose
// (v_perm), which leaves digit i of the four bytes in one dword D_i; the
// activations of the same 20 k are prearranged once per block into dwords X_i
// holding x[5j + i] for j = 0..3, so the 20 products are five dot4s.
// Block layout as in the 2-bit kernel: ks x wr waves, lanes own up to two
// 16-byte chunks (80 trits) of every row of the block.
__device__ inline uint32_t perm_b(uint32_t a, uint32_t b, uint32_t sel)
{
    return __builtin_amdgcn_perm(a, b, sel);
}

// X[g][i] for group g (20 k) of an 80-activation chunk: bytes x[20g + 5j + i].
__device__ inline void arrange_x80(const uint32_t (&r)[20], uint32_t (&X)[4][5])
{
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            uint32_t v = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int idx = 20 * g + 5 * j + i;
                v |= ((r[idx >> 2] >> (8 * (idx & 3))) & 0xFFu) << (8 * j);
            }
            X[g][i] = v;
        }
}

// sum over the 20 trits of packed word w (4 bytes) against X[5].
__device__ inline int dot_word3(uint32_t w, const uint32_t (&X)[5], const uint2 *lut)
{
    const uint2 e0 = lut[w & 0xFFu], e1 = lut[(w >> 8) & 0xFFu];
    const uint2 e2 = lut[(w >> 16) & 0xFFu], e3 = lut[w >> 24];
    const uint32_t t01l = perm_b(e1.x, e0.x, 0x05010400u), t01h = perm_b(e1.x, e0.x, 0x07030602u);
    const uint32_t t23l = perm_b(e3.x, e2.x, 0x05010400u), t23h = perm_b(e3.x, e2.x, 0x07030602u);
    const uint32_t d0 = perm_b(t23l, t01l, 0x05040100u), d1 = perm_b(t23l, t01l, 0x07060302u);
    const uint32_t d2 = perm_b(t23h, t01h, 0x05040100u), d3 = perm_b(t23h, t01h, 0x07060302u);
    const uint32_t u01 = perm_b(e1.y, e0.y, 0x05010400u), u23 = perm_b(e3.y, e2.y, 0x05010400u);
    const uint32_t d4 = perm_b(u23, u01, 0x05040100u);
    int a = __builtin_amdgcn_sdot4((int)d0, (int)X[0], 0, false);
    a = __builtin_amdgcn_sdot4((int)d1, (int)X[1], a, false);
    a = __builtin_amdgcn_sdot4((int)d2, (int)X[2], a, false);
    a = __builtin_amdgcn_sdot4((int)d3, (int)X[3], a, false);
    return __builtin_amdgcn_sdot4((int)d4, (int)X[4], a, false);
}

template <int CPL, int ST>
__global__ __launch_bounds__(GEMV_KS_MAX * 64) void gemv3lut_kernel(
    const int8_t *__restrict__ xq, const int32_t *__restrict__ rowsum, int64_t k,
    const uint4 *__restrict__ packed, int64_t n, int64_t chunks, int64_t share, Out out,
    int64_t ldy, int64_t m0, int ks)
{
    constexpr int R = GEMV_R, RB = GEMV_R * ST;
    __shared__ uint2 lut[256];
    __shared__ int part[GEMV_KS_MAX][GEMV_KS_MAX * RB];
    const int wr = (int)(blockDim.x >> 6) / ks;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kw = wave % ks, rw = wave / ks;
    const int64_t blk0 = (int64_t)blockIdx.x * wr * RB;
    const int64_t row0 = blk0 + (int64_t)rw * RB;

    for (int b = threadIdx.x; b < 243; b += blockDim.x) {
        uint32_t v = (uint32_t)b, lo = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            lo |= (v % 3u) << (8 * i);
            v /= 3u;
        }
        lut[b] = make_uint2(lo, v);
    }

    int64_t coff[CPL];
    bool ok[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int64_t c = kw * share + lane + 64 * j;
        ok[j] = (lane + 64 * j < share) && c < chunks;
        coff[j] = ok[j] ? c : 0;
    }

    uint4 w[2][R][CPL];
    auto load = [&](uint4(&wb)[R][CPL], int s) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            int64_t row = row0 + s * R + r;
            row = row < n ? row : n - 1;
#pragma unroll
            for (int j = 0; j < CPL; ++j) wb[r][j] = load_nt16(packed + row * chunks + coff[j]);
        }
    };
    load(w[0], 0);
    __builtin_amdgcn_sched_barrier(0);

    const int e_rr = threadIdx.x;
    int32_t e_rs = 0;
    double e_gs = 0.0;
    if (threadIdx.x < wr * RB) {
        e_rs = rowsum[m0];
        if (!out.acc) e_gs = epi_gs(out.gamma[0], out.scale[m0]);
    }

    // Activations of this lane's chunks (80 each), prearranged; pieces past K
    // (K a multiple of 16) and chunks the lane does not own are zero.
    uint32_t X[CPL][4][5];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        uint32_t r[20];
        const int64_t k0 = 80 * coff[j];
#pragma unroll
        for (int d = 0; d < 5; ++d) {
            uint4 v = zero4();
            if (ok[j] && k0 + 16 * d < k) v = load16(xq + m0 * k + k0 + 16 * d);
            r[4 * d] = v.x; r[4 * d + 1] = v.y; r[4 * d + 2] = v.z; r[4 * d + 3] = v.w;
        }
        arrange_x80(r, X[j]);
    }
    __syncthreads();   // table ready

#pragma unroll
    for (int s = 0; s < ST; ++s) {
        if (s + 1 < ST) load(w[(s + 1) & 1], s + 1);
        __builtin_amdgcn_sched_barrier(0);
        const int b = s & 1;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            int a = 0;
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                a += dot_word3(w[b][r][j].x, X[j][0], lut);
                a += dot_word3(w[b][r][j].y, X[j][1], lut);
                a += dot_word3(w[b][r][j].z, X[j][2], lut);
                a += dot_word3(w[b][r][j].w, X[j][3], lut);
            }
            const int v = wave_sum_dpp(a);
            if (lane == 63) part[kw][rw * RB + s * R + r] = v;
        }
    }
    __syncthreads();
    if (threadIdx.x < wr * RB && blk0 + e_rr < n) {
        int sum = 0;
        for (int q = 0; q < ks; ++q) sum += part[q][e_rr];
        const int32_t acc = sum - e_rs;
        const int64_t idx = m0 * ldy + blk0 + e_rr;
        if (out.acc)
            out.acc[idx] = acc;
        else
            out.y[idx] = epi_y(acc, e_gs);
    }
}

// Launch shape of the 2-bit GEMV for (N, K): waves per block KS (so that each
// lane holds at most 2 chunks of activations per token), chunks per lane CPL,
// and steps per block ST (a power of two, about 1792 waves in total; with the
// int8 token staged once per block in LDS, about 7168 waves, or 1024 when
// rows are long enough for four waves each, which then share a longer token;
// the kernel that quantises the token in every block has its own shape,
// gemv2_fused_shape).
// Row waves per block WR: blocks of about four waves (fewer, larger
// workgroups dispatch faster, and their outputs are stored together).
struct Gemv2Shape { int ks, cpl, st; int64_t share; int wr; };

Gemv2Shape gemv2_shape(int64_t n, int64_t chunks, int mt, bool token_in_lds = false)
{
    // Two chunks per lane halve the waves per row; on short matrices with up
    // to 128 chunks per row the extra waves of one chunk per lane are faster
    // (measured on the 2B-class down projection, K = 6912).
    int cpl_max = mt <= 2 ? 2 : 1;
    if (chunks <= 128 && n * ((chunks + 63) / 64) <= 8192) cpl_max = 1;
    int ks = (int)((chunks + 64 * cpl_max - 1) / (64 * cpl_max));
    if (ks > GEMV_KS_MAX) ks = GEMV_KS_MAX;
    const int64_t share = (chunks + ks - 1) / ks;
    const int cpl = (int)((share + 63) / 64);
    const int64_t waves = token_in_lds ? (ks >= 4 ? 1024 : 7168) : 1792;
    int64_t per = n * ks / (GEMV_R * waves);
    int st = 1;
    while (st < 8 && 2 * st <= per) st *= 2;
    int wr = ks >= GEMV_WAVES ? 1 : GEMV_WAVES / ks;
    while (wr > 1 && (n + (int64_t)wr * GEMV_R * st - 1) / ((int64_t)wr * GEMV_R * st) < 256) wr /= 2;
    return {ks, cpl, st, share, wr};
}

// Shape of the kernel that quantises the token in every block: the same
// k split, but blocks of up to 8 waves and as many rows per block as still
// give about one block per CU, since every block repeats the quantisation
// (measured on the 2B-class decode matrices).
Gemv2Shape gemv2_fused_shape(int64_t n, int64_t chunks)
{
    Gemv2Shape sh = gemv2_shape(n, chunks, 1);
    auto blocks = [&](int wr, int st) { return (n + (int64_t)wr * GEMV_R * st - 1) / ((int64_t)wr * GEMV_R * st); };
    sh.wr = GEMV_KS_MAX / sh.ks;
    while (sh.wr > 1 && blocks(sh.wr, 1) < 160) sh.wr /= 2;
    sh.st = 1;
    while (sh.st < 8 && blocks(sh.wr, 2 * sh.st) >= 160) sh.st *= 2;
    return sh;
}

template <int MT, int CPL, int ST>
hipError_t launch2_st(bool al, const int8_t *xq, const int32_t *rowsum, int64_t n, int64_t k,
                      const uint8_t *packed, Out out, int64_t m0, const Gemv2Shape &sh,
                      hipStream_t s)
{
    const int64_t chunks = pack2_pitch(k) / 16;
    const int64_t rb = (int64_t)GEMV_R * ST * sh.wr;
    const dim3 grid((unsigned)((n + rb - 1) / rb)), block((unsigned)(64 * sh.ks * sh.wr));
    // one token: staged once per block in LDS (up to 8 vectors per thread)
    const int64_t per = (k / 16 + 64 * sh.ks * sh.wr - 1) / (64 * sh.ks * sh.wr);
    if (MT == 1 && al && k <= GEMV_X_LDS_MAX_K && per <= 8) {
        const size_t lds = (size_t)((k + 15) / 16) * 16;
#define X_CASE(V_)                                                                              \
        if (per <= V_) {                                                                        \
            hipLaunchKernelGGL((gemv2_kernel<1, CPL, ST, true, GEMV_X_LDS, V_>), grid, block,    \
                               lds, s, xq, rowsum, k, (const uint4 *)packed, n, chunks,         \
                               sh.share, out, n, m0, sh.ks, FuseQ{});                           \
            return hipGetLastError();                                                           \
        }
        X_CASE(1) X_CASE(2) X_CASE(4) X_CASE(8)
#undef X_CASE
    }
    if (al)
        hipLaunchKernelGGL((gemv2_kernel<MT, CPL, ST, true>), grid, block, 0, s, xq, rowsum, k,
                           (const uint4 *)packed, n, chunks, sh.share, out, n, m0, sh.ks,
                           FuseQ{});
    else
        hipLaunchKernelGGL((gemv2_kernel<MT, CPL, ST, false>), grid, block, 0, s, xq, rowsum, k,
                           (const uint4 *)packed, n, chunks, sh.share, out, n, m0, sh.ks,
                           FuseQ{});
    return hipGetLastError();
}

// Fused one-token launches: input vectors per thread (VPT) from the token
// length and the block size.
constexpr int GEMV_FUSED_VPT_MAX = 16;

template <int CPL, int ST, int QDT, int VPT>
hipError_t launch2_fused_vpt(const FuseQ &fq, int64_t n, int64_t k, const uint8_t *packed,
                             Out out, const Gemv2Shape &sh, hipStream_t s)
{
    const int64_t chunks = pack2_pitch(k) / 16;
    const int64_t rb = (int64_t)GEMV_R * ST * sh.wr;
    const dim3 grid((unsigned)((n + rb - 1) / rb)), block((unsigned)(64 * sh.ks * sh.wr));
    const size_t lds = (size_t)((k + 15) / 16) * 16;
    hipLaunchKernelGGL((gemv2_kernel<1, CPL, ST, true, QDT, VPT>), grid, block, lds, s,
                       (const int8_t *)nullptr, (const int32_t *)nullptr, k,
                       (const uint4 *)packed, n, chunks, sh.share, out, n, (int64_t)0, sh.ks, fq);
    return hipGetLastError();
}

template <int CPL, int ST, int QDT>
hipError_t launch2_fused_dt(const FuseQ &fq, int64_t n, int64_t k, const uint8_t *packed,
                            Out out, const Gemv2Shape &sh, hipStream_t s)
{
    const int64_t nvec = k / (QDT == DT_BF16 ? 8 : 4), nthr = 64 * sh.ks * sh.wr;
    const int64_t per = (nvec + nthr - 1) / nthr;
    if (per <= 2) return launch2_fused_vpt<CPL, ST, QDT, 2>(fq, n, k, packed, out, sh, s);
    if (per <= 4) return launch2_fused_vpt<CPL, ST, QDT, 4>(fq, n, k, packed, out, sh, s);
    if (per <= 8) return launch2_fused_vpt<CPL, ST, QDT, 8>(fq, n, k, packed, out, sh, s);
    return launch2_fused_vpt<CPL, ST, QDT, 16>(fq, n, k, packed, out, sh, s);
}

template <int CPL, int ST>
hipError_t launch2_fused_st(int dtype, const FuseQ &fq, int64_t n, int64_t k,
                            const uint8_t *packed, Out out, const Gemv2Shape &sh, hipStream_t s)
{
    if (dtype == DT_BF16) return launch2_fused_dt<CPL, ST, DT_BF16>(fq, n, k, packed, out, sh, s);
    return launch2_fused_dt<CPL, ST, DT_F32>(fq, n, k, packed, out, sh, s);
}

template <int CPL>
hipError_t launch2_fused_cpl(int dtype, const FuseQ &fq, int64_t n, int64_t k,
                             const uint8_t *packed, Out out, const Gemv2Shape &sh, hipStream_t s)
{
    switch (sh.st) {
    case 1: return launch2_fused_st<CPL, 1>(dtype, fq, n, k, packed, out, sh, s);
    case 2: return launch2_fused_st<CPL, 2>(dtype, fq, n, k, packed, out, sh, s);
    case 4: return launch2_fused_st<CPL, 4>(dtype, fq, n, k, packed, out, sh, s);
    default: return launch2_fused_st<CPL, 8>(dtype, fq, n, k, packed, out, sh, s);
    }
}

template <int MT, int CPL>
hipError_t launch2_cpl(bool al, const int8_t *xq, const int32_t *rowsum, int64_t n, int64_t k,
                       const uint8_t *packed, Out out, int64_t m0, const Gemv2Shape &sh,
                       hipStream_t s)
{
    switch (sh.st) {
    case 1: return launch2_st<MT, CPL, 1>(al, xq, rowsum, n, k, packed, out, m0, sh, s);
    case 2: return launch2_st<MT, CPL, 2>(al, xq, rowsum, n, k, packed, out, m0, sh, s);
    case 4: return launch2_st<MT, CPL, 4>(al, xq, rowsum, n, k, packed, out, m0, sh, s);
    default: return launch2_st<MT, CPL, 8>(al, xq, rowsum, n, k, packed, out, m0, sh, s);
    }
}

template <int MT>
hipError_t launch2(bool al, const int8_t *xq, const int32_t *rowsum, int64_t n, int64_t k,
                   const uint8_t *packed, Out out, int64_t m0, hipStream_t s)
{
    const Gemv2Shape sh =
        gemv2_shape(n, pack2_pitch(k) / 16, MT, MT == 1 && al && k <= GEMV_X_LDS_MAX_K);
    if (sh.cpl == 1) return launch2_cpl<MT, 1>(al, xq, rowsum, n, k, packed, out, m0, sh, s);
    return launch2_cpl<MT, 2>(al, xq, rowsum, n, k, packed, out, m0, sh, s);
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


// ---- one token with the decoder block's glue inside (prologue / epilogue) ----
// Every block forms the token's pre-norm values v itself (NORM_RESIDUAL: the
// residual stream plus the previous product's output, the sum stored once by
// block 0; NORM_GQA: the value vectors of the first token's attention,
// expanded over the query heads; NORM_F64: double values from a squared-ReLU
// epilogue), applies RMSNorm with unit gain in double precision, rounds to
// float and quantises with the activation quantiser's arithmetic into an LDS
// copy of the int8 token; then the 2-bit GEMV of the block's rows runs as in
// gemv2_kernel.  RELU2: the weight rows are taken as interleaved pairs,
// logical row 2i = gate row i and 2i + 1 = up row i of the packed up/gate
// matrix, and the block writes v[i] = relu(y_gate)^2 * y_up in double (y as
// the product would store it) instead of y.
template <int PRO, bool RELU2, int CPL, int ST, int EPT>
__global__ __launch_bounds__(GEMV_KS_MAX * 64) void gemv_norm_kernel(
    NormArgs a, int64_t k, const uint4 *__restrict__ packed, int64_t n, int64_t chunks,
    int64_t share, Out out, int ks)
{
    constexpr int R = GEMV_R, RB = GEMV_R * ST;
    __shared__ int part[GEMV_KS_MAX][GEMV_KS_MAX * RB];
    __shared__ double red_d[GEMV_KS_MAX], red_vm[GEMV_KS_MAX];
    __shared__ int red_i[GEMV_KS_MAX];
    extern __shared__ uint4 q_lds[];   // the int8 token, K bytes (rounded up to 16)
    const int nthr = (int)blockDim.x, nw = nthr >> 6;
    const int wr = nw / ks;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kw = wave % ks, rw = wave / ks;
    const int64_t blk0 = (int64_t)blockIdx.x * wr * RB;
    const int64_t row0 = blk0 + (int64_t)rw * RB;
    const int kk = (int)k;

    int64_t coff[CPL];
    bool ok[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int64_t c = kw * share + lane + 64 * j;
        ok[j] = (lane + 64 * j < share) && c < chunks;
        coff[j] = ok[j] ? c : 0;
    }
    // logical row -> packed row (RELU2: gate / up pairs)
    auto phys = [&](int64_t row) __attribute__((always_inline)) {
        row = row < n ? row : n - 1;
        return RELU2 ? ((row & 1) ? a.f + (row >> 1) : (row >> 1)) : row;
    };
    constexpr int PF = GEMV_PF < ST ? GEMV_PF : ST;
    uint4 w[PF + 1][R][CPL];
    auto load = [&](uint4(&wb)[R][CPL], int s) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t row = phys(row0 + s * R + r);
#pragma unroll
            for (int j = 0; j < CPL; ++j) wb[r][j] = load_nt16(packed + row * chunks + coff[j]);
        }
    };
    // The token's loads go out first, then the first steps' weight loads, and
    // only then is anything computed from the token (an addition or a
    // conversion before the weight loads would wait for the token first);
    // block 0's copy of the new residual is stored after all loads are issued.
    double v[EPT];
    float xo[EPT], ad[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int i = threadIdx.x + nthr * j, ic = i < kk ? i : kk - 1;
        if (PRO == NORM_RESIDUAL) {
            xo[j] = ((const float *)a.src)[ic];
        } else if (PRO == NORM_GQA) {
            const unsigned hd = (unsigned)a.head_dim, head = (unsigned)ic / hd;
            const unsigned d = (unsigned)ic - head * hd;
            xo[j] = ((const float *)a.src)[a.col + (int64_t)(head / (unsigned)a.group) * hd + d];
        } else {
            v[j] = ((const double *)a.src)[ic];
        }
    }
    if (PRO == NORM_RESIDUAL && a.add)
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
            const int i = threadIdx.x + nthr * j;
            ad[j] = a.add[i < kk ? i : kk - 1];
        }
    // gamma goes out after the token, before the weights (a vector load):
    // read in the epilogue, its latency would follow the block's last barrier
    const float gamma = __uint_as_float(vload_u32(out.gamma));
#pragma unroll
    for (int q = 0; q < PF; ++q) load(w[q], q);
    __builtin_amdgcn_sched_barrier(0);
    if (PRO == NORM_RESIDUAL && a.add)
#pragma unroll
        for (int j = 0; j < EPT; ++j) xo[j] += ad[j];
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        if (PRO != NORM_F64) v[j] = (double)xo[j];
        if ((int)threadIdx.x + nthr * j >= kk) v[j] = 0.0;
    }
    if (PRO == NORM_RESIDUAL && a.add && blockIdx.x == 0)
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
            const int i = threadIdx.x + nthr * j;
            if (i < kk) a.x_out[i] = xo[j];
        }

    // RMSNorm: sum of squares in double over the block, with max |v| in the
    // same reduction (the quantiser's max |h| follows from it exactly)
    double ss = 0.0, vm = 0.0;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        ss += v[j] * v[j];
        vm = fmax(vm, fabs(v[j]));
    }
    block_ss_vmax(ss, vm, red_d, red_vm, nw);
    const double inv = 1.0 / sqrt(ss / (double)k + a.eps);
    float h[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) h[j] = (float)(v[j] * inv);
    const float amax = vm > 0.0 ? (float)(vm * inv) : 0.0f;
    const float qs = act_scale(amax);
    int sum = 0;
    int8_t *ql = (int8_t *)q_lds;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int i = threadIdx.x + nthr * j;
        if (i >= kk) continue;
        const int8_t q = quant1(h[j], qs);
        sum += q;
        ql[i] = q;
        if (a.xq && blockIdx.x == 0) a.xq[i] = q;
    }
    // zero the pad bytes of the last 16-byte piece
    if ((int)threadIdx.x < (16 - (kk & 15)) % 16) ql[kk + threadIdx.x] = 0;
    sum = wave_sum_dpp(sum);
    if (lane == 63) red_i[wave] = sum;
    __syncthreads();
    int e_rs = 0;
    for (int q = 0; q < nw; ++q) e_rs += red_i[q];
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (a.scale) a.scale[0] = qs;
        if (a.rowsum) a.rowsum[0] = e_rs;
    }

    uint4 xv[CPL][4];
#pragma unroll
    for (int j = 0; j < CPL; ++j)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const int64_t e0 = 64 * coff[j] + 16 * d;
            xv[j][d] = (ok[j] && e0 < k) ? nibble_split(q_lds[e0 / 16]) : zero4();
        }
    // gamma / s, formed here: gamma (a vector load issued before the weights)
    // has arrived by the time the first weights have
    const double gs = epi_gs(gamma, qs);

#pragma unroll
    for (int s = 0; s < ST; ++s) {
        if (s + PF < ST) load(w[(s + PF) % (PF + 1)], s + PF);
        __builtin_amdgcn_sched_barrier(0);
        const int b = s % (PF + 1);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            int ah = 0;
            uint32_t al = 0;
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                dot8_word(w[b][r][j].x, xv[j][0], ah, al);
                dot8_word(w[b][r][j].y, xv[j][1], ah, al);
                dot8_word(w[b][r][j].z, xv[j][2], ah, al);
                dot8_word(w[b][r][j].w, xv[j][3], ah, al);
            }
            const int vsum = wave_sum_dpp(16 * ah + (int)al);
            if (lane == 63) part[kw][rw * RB + s * R + r] = vsum;
        }
    }
    __syncthreads();
    const int nout = wr * RB;
    const int e_rr = threadIdx.x;
    if (RELU2) {
        // thread e_rr < nout / 2 finishes the pair of logical rows 2 e_rr, 2 e_rr + 1
        if (e_rr < nout / 2 && blk0 + 2 * e_rr + 1 < n) {
            int sg = 0, su = 0;
            for (int q = 0; q < ks; ++q) {
                sg += part[q][2 * e_rr];
                su += part[q][2 * e_rr + 1];
            }
            const float yg = epi_y(sg - e_rs, gs), yu = epi_y(su - e_rs, gs);
            const double gd = yg > 0.0f ? (double)yg : 0.0;
            a.v[(blk0 >> 1) + e_rr] = gd * gd * (double)yu;
        }
    } else if (e_rr < nout && blk0 + e_rr < n) {
        int vsum = 0;
        for (int q = 0; q < ks; ++q) vsum += part[q][e_rr];
        out.y[blk0 + e_rr] = epi_y(vsum - e_rs, gs);
    }
}

template <int PRO, bool RELU2, int CPL, int ST>
hipError_t launch_norm_ept(const NormArgs &a, int64_t n, int64_t k, const uint8_t *packed,
                           Out out, const Gemv2Shape &sh, hipStream_t s)
{
    const int64_t chunks = pack2_pitch(k) / 16;
    const int64_t rb = (int64_t)GEMV_R * ST * sh.wr;
    const dim3 grid((unsigned)((n + rb - 1) / rb)), block((unsigned)(64 * sh.ks * sh.wr));
    const size_t lds = (size_t)((k + 15) / 16) * 16;
    const int64_t per = (k + 64 * sh.ks * sh.wr - 1) / (64 * sh.ks * sh.wr);
#define NORM_CASE(E_)                                                                           \
    if (per <= E_) {                                                                            \
        hipLaunchKernelGGL((gemv_norm_kernel<PRO, RELU2, CPL, ST, E_>), grid, block, lds, s, a, \
                           k, (const uint4 *)packed, n, chunks, sh.share, out, sh.ks);          \
        return hipGetLastError();                                                               \
    }
    NORM_CASE(4) NORM_CASE(8) NORM_CASE(16) NORM_CASE(32)
#undef NORM_CASE
    return hipErrorInvalidValue;
}

template <int PRO, bool RELU2, int CPL>
hipError_t launch_norm_cpl(const NormArgs &a, int64_t n, int64_t k, const uint8_t *packed,
                           Out out, const Gemv2Shape &sh, hipStream_t s)
{
    switch (sh.st) {
    case 1: return launch_norm_ept<PRO, RELU2, CPL, 1>(a, n, k, packed, out, sh, s);
    case 2: return launch_norm_ept<PRO, RELU2, CPL, 2>(a, n, k, packed, out, sh, s);
    case 4: return launch_norm_ept<PRO, RELU2, CPL, 4>(a, n, k, packed, out, sh, s);
    default: return launch_norm_ept<PRO, RELU2, CPL, 8>(a, n, k, packed, out, sh, s);
    }
}

template <int PRO, bool RELU2>
hipError_t launch_norm_pro(const NormArgs &a, int64_t n, int64_t k, const uint8_t *packed,
                           Out out, hipStream_t s)
{
    const Gemv2Shape sh = gemv2_fused_shape(n, pack2_pitch(k) / 16);
    if (sh.cpl == 1) return launch_norm_cpl<PRO, RELU2, 1>(a, n, k, packed, out, sh, s);
    return launch_norm_cpl<PRO, RELU2, 2>(a, n, k, packed, out, sh, s);
}

}  // namespace

hipError_t launch_gemv_pack2(const int8_t *xq, const int32_t *rowsum, int64_t m,
                             const uint8_t *packed, int64_t n, int64_t k, Out out, hipStream_t s)
{
    const bool al = (k % 16) == 0;
    const int64_t chunks = pack2_pitch(k) / 16;
    if (chunks > (int64_t)GEMV_KS_MAX * 128) {
        const dim3 grid((unsigned)((n + 3) / 4)), block(256);
        if (al)
            hipLaunchKernelGGL((gemv2_long_kernel<true>), grid, block, 0, s, xq, rowsum, k,
                               (const uint4 *)packed, n, chunks, out, n, m);
        else
            hipLaunchKernelGGL((gemv2_long_kernel<false>), grid, block, 0, s, xq, rowsum, k,
                               (const uint4 *)packed, n, chunks, out, n, m);
        return hipGetLastError();
    }
    for (int64_t m0 = 0; m0 < m; m0 += 4) {
        const int64_t mt = (m - m0) < 4 ? (m - m0) : 4;
        hipError_t e;
        switch (mt) {
        case 1: e = launch2<1>(al, xq, rowsum, n, k, packed, out, m0, s); break;
        case 2: e = launch2<2>(al, xq, rowsum, n, k, packed, out, m0, s); break;
        case 3: e = launch2<3>(al, xq, rowsum, n, k, packed, out, m0, s); break;
        default: e = launch2<4>(al, xq, rowsum, n, k, packed, out, m0, s); break;
        }
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

bool gemv_fused_supported(int64_t m, int64_t n, int64_t k, int dtype)
{
    // one token, whole 16-value pieces, the int8 token within 16 KB of LDS and
    // at most 16 input vectors per thread
    if (m != 1 || n < 1 || k % 16 != 0 || k > 16384) return false;
    const Gemv2Shape sh = gemv2_fused_shape(n, pack2_pitch(k) / 16);
    const int64_t nvec = k / (dtype == DT_BF16 ? 8 : 4), nthr = 64 * sh.ks * sh.wr;
    return nvec <= nthr * GEMV_FUSED_VPT_MAX;
}

hipError_t launch_gemv_pack2_fused(const void *x, int dtype, int8_t *xq, float *scale,
                                   int32_t *rowsum, const uint8_t *packed, int64_t n, int64_t k,
                                   Out out, hipStream_t s)
{
    if (!gemv_fused_supported(1, n, k, dtype) || out.acc) return hipErrorInvalidValue;
    const FuseQ fq{x, xq, scale, rowsum};
    const Gemv2Shape sh = gemv2_fused_shape(n, pack2_pitch(k) / 16);
    if (sh.cpl == 1) return launch2_fused_cpl<1>(dtype, fq, n, k, packed, out, sh, s);
    return launch2_fused_cpl<2>(dtype, fq, n, k, packed, out, sh, s);
}

int64_t gemv3_workspace_bytes(int64_t m, int64_t n, int64_t k)
{
    return gemv3sum_workspace_bytes(m, n, k);
}

hipError_t launch_gemv_pack3(const int8_t *xq, const int32_t *rowsum, int64_t m,
                             const uint8_t *packed, int64_t n, int64_t k, Out out, void *ws,
                             hipStream_t s)
{
    // one token: the digit table where it runs (K a multiple of 16; measured
    // faster than the partial-sum tables on the 70B-class matrices), else the
    // partial-sum tables on matrices of many rows
    if (gemv3lut_supported(m, k)) return launch_gemv3lut(xq, rowsum, packed, n, k, out, s);
    if (gemv3sum_slices(m, n, k) > 0)
        return launch_gemv3sum(xq, rowsum, packed, n, k, out, (int32_t *)ws, s);
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

bool gemv3lut_supported(int64_t m, int64_t k)
{
    return m == 1 && (k % 16) == 0 && pack3_pitch(k) / 16 <= (int64_t)GEMV_KS_MAX * 128;
}

hipError_t launch_gemv3lut(const int8_t *xq, const int32_t *rowsum, const uint8_t *packed,
                           int64_t n, int64_t k, Out out, hipStream_t s)
{
    const int64_t chunks3 = pack3_pitch(k) / 16;
    {
        // one token: table decode, shaped like the 2-bit kernel; rows of at
        // most 128 chunks take one chunk per lane (twice the waves, half the
        // registers each: 70B-class K = 8192 18.8 -> 17.6 us; on K = 28672,
        // 359 chunks, two chunks per lane stay faster: 16.3 against 18.3 us)
        const Gemv2Shape sh = gemv2_shape(n, chunks3, chunks3 <= 128 ? 3 : 1);
        const int64_t rb = (int64_t)GEMV_R * sh.st * sh.wr;
        const dim3 grid((unsigned)((n + rb - 1) / rb)), block((unsigned)(64 * sh.ks * sh.wr));
        const uint4 *pk = (const uint4 *)packed;
#define G3_CASE(CPL_, ST_)                                                                      \
        if (sh.cpl == CPL_ && sh.st == ST_) {                                                   \
            hipLaunchKernelGGL((gemv3lut_kernel<CPL_, ST_>), grid, block, 0, s, xq, rowsum, k,  \
                               pk, n, chunks3, sh.share, out, n, (int64_t)0, sh.ks);            \
            return hipGetLastError();                                                           \
        }
        G3_CASE(1, 1) G3_CASE(1, 2) G3_CASE(1, 4) G3_CASE(1, 8)
        G3_CASE(2, 1) G3_CASE(2, 2) G3_CASE(2, 4) G3_CASE(2, 8)
#undef G3_CASE
        return hipErrorInvalidValue;
    }
}

}  // namespace bl

namespace bl {

bool gemv_norm_supported(int64_t n, int64_t k)
{
    if (n < 1 || k < 1 || k > NORM_MAX_K) return false;
    const Gemv2Shape sh = gemv2_fused_shape(n, pack2_pitch(k) / 16);
    return k <= (int64_t)64 * sh.ks * sh.wr * 32;
}

hipError_t launch_gemv_norm(const NormArgs &a, int64_t n, int64_t k, const uint8_t *packed,
                            Out out, bool relu2, hipStream_t s)
{
    if (!gemv_norm_supported(n, k)) return hipErrorInvalidValue;
    if (relu2) {
        if (a.pro == NORM_RESIDUAL) return launch_norm_pro<NORM_RESIDUAL, true>(a, n, k, packed, out, s);
        if (a.pro == NORM_GQA) return launch_norm_pro<NORM_GQA, true>(a, n, k, packed, out, s);
        return launch_norm_pro<NORM_F64, true>(a, n, k, packed, out, s);
    }
    if (a.pro == NORM_RESIDUAL) return launch_norm_pro<NORM_RESIDUAL, false>(a, n, k, packed, out, s);
    if (a.pro == NORM_GQA) return launch_norm_pro<NORM_GQA, false>(a, n, k, packed, out, s);
    return launch_norm_pro<NORM_F64, false>(a, n, k, packed, out, s);
}

}  // namespace bl
