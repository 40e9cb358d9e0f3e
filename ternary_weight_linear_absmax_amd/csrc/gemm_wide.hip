// Ternary x int8 GEMM for prefill-sized products: wide block tiles on the
// gfx950 int8 matrix cores, packed weights straight from memory to registers.
//
// Source: asi.tokyo BitNet b1.58 2B4T article, packing paragraph (trits packed
// four per byte, unpacked beside the arithmetic units, multiplied with 8-bit
// activations) and its closing remark that today's hardware runs ternary
// weights as int8.  The unit is v_mfma_i32_32x32x32_i8.
//
// Operand layout of v_mfma_i32_32x32x32_i8 (lane l, h = l / 32):
//   A: 16 bytes = A[i = l % 32][16 k-values], B: 16 bytes = B[16 k-values][j = l % 32],
//   D: register r = D[i = 8(r/4) + 4h + r%4][j = l % 32].
// Which physical k a lane's 16 values stand for is free as long as A and B
// agree.  Here, in a stage of 128 k at k0, step p = 0..3 gives lane half h the
// k-values k0 + 64h + 16p .. +15: for B that is packed word p of the 16 bytes
// k0/4 + 16h .. +15 of the lane's weight row (one 16-byte load covers a whole
// stage), unpacked as (w >> 2i) & 0x03030303, i = 0..3 (the codes t + 1 of
// four consecutive k in each register); for A it is bytes 64h + 16p .. +15 of
// the token row in the stage's LDS tile.
//
// Block: four waves side by side, each owning a 64 x 128 output tile (two
// 32-row blocks x four 32-column blocks: eight MFMAs per k step, every unpacked
// weight operand used twice, every activation fragment four times), so the
// block tile is 64 tokens x 512 weight rows and the block's activation tile
// (64 x 128 bytes per stage) is loaded from memory once and read from LDS by
// all four waves.  The packed weights never touch LDS: each lane loads its 16
// bytes per stage into a register ring NB stages ahead, through the caches
// (each weight tile is read again by the other token tiles).  Activations go
// through a two-slot register ring into a double-buffered LDS tile (one
// barrier per stage); the next stage's fragments are read from LDS while the
// current stage's MFMAs run.
//
// The B operand carries the codes t + 1; the epilogue subtracts the token's
// row sum of q (exact integer arithmetic), then rescales by gamma / s.  The
// finished 64 x 128 tile of a wave leaves through a wave-private LDS area in
// two halves of 32 rows, written in the MFMA register layout and read back
// along rows, so every lane stores 16 contiguous bytes.
//
// Split-K: S > 1 slices of the k range store their int32 partial tiles in
// their own slice of the workspace [S][M][N] (plain stores, no atomics); the
// split-k finish kernel adds them in slice order and applies the epilogue.
#include "internal.h"

namespace bl {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int WBK = 128;              // k per stage
constexpr int WBM = 64;               // tokens per block
constexpr int WLDA = WBK + 16;        // padded LDS row of the activation tile (bytes)
#ifndef WIDE_NB
#define WIDE_NB 4
#endif
#ifndef WIDE_B_NT
#define WIDE_B_NT 0
#endif
#ifndef WIDE_NA
#define WIDE_NA 2
#endif
constexpr int WNA = WIDE_NA;          // activation register ring (stages)
constexpr int WNB = WIDE_NB;          // weight register ring (stages)
constexpr int WNXCD = 8;
// WWN 32-column blocks per wave: the block tile is 64 x 128 WWN
template <int WWN> constexpr int wbn() { return 4 * 32 * WWN; }
template <int WWN> constexpr int wepl() { return 32 * WWN + 4; }   // epilogue LDS row (ints)

enum : int { WEP_PARTIAL = 0, WEP_ACC = 1, WEP_Y = 2 };

__device__ inline v4i unpack_w(uint32_t w)
{
    v4i r;
    r[0] = (int)(w & 0x03030303u);
    r[1] = (int)((w >> 2) & 0x03030303u);
    r[2] = (int)((w >> 4) & 0x03030303u);
    r[3] = (int)((w >> 6) & 0x03030303u);
    return r;
}

__device__ inline uint32_t word_p(const uint4 &v, int p)
{
    return p == 0 ? v.x : p == 1 ? v.y : p == 2 ? v.z : v.w;
}

constexpr int lcm_int(int a, int b) { return a / gcd_int(a, b) * b; }

template <int WWN, int KG>
__global__ __launch_bounds__(256 * KG) void gemm_wide_kernel(
    const int8_t *__restrict__ xq, const int32_t *__restrict__ rowsum, int64_t m, int64_t k,
    const uint8_t *__restrict__ packed, int64_t n, int64_t pitch, int tiles_m, int64_t units,
    int64_t per_xcd, int splits, int stages_per, Out out, int64_t ldy, int32_t *__restrict__ ws)
{
    static_assert(KG == 1 || (KG == 2 && WWN == 2), "two k-groups with 64-column waves");
    constexpr int WBN = wbn<WWN>(), WEPL = wepl<WWN>();
    __shared__ __attribute__((aligned(16))) uint8_t a_lds[KG][2][WBM * WLDA];
    __shared__ __attribute__((aligned(16))) int32_t e_lds[4][32 * WEPL];
    // blocks b, b + 8, ... run on one XCD: give each XCD a contiguous range of
    // units (the splits of a tile, then the token tiles of a weight-row
    // block), so that neighbours share activation rows and weight rows in
    // that XCD's L2
    const int64_t u = ((int64_t)blockIdx.x % WNXCD) * per_xcd + (int64_t)blockIdx.x / WNXCD;
    if (u >= units) return;
    const int64_t tile = u / splits;
    const int split = (int)(u % splits);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int kg = wave >> 2, wc = wave & 3, tg = tid & 255;   // k-group, column wave, thread in group
    const int h = lane >> 5, l32 = lane & 31;
    const int tm = (int)(tile % tiles_m);
    const int64_t tn = tile / tiles_m;
    const int64_t m0 = (int64_t)tm * WBM, n0 = tn * WBN;
    const int nk_total = (int)((k + WBK - 1) / WBK);
    const int kt0 = split * stages_per;
    int nk = nk_total - kt0;
    nk = nk < stages_per ? nk : stages_per;
    nk = nk > 0 ? nk : 0;
    // the k-groups take consecutive halves of the slice's stages; both run
    // nloop stages (one barrier each), stages past a group's own range are
    // written as zeros
    const int nloop = (nk + KG - 1) / KG;
    const int g0 = kt0 + kg * nloop;                       // first stage of this group
    int nk_g = nk - kg * nloop;
    nk_g = nk_g < nloop ? nk_g : nloop;
    nk_g = nk_g > 0 ? nk_g : 0;
    const int64_t k_end = (int64_t)(g0 + nk_g) * WBK < k ? (int64_t)(g0 + nk_g) * WBK : k;
    const int ep_mode = splits > 1 ? WEP_PARTIAL : out.acc ? WEP_ACC : WEP_Y;

    v16i acc[2][WWN];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int s = 0; s < WWN; ++s)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][s][r] = 0;

    if (nloop > 0) {
        // per-lane row bases, fixed for the whole k loop (rows clamped into
        // the matrices: clamped rows feed outputs that are never stored)
        uint32_t aoff[2];
        int acol[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int e = tg + 256 * i;
            int64_t gm = m0 + (e >> 3);
            gm = gm < m ? gm : m - 1;
            acol[i] = (e & 7) * 16;
            aoff[i] = (uint32_t)(gm * k + acol[i]);
        }
        uint32_t boff[WWN];
#pragma unroll
        for (int s = 0; s < WWN; ++s) {
            int64_t row = n0 + wc * 32 * WWN + 32 * s + l32;
            row = row < n ? row : n - 1;
            boff[s] = (uint32_t)(row * pitch);
        }
        const int last = nk_g > 0 ? nk_g - 1 : 0;

        // Stage j of the group (clamped to its last one).  Loads use in-row
        // offsets clamped into the row, so every address is valid; activation
        // pieces past the group's range or past K are zeroed when written to
        // LDS, and the weight bytes they meet then contribute nothing.
        auto ld_a = [&](uint4 (&r)[2], int j) __attribute__((always_inline)) {
            const int jj = j < last ? j : last;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                int64_t o = (int64_t)(g0 + jj) * WBK;
                if (o > k - 16 - acol[i]) o = k - 16 - acol[i];
                if (o < -acol[i]) o = -acol[i];
                r[i] = load16(xq + aoff[i] + o);
            }
        };
        auto st_a = [&](uint8_t *buf, const uint4 (&r)[2], int j) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int e = tg + 256 * i;
                uint4 v = r[i];
                if ((int64_t)(g0 + j) * WBK + acol[i] >= k_end) v = make_uint4(0u, 0u, 0u, 0u);
                *(uint4 *)(buf + (e >> 3) * WLDA + (e & 7) * 16) = v;
            }
        };
        auto ld_b = [&](uint4 (&r)[WWN], int j) __attribute__((always_inline)) {
            const int jj = j < last ? j : last;
            int64_t byte = (int64_t)(g0 + jj) * (WBK / 4) + 16 * h;
            byte = byte < pitch - 16 ? byte : pitch - 16;
#pragma unroll
            for (int s = 0; s < WWN; ++s)
                r[s] = WIDE_B_NT ? load_nt16(packed + boff[s] + byte) : load16(packed + boff[s] + byte);
        };
        // this wave's A fragments of one stage: 4 k steps x 2 row blocks
        auto read_frags = [&](v4i (&af)[4][2], const uint8_t *buf) __attribute__((always_inline)) {
#pragma unroll
            for (int p = 0; p < 4; ++p)
#pragma unroll
                for (int a = 0; a < 2; ++a) {
                    const uint4 v = load16(buf + (32 * a + l32) * WLDA + 64 * h + 16 * p);
                    af[p][a] = v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
                }
        };
        auto mma = [&](const v4i (&af)[4][2], const uint4 (&bw)[WWN]) __attribute__((always_inline)) {
#pragma unroll
            for (int p = 0; p < 4; ++p) {
#pragma unroll
                for (int s = 0; s < WWN; ++s) {
                    const v4i bf = unpack_w(word_p(bw[s], p));
#pragma unroll
                    for (int a = 0; a < 2; ++a)
                        acc[a][s] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[p][a], bf, acc[a][s],
                                                                          0, 0, 0);
                }
            }
        };

        uint8_t(&abuf)[2][WBM * WLDA] = a_lds[kg];
        uint4 areg[WNA][2];
        uint4 breg[WNB][WWN];
        v4i af[2][4][2];
#pragma unroll
        for (int j = 0; j < WNB - 1; ++j) ld_b(breg[j], j);
        ld_a(areg[0], 0);
        ld_a(areg[1], 1);
        st_a(abuf[0], areg[0], 0);
        st_a(abuf[1], areg[1], 1);
#pragma unroll
        for (int j = 0; j < WNA; ++j) ld_a(areg[j], 2 + j);
        __syncthreads();
        read_frags(af[0], abuf[0]);
        __syncthreads();   // buffer 0 is rewritten in stage 0

        // Stage j: issue the weight loads of stage j + NB - 1, read the next
        // stage's fragments from LDS, run this stage's MFMAs from registers,
        // write stage j + 2's activations into the buffer this stage's
        // fragments came from, issue the activation loads of stage
        // j + 2 + NA, one barrier.  sched_barrier keeps the phases apart so
        // that no LDS wait lands in front of the MFMAs.
        auto stage = [&](auto jc, int j) __attribute__((always_inline)) {
            constexpr int J = decltype(jc)::value;
            constexpr int C = J & 1;
            ld_b(breg[(J + WNB - 1) % WNB], j + WNB - 1);
            read_frags(af[C ^ 1], abuf[C ^ 1]);
            __builtin_amdgcn_sched_barrier(0);
            mma(af[C], breg[J % WNB]);
            __builtin_amdgcn_sched_barrier(0);
            if (j + 2 < nloop) st_a(abuf[C], areg[J % WNA], j + 2);
            ld_a(areg[J % WNA], j + 2 + WNA);
            __syncthreads();
            __builtin_amdgcn_sched_barrier(0);
        };
        constexpr int U = lcm_int(lcm_int(2, WNA), WNB);
        const int nu = nloop - nloop % U;
        for (int j = 0; j < nu; j += U)
            static_for<U>([&](auto jc) __attribute__((always_inline)) { stage(jc, j + jc); });
        static_for<U - 1>([&](auto jc) __attribute__((always_inline)) {
            if (nu + jc < nloop) stage(jc, nu + jc);
        });
    }
    if constexpr (KG == 2) {
        // the second k-group's sums join the first's through LDS, one 32-row
        // block at a time (the activation buffers are free after the loop)
        int32_t *red = (int32_t *)&a_lds[0][0][0] + wc * (WWN * 16 * 64);
        static_assert(4 * WWN * 16 * 64 * 4 <= KG * 2 * WBM * WLDA, "reduction fits");
#pragma unroll
        for (int a = 0; a < 2; ++a) {
            __syncthreads();
            if (kg == 1) {
#pragma unroll
                for (int s = 0; s < WWN; ++s)
#pragma unroll
                    for (int r = 0; r < 16; ++r) red[(s * 16 + r) * 64 + lane] = acc[a][s][r];
            }
            __syncthreads();
            if (kg == 0) {
#pragma unroll
                for (int s = 0; s < WWN; ++s)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[a][s][r] += red[(s * 16 + r) * 64 + lane];
            }
        }
        if (kg == 1) return;
    }

    // Epilogue through this wave's LDS area, 32 rows at a time: the
    // accumulators go in as written by the MFMA (register r of lane (l32, h)
    // is row 8(r/4) + 4h + r%4, column 32 s + l32), then every lane reads 4
    // consecutive columns of one row and stores 16 bytes.
    int32_t *el = e_lds[wc];
    const int64_t col0 = n0 + wc * 32 * WWN;
    int32_t *dst = ep_mode == WEP_PARTIAL ? ws + (int64_t)split * m * n
                   : ep_mode == WEP_ACC   ? out.acc
                                          : (int32_t *)out.y;
    const int64_t ld = ep_mode == WEP_PARTIAL ? n : ldy;
    const bool vec = (ld % 4) == 0 && ((uintptr_t)dst & 15) == 0;
    const float gamma = ep_mode == WEP_Y ? out.gamma[0] : 0.0f;
#pragma unroll
    for (int a = 0; a < 2; ++a) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = 8 * (r / 4) + 4 * h + (r % 4);
#pragma unroll
            for (int s = 0; s < WWN; ++s) el[row * WEPL + 32 * s + l32] = acc[a][s][r];
        }
        // the wave's lanes exchange values through its LDS area
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // 32 rows x 8 WWN four-column groups: 4 WWN per lane
#pragma unroll 4
        for (int q = 0; q < 4 * WWN; ++q) {
            const int e = lane + 64 * q;
            const int row = e / (8 * WWN), c = 4 * (e % (8 * WWN));
            const int64_t gm = m0 + 32 * a + row, gn = col0 + c;
            const v4i v = *(const v4i *)(el + row * WEPL + c);
            if (gm >= m || gn >= n) continue;
            v4i o = v;
            if (ep_mode != WEP_PARTIAL) {
                const int32_t rs = rowsum[gm];
                o = v - rs;
                if (ep_mode == WEP_Y) {
                    const double gs = epi_gs(gamma, out.scale[gm]);
                    o = v4i{__float_as_int(epi_y(o[0], gs)), __float_as_int(epi_y(o[1], gs)),
                            __float_as_int(epi_y(o[2], gs)), __float_as_int(epi_y(o[3], gs))};
                }
            }
            int32_t *d = dst + gm * ld + gn;
            if (vec && gn + 3 < n) {
                *(v4i *)d = o;
            } else {
                for (int j = 0; j < 4 && gn + j < n; ++j) d[j] = o[j];
            }
        }
        // every lane has read the half before the next one is written
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

}  // namespace

int64_t gemm_wide_units(int64_t m, int64_t n, int splits, int wn)
{
    return ((m + WBM - 1) / WBM) * ((n + 128 * wn - 1) / (128 * wn)) * splits;
}

// Columns per wave (32-column blocks) and k slices of the wide kernel for a
// shape: 64 x 512 tiles when they fill the CUs, else 64 x 256 ones; the k
// range is split only when even those leave most CUs idle (the split
// partial sums of a large output cost more memory traffic than the idle CUs).
GemmWide gemm_wide_config(int64_t m, int64_t n, int64_t k)
{
    const int64_t nk = (k + WBK - 1) / WBK;
    int wn = gemm_wide_units(m, n, 1, 4) >= 256 ? 4 : 2;
    const int64_t tiles = gemm_wide_units(m, n, 1, wn);
    int64_t sp = 1;
    if (tiles < 128) {
        sp = (256 + tiles - 1) / tiles;
        if (sp > nk / 8) sp = nk / 8;
        if (sp < 1) sp = 1;
        // no empty slice: every slice starts before the end of the k range
        while (sp > 1 && (sp - 1) * ((nk + sp - 1) / sp) >= nk) --sp;
    }
    // two k-groups per block (eight waves) only where the k range is split:
    // timed faster there, slower on unsplit products
    return {wn, (int)sp, (wn == 2 && sp > 1) ? 2 : 1};
}

int gemm_wide_splits(int64_t m, int64_t n, int64_t k) { return gemm_wide_config(m, n, k).splits; }

template <int WWN, int KG>
static hipError_t launch_wide_wn(const int8_t *xq, const int32_t *rowsum, int64_t m,
                                 const uint8_t *packed, int64_t n, int64_t k, Out out, int splits,
                                 int32_t *ws, hipStream_t s, int64_t ldy)
{
    const int tiles_m = (int)((m + WBM - 1) / WBM);
    const int64_t units = gemm_wide_units(m, n, splits, WWN);
    const int64_t nk = (k + WBK - 1) / WBK;
    const int stages_per = (int)((nk + splits - 1) / splits);
    const int64_t per_xcd = (units + WNXCD - 1) / WNXCD;
    hipLaunchKernelGGL((gemm_wide_kernel<WWN, KG>), dim3((unsigned)(per_xcd * WNXCD)), dim3(256 * KG), 0, s,
                       xq, rowsum, m, k, packed, n, pack2_pitch(k), tiles_m, units, per_xcd,
                       splits, stages_per, out, ldy, ws);
    return hipGetLastError();
}

hipError_t launch_gemm_wide_cfg(const int8_t *xq, const int32_t *rowsum, int64_t m,
                                const uint8_t *packed, int64_t n, int64_t k, Out out,
                                GemmWide c, int32_t *ws, hipStream_t s, int64_t ldy, bool finish)
{
    hipError_t e = c.wn == 4 ? launch_wide_wn<4, 1>(xq, rowsum, m, packed, n, k, out, c.splits, ws, s, ldy)
                   : c.kg == 2 ? launch_wide_wn<2, 2>(xq, rowsum, m, packed, n, k, out, c.splits, ws, s, ldy)
                               : launch_wide_wn<2, 1>(xq, rowsum, m, packed, n, k, out, c.splits, ws, s, ldy);
    if (e != hipSuccess || c.splits == 1 || !finish) return e;
    return launch_splitk_finish(ws, rowsum, m, n, c.splits, out, ldy, s);
}

hipError_t launch_gemm_wide(const int8_t *xq, const int32_t *rowsum, int64_t m,
                            const uint8_t *packed, int64_t n, int64_t k, Out out, int splits,
                            int32_t *ws, hipStream_t s, int64_t ldy, bool finish)
{
    GemmWide c = gemm_wide_config(m, n, k);
    c.splits = splits;
    return launch_gemm_wide_cfg(xq, rowsum, m, packed, n, k, out, c, ws, s, ldy, finish);
}

}  // namespace bl
