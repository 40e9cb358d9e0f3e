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
// Block: four waves in a 2 x 2 arrangement, each owning a (32 WM) x (32 WN)
// output tile, so the block tile is (64 WM) x (64 WN); k advances in stages of
// 128.  Activations go through a two-slot register ring (loads issued two
// stages ahead) into a double-buffered, padded LDS tile; packed weights go
// into a four-slot register ring (loads issued three stages ahead).  Within
// the loop every address is a per-lane offset fixed at the start plus a
// uniform stage offset, so the stage costs no address arithmetic.  Blocks are
// numbered so that consecutive tiles (which share weight columns) land on the
// same XCD and its L2.  Tiles with two weight-column blocks per wave (WN >= 2)
// run the warp-specialised variant further down instead: producer waves move
// both operands of each stage straight from global memory into an LDS ring
// (gfx950 direct loads), and the math waves read both from LDS.
//
// Split-K (S > 1 slices of the k range) stores each slice's int32 partial
// tile into its own slice of a workspace [S][M][N] (plain stores, no
// atomics); a second kernel adds the S partial sums in slice order and
// applies the epilogue.  Integer addition makes the result exact; the
// workspace needs no initial contents.
//
// Outputs leave through LDS: the finished tile is written there with the
// epilogue applied and stored row by row with 16-byte stores (see the
// epilogue helpers below).
#include <type_traits>
#include <utility>

#include "dma.h"
#include "internal.h"

namespace bl {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// weight loads: non-temporal (1) or cached (0)
#ifndef GEMM_B_NT
#define GEMM_B_NT 0
#endif

constexpr int BK = 128;
constexpr int LDA = BK + 16;            // padded LDS row (bytes)
constexpr int NXCD = 8;


// Global -> register load of this thread's pieces of the [BM x BK] A tile.
// AL (K a multiple of 16): every load is issued unconditionally from a clamped,
// in-bounds address; pieces past K are zeroed later, when the tile is written
// to LDS, so no wait is forced here.  Rows past M carry duplicate data whose
// outputs are never stored.  !AL: byte-wise loads with bounds checks.
template <int BM, bool AL>
__device__ inline void load_a(const int8_t *__restrict__ xq, int64_t m, int64_t k, int64_t m0,
                              int64_t k0, uint4 (&regs)[BM / 32], int tid)
{
#pragma unroll
    for (int i = 0; i < BM / 32; ++i) {
        const int e = tid + 256 * i;
        const int row = e >> 3, col = (e & 7) * 16;
        int64_t gm = m0 + row, gk = k0 + col;
        if (AL) {
            gm = gm < m ? gm : m - 1;
            gk = gk < k ? gk : k - 16;
            regs[i] = load16(xq + gm * k + gk);
        } else {
            uint4 v = zero4();
            if (gm < m) {
                const int8_t *p = xq + gm * k + gk;
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
            regs[i] = v;
        }
    }
}

// Register -> LDS store of the A tile for the stage at k0 (pieces past K
// zeroed).
template <int BM, bool AL>
__device__ inline void store_a(uint8_t *lds, const uint4 (&regs)[BM / 32], int64_t k0, int64_t k,
                               int tid)
{
#pragma unroll
    for (int i = 0; i < BM / 32; ++i) {
        const int e = tid + 256 * i;
        const int row = e >> 3, col = (e & 7) * 16;
        uint4 v = regs[i];
        if (AL && k0 + col >= k) v = zero4();
        *(uint4 *)(lds + row * LDA + col) = v;
    }
}

// This lane's 16 packed bytes (64 trits) of weight row nrow for the stage at
// k0: bytes k0/4 + 16h .. +15.  The address is clamped into the matrix, so the
// load is unconditional: rows past N only feed outputs that are not stored,
// and bytes past the row meet activations that are zero there.
__device__ inline uint4 load_b(const uint8_t *__restrict__ packed, int64_t pitch, int64_t n,
                               int64_t nrow, int64_t k0, int h)
{
    int64_t byte = (k0 / 4) + 16 * h;
    byte = byte < pitch ? byte : pitch - 16;
    const int64_t row = nrow < n ? nrow : n - 1;
    return load_nt16(packed + row * pitch + byte);
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

// Fast-path stage loads: a per-lane offset fixed for the whole k loop plus a
// uniform stage offset (stage index clamped to the last full stage).
template <int BM>
__device__ __forceinline__ void ld_a(uint4 (&r)[BM / 32], const int8_t *abase,
                                     const uint32_t (&aoff)[BM / 32], int kt, int nfull)
{
    const int8_t *p = abase + (int64_t)(kt < nfull ? kt : nfull - 1) * BK;
#pragma unroll
    for (int i = 0; i < BM / 32; ++i) r[i] = load16(p + aoff[i]);
}

template <int WN>
__device__ __forceinline__ void ld_b(uint4 (&r)[WN], const uint8_t *bbase,
                                     const uint32_t (&boff)[WN], int kt, int nfull)
{
    const uint8_t *p = bbase + (int64_t)(kt < nfull ? kt : nfull - 1) * (BK / 4);
#pragma unroll
    for (int s = 0; s < WN; ++s) r[s] = GEMM_B_NT ? load_nt16(p + boff[s]) : load16(p + boff[s]);
}

template <int BM>
__device__ __forceinline__ void st_a(uint8_t *lds_buf, const uint4 (&r)[BM / 32], int tid)
{
#pragma unroll
    for (int i = 0; i < BM / 32; ++i) {
        const int e = tid + 256 * i;
        *(uint4 *)(lds_buf + (e >> 3) * LDA + (e & 7) * 16) = r[i];
    }
}

#ifndef GEMM_NA
#define GEMM_NA 2
#endif
#ifndef GEMM_SPECIALISED
#define GEMM_SPECIALISED 1
#endif
// Stages in the LDS ring of the warp-specialised kernel: four for 64 x 128
// tiles (a 49 KB ring, three blocks per CU), six for 128 x 128 tiles (one
// block per CU either way; the deeper ring keeps three stages of loads in
// flight, which pays when the weights stream from HBM).  Timed with ten
// rotating weight copies: 64 x 128 with six stages 28.3 against 24.9 us on
// 512 x 8640 x 3200; 128 x 128 with four stages 39.8 against 38.7 us on
// 128 x 28672 x 8192.
template <int WM, int WN>
constexpr int gemm3_ring()
{
#ifdef GEMM3_NS
    return GEMM3_NS;
#else
    return WM == 1 ? 4 : 6;
#endif
}
#ifndef GEMM_NB
#define GEMM_NB 4
#endif


// Stages after which every register/LDS ring is back at slot 0.
constexpr int ring_period(int na, int nb)
{
    const int l = 2 * na / gcd_int(2, na);
    return l * nb / gcd_int(l, nb);
}

// Tile of block b: consecutive tile ids on one XCD (blocks b, b+8, ... share an
// XCD); tiles are numbered m-fastest so neighbours share weight columns.
__device__ inline int64_t tile_of_block(int64_t b, int64_t q)
{
    return (b % NXCD) * q + b / NXCD;
}

// ---- epilogue through LDS ---------------------------------------------------------
// The block's accumulators are written, with the epilogue applied, into a
// [BM][BN + 4] int32 tile in LDS (y values as float bits), and then all the
// block's threads store the tile row by row with 16-byte stores.  The MFMA
// register layout would otherwise give 4-byte stores of 32 consecutive
// columns and two rows per instruction, a quarter of the store width, all
// issued at the end of every block; the row operands (row sum, gamma / s)
// are read into LDS before the k loop instead of after it.
enum : int { EP_PARTIAL = 0, EP_ACC = 1, EP_Y = 2 };

template <int BM, int BN>
constexpr int ep_tile_bytes() { return BM * (BN + 4) * 4; }

// Row operands of rows m0 .. m0 + BM - 1 (clamped), by threads 0 .. BM - 1.
template <int BM>
__device__ inline void ep_rows(int tid, int64_t m0, int64_t m, const int32_t *rowsum,
                               const Out &out, int mode, int32_t *ep_rs, double *ep_gs)
{
    if (tid >= BM || mode == EP_PARTIAL) return;
    int64_t gm = m0 + tid;
    gm = gm < m ? gm : m - 1;
    ep_rs[tid] = rowsum[gm];
    ep_gs[tid] = mode == EP_Y ? epi_gs(out.gamma[0], out.scale[gm]) : 0.0;
}

// Lane (l32, h) of math wave (wm, wn), register r of acc[a][s]: row
// 32 WM wm + 32 a + 8 (r / 4) + 4 h + r % 4, column 32 WN wn + 32 s + l32.
template <int WM, int WN>
__device__ inline void ep_put(int32_t *tile, const v16i (&acc)[WM][WN], int wm, int wn, int h,
                              int l32, const int32_t *ep_rs, const double *ep_gs, int mode)
{
    constexpr int LT = 64 * WN + 4;
#pragma unroll
    for (int a = 0; a < WM; ++a)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = wm * 32 * WM + 32 * a + 8 * (r / 4) + 4 * h + (r % 4);
            const int32_t rs = mode == EP_PARTIAL ? 0 : ep_rs[row];
            const double gs = mode == EP_Y ? ep_gs[row] : 0.0;
#pragma unroll
            for (int s = 0; s < WN; ++s) {
                const int32_t v = acc[a][s][r] - rs;
                tile[row * LT + wn * 32 * WN + 32 * s + l32] =
                    mode == EP_Y ? __float_as_int(epi_y(v, gs)) : v;
            }
        }
}

// Stores the tile to dst[(row) * ld + col] for rows m0.. < m, columns n0.. < n.
// The 16-byte stores are non-temporal: the tile is not read again by this
// kernel, and streaming it out keeps the last tiles' stores from piling up in
// the cache at the end of the launch (512 x 8640 x 3200: 24.3 -> 23.3 us,
// 128 x 28672 x 8192: 35.9 -> 35.1 us in paired graph-replay timing).
template <int BM, int BN>
__device__ inline void ep_store(const int32_t *tile, int tid, int nthreads, int64_t m0,
                                int64_t n0, int64_t m, int64_t n, int32_t *dst, int64_t ld)
{
    constexpr int LT = BN + 4, C4 = BN / 4;
    const bool vec = (ld % 4) == 0 && ((uintptr_t)dst & 15) == 0;
    for (int e = tid; e < BM * C4; e += nthreads) {
        const int row = e / C4, c = 4 * (e % C4);
        const int64_t gm = m0 + row, gn = n0 + c;
        if (gm >= m || gn >= n) continue;
        const v4i v = *(const v4i *)(tile + row * LT + c);
        int32_t *d = dst + gm * ld + gn;
        if (vec && gn + 3 < n) {
            __builtin_nontemporal_store(v, (v4i *)d);
        } else {
            for (int j = 0; j < 4 && gn + j < n; ++j) d[j] = v[j];
        }
    }
}

template <int WM, int WN, bool AL, int NA = GEMM_NA, int NB = GEMM_NB>
__global__ __launch_bounds__(256) void gemm2_kernel(const int8_t *__restrict__ xq,
                                                    const int32_t *__restrict__ rowsum,
                                                    int64_t m, int64_t k,
                                                    const uint8_t *__restrict__ packed, int64_t n,
                                                    int64_t pitch, int tiles_m, int64_t tiles,
                                                    int64_t per_xcd, int splits, int stages_per,
                                                    Out out, int64_t ldy, int32_t *__restrict__ ws)
{
    constexpr int BM = 64 * WM, BN = 64 * WN;
    // the LDS epilogue needs the A double buffer to hold the output tile
    constexpr bool LDS_EP = ep_tile_bytes<BM, BN>() <= 2 * BM * LDA;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][BM * LDA];
    __shared__ int32_t ep_rs[BM];
    __shared__ double ep_gs[BM];
    const int64_t t = tile_of_block(blockIdx.x, per_xcd);
    if (t >= tiles * splits) return;
    const int64_t tile = t / splits;
    const int split = (int)(t % splits);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int h = lane >> 5, l32 = lane & 31;
    const int tm = (int)(tile % tiles_m);
    const int64_t tn = tile / tiles_m;
    const int64_t m0 = (int64_t)tm * BM, n0 = tn * BN;
    const int nk_total = (int)((k + BK - 1) / BK);
    const int kt0 = split * stages_per;
    const int kt1 = kt0 + stages_per < nk_total ? kt0 + stages_per : nk_total;
    const int nk = kt1 - kt0;
    const int ep_mode = splits > 1 ? EP_PARTIAL : out.acc ? EP_ACC : EP_Y;

    v16i acc[WM][WN];
#pragma unroll
    for (int a = 0; a < WM; ++a)
#pragma unroll
        for (int s = 0; s < WN; ++s)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][s][r] = 0;

    int64_t nrow[WN];
#pragma unroll
    for (int s = 0; s < WN; ++s) nrow[s] = n0 + wn * 32 * WN + 32 * s + l32;

    // This wave's A fragments of one stage: 4 k-steps x WM row blocks.
    auto read_frags = [&](v4i (&af)[4][WM], const uint8_t *la) __attribute__((always_inline)) {
#pragma unroll
        for (int p = 0; p < 4; ++p)
#pragma unroll
            for (int a = 0; a < WM; ++a) {
                const int row = wm * 32 * WM + 32 * a + l32;
                const uint4 v = load16(la + row * LDA + 64 * h + 16 * p);
                af[p][a] = v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
            }
    };
    // The MFMAs of one stage: A fragments from registers, B unpacked from
    // this lane's packed weight words.
    auto mma = [&](const v4i (&af)[4][WM], const uint4 (&bw)[WN]) __attribute__((always_inline)) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            v4i bf[WN];
#pragma unroll
            for (int s = 0; s < WN; ++s) bf[s] = unpack_word(word_of(bw[s], p));
#pragma unroll
            for (int a = 0; a < WM; ++a)
#pragma unroll
                for (int s = 0; s < WN; ++s)
                    acc[a][s] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[p][a], bf[s], acc[a][s],
                                                                      0, 0, 0);
        }
    };

    // Full stages (k0 + 128 <= K) of this slice run through the pipelined
    // loop; a final partial stage, and every stage when K is not a multiple
    // of 16, take the bounds-checked path below.
    int nfull = 0;
    if (AL) {
        const int64_t full_total = k / BK;
        nfull = (int)(kt1 <= full_total ? nk : (full_total > kt0 ? full_total - kt0 : 0));
    }
    if (nfull > 0) {
        // Per-lane byte offsets, fixed for the whole k loop (rows clamped into
        // the matrix); a stage only adds a uniform offset.
        uint32_t aoff[BM / 32];
#pragma unroll
        for (int i = 0; i < BM / 32; ++i) {
            const int e = tid + 256 * i;
            int64_t gm = m0 + (e >> 3);
            gm = gm < m ? gm : m - 1;
            aoff[i] = (uint32_t)(gm * k + (e & 7) * 16);
        }
        uint32_t boff[WN];
#pragma unroll
        for (int s = 0; s < WN; ++s) {
            const int64_t row = nrow[s] < n ? nrow[s] : n - 1;
            boff[s] = (uint32_t)(row * pitch + 16 * h);
        }
        const int8_t *abase = xq + (int64_t)kt0 * BK;
        const uint8_t *bbase = packed + (int64_t)kt0 * (BK / 4);
        // Pipeline of stage j (all rings indexed by j mod ring size, fixed at
        // compile time by the unrolled stage index J):
        //   packed weights: loaded at stage j - (NB - 1) into an NB-slot
        //                   register ring;
        //   activations:    loaded at stage j - 2 - NA into an NA-slot register
        //                   ring, written to LDS buffer j mod 2 at stage j - 2;
        //   A fragments:    read from LDS at stage j - 1 into a 2-slot ring.
        // So a stage issues its loads, reads the next stage's fragments, runs
        // its MFMAs from registers, writes a later stage's activations, and
        // ends with one barrier; no LDS latency sits in front of the MFMAs.
        // Loads are unconditional (stage index clamped to the last full
        // stage), so the control flow is straight and the compiler counts
        // outstanding loads exactly.
        uint4 areg[NA][BM / 32];
        uint4 breg[NB][WN];
        v4i af[2][4][WM];
#pragma unroll
        for (int j = 0; j < NB - 1; ++j) ld_b<WN>(breg[j], bbase, boff, j, nfull);
        ld_a<BM>(areg[0], abase, aoff, 0, nfull);
        ld_a<BM>(areg[1], abase, aoff, 1, nfull);
        st_a<BM>(lds[0], areg[0], tid);
        st_a<BM>(lds[1], areg[1], tid);
#pragma unroll
        for (int j = 0; j < NA; ++j) ld_a<BM>(areg[j], abase, aoff, 2 + j, nfull);
        // row operands of the epilogue, read while the stage loads are in flight
        if (LDS_EP) ep_rows<BM>(tid, m0, m, rowsum, out, ep_mode, ep_rs, ep_gs);
        __syncthreads();
        read_frags(af[0], lds[0]);
        __syncthreads();   // buffer 0 is rewritten in stage 0

        auto stage = [&](auto jc, int j) __attribute__((always_inline)) {
            constexpr int J = decltype(jc)::value;
            constexpr int C = J & 1;
            // The compiler may interleave the phases (the next stage's
            // fragment reads and activation stores between this stage's
            // MFMAs): timed 1-2% faster on the M=64 products than keeping
            // them apart with scheduling barriers.  Nothing moves across the
            // block barrier.
            ld_b<WN>(breg[(J + NB - 1) % NB], bbase, boff, j + NB - 1, nfull);
            read_frags(af[C ^ 1], lds[C ^ 1]);
            mma(af[C], breg[J % NB]);
            st_a<BM>(lds[C], areg[J % NA], tid);
            ld_a<BM>(areg[J % NA], abase, aoff, j + 2 + NA, nfull);
            __syncthreads();
            __builtin_amdgcn_sched_barrier(0);
        };
        constexpr int U = ring_period(NA, NB);
        const int nu = nfull - nfull % U;
        for (int j = 0; j < nu; j += U)
            static_for<U>([&](auto jc) __attribute__((always_inline)) { stage(jc, j + jc); });
        static_for<U - 1>([&](auto jc) __attribute__((always_inline)) {
            if (nu + jc < nfull) stage(jc, nu + jc);
        });
    }
    if (LDS_EP && nfull == 0) ep_rows<BM>(tid, m0, m, rowsum, out, ep_mode, ep_rs, ep_gs);
    // Bounds-checked stages: the partial last stage, or all stages when K is
    // not a multiple of 16.  Loads are masked per piece; not pipelined.
    for (int kt = nfull; kt < nk; ++kt) {
        const int64_t k0 = (int64_t)(kt0 + kt) * BK;
        uint4 r[BM / 32];
        uint4 bw[WN];
        load_a<BM, AL>(xq, m, k, m0, k0, r, tid);
#pragma unroll
        for (int s = 0; s < WN; ++s) bw[s] = load_b(packed, pitch, n, nrow[s], k0, h);
        __syncthreads();
        store_a<BM, AL>(lds[0], r, k0, k, tid);
        __syncthreads();
        v4i af[4][WM];
        read_frags(af, lds[0]);
        mma(af, bw);
    }

    // LDS epilogue where the tile fits the A buffers (split partial tiles of
    // these small blocks are stored directly: measured faster than the extra
    // barrier and LDS round trip)
    if constexpr (LDS_EP) {
        if (ep_mode != EP_PARTIAL) {
            __syncthreads();   // every wave is done with the A buffers
            int32_t *tile_lds = (int32_t *)&lds[0][0];
            ep_put<WM, WN>(tile_lds, acc, wm, wn, h, l32, ep_rs, ep_gs, ep_mode);
            __syncthreads();
            int32_t *dst = ep_mode == EP_ACC ? out.acc : (int32_t *)out.y;
            ep_store<BM, BN>(tile_lds, tid, 256, m0, n0, m, n, dst, ldy);
            return;
        }
    }
    // Direct epilogue (split partial tiles, and tiles larger than the A
    // buffers).  Per-row operands are loaded for all of this lane's rows
    // first (clamped indices, unconditional), then the stores are predicated.
    if (splits > 1) {
#pragma unroll
        for (int a = 0; a < WM; ++a)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t gm = m0 + wm * 32 * WM + 32 * a + 8 * (r / 4) + 4 * h + (r % 4);
#pragma unroll
                for (int s = 0; s < WN; ++s)
                    if (gm < m && nrow[s] < n) ws[((int64_t)split * m + gm) * n + nrow[s]] = acc[a][s][r];
            }
        return;
    }
    const float gamma = out.acc ? 0.0f : out.gamma[0];
#pragma unroll
    for (int a = 0; a < WM; ++a) {
        int32_t rs[16];
        double gs[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            int64_t gm = m0 + wm * 32 * WM + 32 * a + 8 * (r / 4) + 4 * h + (r % 4);
            gm = gm < m ? gm : m - 1;
            rs[r] = rowsum[gm];
            gs[r] = out.acc ? 0.0 : epi_gs(gamma, out.scale[gm]);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t gm = m0 + wm * 32 * WM + 32 * a + 8 * (r / 4) + 4 * h + (r % 4);
#pragma unroll
            for (int s = 0; s < WN; ++s) {
                if (gm >= m || nrow[s] >= n) continue;
                const int32_t v = acc[a][s][r] - rs[r];
                if (out.acc)
                    out.acc[gm * ldy + nrow[s]] = v;
                else
                    out.y[gm * ldy + nrow[s]] = epi_y(v, gs[r]);
            }
        }
    }
}

// ---- warp-specialised variant ------------------------------------------------
// Eight waves: four math waves (the 2 x 2 arrangement above) and four
// producer waves.  The producers move every stage from global memory straight
// into LDS with gfx950's direct loads (global_load_lds_dwordx4: each
// instruction writes 64 x 16 bytes, lane i at byte 16 i of a 1 KB block), so
// no stage passes through registers and no ds_write competes with the math
// waves' fragment reads (measured: LDS reads next to direct loads run at
// their full rate, next to ds_write_b128 at about 60% of it).  LDS holds a
// ring of NS stages of BKT k (128, or 256 where the tiles fit one round of
// the CUs), each activations [BM][BKT] and packed weights [BN][BKT/4]
// without padding; the 16-byte chunks of a row are permuted (activations:
// chunk c of row r at c ^ g3_fa(r); weights: chunk c at c ^ g3_fb(r)) so
// that a fragment read of consecutive rows touches distinct 16-byte bank
// groups, which is what the padding did before.
// Iteration j (one block barrier each):
//   producers: issue stage j + NS - 1 into the slot of stage j - 1 (read for
//              the last time in iteration j - 1), then wait until stage j + 2
//              has landed (NS - 3 stages stay in flight across the barrier);
//   math:      run the MFMAs of stage j piece by piece (BKT / 32 pieces of
//              32 k), reading each piece's A fragments two pieces ahead: the
//              last two pieces read pieces 0 and 1 and the weight words of
//              stage j + 1.
// Producers wait on their own load counter and pass the barrier without a
// memory fence: a fence there would drain every load in flight.  Loads of a
// stage that ends past K are clamped into their rows; the activation chunks
// past K are then zeroed in LDS (weights past K meet zero activations).
// Chunk permutations: a fragment read of 16 consecutive rows (one lane half)
// must touch 16 distinct 16-byte groups of a 256-byte bank window.
// Activation rows of 128 bytes (BKT = 128) pair up in one window, so the
// permutation separates the eight rows of each parity; rows of 256 bytes
// (BKT = 256) each span the window, so it separates all sixteen.
template <int BKT>
__device__ inline int g3_fa(int r) { return BKT == 128 ? (r ^ (r >> 3)) & 7 : r & 15; }
// weight rows of 32 bytes (BKT = 128, two chunks; eight rows per window) or
// of 64 bytes (BKT = 256, four chunks; four rows per window)
template <int BKT>
__device__ inline int g3_fb(int r)
{
    return BKT == 128 ? ((r >> 2) ^ (r >> 3)) & 1 : (r >> 2) & 3;
}

template <int WM, int WN, int NS, int BKT = BK>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4))) void gemm3_kernel(
    const int8_t *__restrict__ xq, const int32_t *__restrict__ rowsum, int64_t m, int64_t k,
    const uint8_t *__restrict__ packed, int64_t n, int64_t pitch, int tiles_m, int64_t tiles,
    int64_t per_xcd, int splits, int stages_per, Out out, int64_t ldy, int32_t *__restrict__ ws)
{
    static_assert(WN >= 2 && NS >= 4, "weight tiles of whole 1 KB transfers, two stages in flight");
    constexpr int BM = 64 * WM, BN = 64 * WN;
    constexpr int LB = BKT / 4;          // bytes of one packed weight row per stage
    constexpr int SA = BM * BKT, SB = BN * LB, SS = SA + SB;    // bytes per stage slot
    constexpr int PA = SA / 4096;        // 1 KB activation transfers per producer wave and stage
    constexpr int PB = SB / 4096;        // 1 KB weight transfers per producer wave and stage
    constexpr int PT = PA + PB;
    constexpr int NP = BKT / 32;         // 32-k pieces per stage
    constexpr int CB = BKT / 128;        // 16-byte weight chunks per lane and stage
    // EPL: the ring takes all of the LDS, so the epilogue's row operands are
    // held in the producers' registers during the k loop and written behind
    // the output tile in the drained ring afterwards
    constexpr bool EPL = NS * SS + BM * 12 > 163840;
    constexpr int EPO = EPL ? ep_tile_bytes<BM, BN>() : NS * SS;   // row operands' offset
    __shared__ __attribute__((aligned(16))) uint8_t lds[NS * SS + (EPL ? 0 : BM * 12)];
    int32_t *const ep_rs = (int32_t *)(lds + EPO);
    double *const ep_gs = (double *)(lds + EPO + BM * 4);
    static_assert(ep_tile_bytes<BM, BN>() + (EPL ? BM * 12 : 0) <= NS * SS,
                  "the output tile (and, with EPL, the row operands) fits the LDS ring");
    const int64_t t = tile_of_block(blockIdx.x, per_xcd);
    if (t >= tiles * splits) return;
    const int64_t tile = t / splits;
    const int split = (int)(t % splits);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const bool producer = wave >= 4;
    const int tm = (int)(tile % tiles_m);
    const int64_t tn = tile / tiles_m;
    const int64_t m0 = (int64_t)tm * BM, n0 = tn * BN;
    const int nk_total = (int)((k + BKT - 1) / BKT);
    const int kt0 = split * stages_per;
    const int kt1 = kt0 + stages_per < nk_total ? kt0 + stages_per : nk_total;
    const int nk = kt1 - kt0;
    const int ep_mode = splits > 1 ? EP_PARTIAL : out.acc ? EP_ACC : EP_Y;
    if (nk <= 0) {
        // an empty k slice still stores its partial tile (zeros): the finish
        // adds every slice, and the workspace has no required contents
        if (ep_mode == EP_PARTIAL) {
            int32_t *tl = (int32_t *)lds;
            for (int e = threadIdx.x; e < BM * (BN + 4); e += 512) tl[e] = 0;
            __syncthreads();
            ep_store<BM, BN>(tl, threadIdx.x, 512, m0, n0, m, n, ws + (int64_t)split * m * n, n);
        }
        return;
    }

    if (producer) {
        const int pw = wave - 4;
        int32_t epl_rs = 0;
        double epl_gs = 0.0;
        if constexpr (EPL) {
            // this thread's row operands of the epilogue, loaded now
            const int pt = threadIdx.x - 256;
            if (pt < BM && ep_mode != EP_PARTIAL) {
                int64_t gm = m0 + pt;
                gm = gm < m ? gm : m - 1;
                epl_rs = rowsum[gm];
                epl_gs = ep_mode == EP_Y ? epi_gs(out.gamma[0], out.scale[gm]) : 0.0;
            }
        }
        // Per-lane sources, fixed for the loop: transfer q of this wave fills
        // LDS bytes [1024 qi, 1024 qi + 1024) of the slot's activation (or
        // weight) part, qi = pw * PA + q (or pw * PB + q); lane i writes the
        // chunk at byte 16 i of it.  Rows are clamped into the matrices.
        uint32_t aoff[PA], boff[PB];
        int acol[PA], bhalf[PB];
#pragma unroll
        for (int q = 0; q < PA; ++q) {
            const int r = (1024 / BKT) * (pw * PA + q) + lane / (BKT / 16);
            const int c = (lane % (BKT / 16)) ^ g3_fa<BKT>(r);
            int64_t gm = m0 + r;
            gm = gm < m ? gm : m - 1;
            acol[q] = 16 * c;
            aoff[q] = (uint32_t)(gm * k + 16 * c);
        }
#pragma unroll
        for (int q = 0; q < PB; ++q) {
            const int r = (1024 / LB) * (pw * PB + q) + lane / (LB / 16);
            const int hh = (lane % (LB / 16)) ^ g3_fb<BKT>(r);
            int64_t row = n0 + r;
            row = row < n ? row : n - 1;
            bhalf[q] = 16 * hh;
            boff[q] = (uint32_t)(row * pitch + 16 * hh);
        }
        const int full_end = (int)(k / BKT) - kt0;   // stages [0, full_end) lie inside K
        auto issue = [&](int st) __attribute__((always_inline)) {
            uint8_t *slot = lds + (st % NS) * SS;
            const int64_t k0 = (int64_t)(kt0 + st) * BKT;
            if (st < full_end) {
                const int8_t *ab = xq + k0;
                const uint8_t *bb = packed + k0 / 4;
#pragma unroll
                for (int q = 0; q < PA; ++q) dl_load16(ab + aoff[q], slot + 1024 * (pw * PA + q));
#pragma unroll
                for (int q = 0; q < PB; ++q) dl_load16(bb + boff[q], slot + SA + 1024 * (pw * PB + q));
                return;
            }
#pragma unroll
            for (int q = 0; q < PA; ++q) {
                const int64_t kk = k0 + acol[q] < k ? k0 : k - 16 - acol[q];
                dl_load16(xq + aoff[q] + kk, slot + 1024 * (pw * PA + q));
            }
#pragma unroll
            for (int q = 0; q < PB; ++q) {
                int64_t byte = k0 / 4;
                byte = byte + bhalf[q] + 16 <= pitch ? byte : pitch - 16 - bhalf[q];
                dl_load16(packed + boff[q] + byte, slot + SA + 1024 * (pw * PB + q));
            }
        };
        // Activation chunks past K of the stage st (once its loads have landed).
        auto zero_tail = [&](int st) __attribute__((always_inline)) {
            if (st < full_end || st >= nk) return;
            uint8_t *slot = lds + (st % NS) * SS;
            const int64_t k0 = (int64_t)(kt0 + st) * BKT;
#pragma unroll
            for (int q = 0; q < PA; ++q)
                if (k0 + acol[q] >= k) *(uint4 *)(slot + 1024 * (pw * PA + q) + 16 * lane) = zero4();
        };
        // prologue: stages 0 .. NS - 2 in flight; stages 0 and 1 landed
        static_for<NS - 1>([&](auto sc) __attribute__((always_inline)) {
            if (decltype(sc)::value < nk) issue(decltype(sc)::value);
        });
        if (nk >= NS - 1) __builtin_amdgcn_s_waitcnt(dl_vmcnt((NS - 3) * PT));
        else __builtin_amdgcn_s_waitcnt(dl_vmcnt(0));
        zero_tail(0);
        zero_tail(1);
        __builtin_amdgcn_s_waitcnt(DL_LGKM0);
        dl_barrier();
        for (int j = 0; j < nk; ++j) {
            if (j + NS - 1 < nk) {
                issue(j + NS - 1);
                __builtin_amdgcn_s_waitcnt(dl_vmcnt((NS - 3) * PT));
            } else {
                __builtin_amdgcn_s_waitcnt(dl_vmcnt(0));
                zero_tail(j + 2);
                __builtin_amdgcn_s_waitcnt(DL_LGKM0);
            }
            dl_barrier();
        }
        if constexpr (EPL) {
            // the ring is drained (every stage landed and consumed): the row
            // operands go behind the output tile's place, then one barrier
            // publishes them to the math waves
            const int pt = threadIdx.x - 256;
            if (pt < BM) {
                ep_rs[pt] = epl_rs;
                ep_gs[pt] = epl_gs;
            }
            __syncthreads();
        }
    } else {
    // ---- math waves ----
    const int wm = wave & 1, wn = wave >> 1;
    const int h = lane >> 5, l32 = lane & 31;
    v16i acc[WM][WN];
#pragma unroll
    for (int a = 0; a < WM; ++a)
#pragma unroll
        for (int s = 0; s < WN; ++s)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][s][r] = 0;

    // row operands of the epilogue, visible after the first barrier
    if constexpr (!EPL) ep_rows<BM>(threadIdx.x, m0, m, rowsum, out, ep_mode, ep_rs, ep_gs);
    // Fragments stream two k pieces ahead of the MFMAs: while the MFMAs of
    // piece p of stage j run, piece p + 2 is read from LDS (pieces 0 and 1 of
    // stage j + 1 during pieces 2 and 3, with the stage's weight words).
    // The weight operands are unpacked one piece ahead, interleaved with the
    // MFMAs (timed: 128 x 128 tiles 8-11% faster than unpacking a piece
    // before its MFMAs behind scheduling barriers, 64 x 128 tiles 1-3%).
    // Four pieces of A and two stages of weight words are live: 76 registers
    // with 64 x 128 tiles, so with the 49 KB ring three blocks share a CU and
    // fill each other's waits.  The last stage also reads a next stage that
    // does not exist: those reads stay inside the LDS ring and their values
    // are never used.
    // lane half h takes the stage's k range [BKT/2 h, BKT/2 (h + 1)): piece p
    // is activation chunk NP h + p, and word p % 4 of weight chunk CB h + p / 4
    // (64 trits per chunk)
    auto read_a = [&](v4i (&a)[WM], const uint8_t *slot, int p) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < WM; ++i) {
            const int row = wm * 32 * WM + 32 * i + l32;
            const uint4 v = load16(slot + row * BKT + 16 * ((NP * h + p) ^ g3_fa<BKT>(row)));
            a[i] = v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
        }
    };
    auto read_b = [&](uint4 (&b)[WN][CB], const uint8_t *slot) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < WN; ++s) {
            const int row = wn * 32 * WN + 32 * s + l32;
#pragma unroll
            for (int c = 0; c < CB; ++c)
                b[s][c] = load16(slot + SA + row * LB + 16 * ((CB * h + c) ^ g3_fb<BKT>(row)));
        }
    };
    v4i af[4][WM];
    uint4 bw[WN][CB], bn[WN][CB];
    __syncthreads();          // stages 0 and 1 are in LDS
    read_a(af[0], lds, 0);
    read_a(af[1], lds, 1);
    read_b(bw, lds);
    v4i bfc[WN];              // unpacked weights of the current piece
#pragma unroll
    for (int s = 0; s < WN; ++s) bfc[s] = unpack_word(word_of(bw[s][0], 0));
    int cur = 0;              // ring slot of stage j
    for (int j = 0; j < nk; ++j) {
        const int nxt = cur == NS - 1 ? 0 : cur + 1;
        const uint8_t *slot = lds + cur * SS, *nslot = lds + nxt * SS;
        static_for<NP>([&](auto pc) __attribute__((always_inline)) {
            constexpr int P = decltype(pc)::value;
            if constexpr (P < NP - 2) {
                read_a(af[(P + 2) % 4], slot, P + 2);
            } else {
                read_a(af[(P + 2) % 4], nslot, P + 2 - NP);
                if (P == NP - 2) read_b(bn, nslot);
            }
            // This piece's MFMAs on the weights unpacked during the previous
            // piece, each followed by the unpack (7 VALU) of one weight
            // operand of the next piece (piece 0 of stage j + 1 after piece 3).
            v4i bfn[WN];
#pragma unroll
            for (int s = 0; s < WN; ++s) {
#pragma unroll
                for (int a = 0; a < WM; ++a)
                    acc[a][s] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[P % 4][a], bfc[s],
                                                                      acc[a][s], 0, 0, 0);
                if constexpr (P < NP - 1)
                    bfn[s] = unpack_word(word_of(bw[s][(P + 1) / 4], (P + 1) % 4));
                else
                    bfn[s] = unpack_word(word_of(bn[s][0], 0));
            }
#pragma unroll
            for (int s = 0; s < WN; ++s) {
                __builtin_amdgcn_sched_group_barrier(0x008, WM, 0);   // MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);    // VALU
            }
#pragma unroll
            for (int s = 0; s < WN; ++s) bfc[s] = bfn[s];
        });
#pragma unroll
        for (int s = 0; s < WN; ++s)
#pragma unroll
            for (int c = 0; c < CB; ++c) bw[s][c] = bn[s][c];
        cur = nxt;
        // No fence: the fragment reads still in flight here are of stage
        // j + 1, whose slot is refilled only after three more barriers, and
        // every read of stage j has been consumed by this stage's MFMAs; so
        // their latency overlaps the barrier instead of preceding it.
        dl_barrier();
    }

    // Epilogue: the accumulators into the output tile in the ring (every
    // wave is past its last ring access after the final barrier of the loop)
    if constexpr (EPL) __syncthreads();   // the producers' row operands
    ep_put<WM, WN>((int32_t *)lds, acc, wm, wn, h, l32, ep_rs, ep_gs, ep_mode);
    }
    // all waves store the tile
    __syncthreads();
    int32_t *dst = ep_mode == EP_PARTIAL ? ws + (int64_t)split * m * n
                   : ep_mode == EP_ACC   ? out.acc
                                         : (int32_t *)out.y;
    ep_store<BM, BN>((const int32_t *)lds, threadIdx.x, 512, m0, n0, m, n, dst,
                     ep_mode == EP_PARTIAL ? n : ldy);
}

// Split-K epilogue: sum of the splits' partial tiles, slice by slice in split order (exact
// int32), then the epilogue.
__global__ __launch_bounds__(256) void splitk_finish_kernel(const int32_t *__restrict__ ws,
                                                            const int32_t *__restrict__ rowsum,
                                                            int64_t m, int64_t n, int splits,
                                                            Out out, int64_t ldy)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= m * n) return;
    const int64_t gm = i / n, gn = i % n;
    int32_t v = 0;
    for (int sp = 0; sp < splits; ++sp) v += ws[sp * m * n + i];
    store_out(out, ldy, gm, gn, v, rowsum[gm]);
}

// Same sums, four consecutive columns of one row per thread (N a multiple of
// 4, so the slices and the output rows stay 16-byte aligned; vec: the
// output too): 16-byte loads and stores, one gamma / s per four outputs.
// The row operands and the slices' loads, up to four at a time, are issued
// before the first add (slices past `splits` are masked, not branched), so
// that a launch waits for one round of memory latency per four slices
// rather than one per slice (70B-class 16 x 8192 x 28672 product with four
// slices, paired graph-replay timing: 20.0 -> 19.5 us in total).
__global__ __launch_bounds__(256) void splitk_finish4_kernel(const int32_t *__restrict__ ws,
                                                             const int32_t *__restrict__ rowsum,
                                                             int64_t m, int64_t n, int splits,
                                                             Out out, int64_t ldy, bool vec)
{
    const int64_t e = 4 * ((int64_t)blockIdx.x * 256 + threadIdx.x);
    if (e >= m * n) return;
    const int64_t gm = e / n, gn = e % n;
    const int32_t rs = rowsum[gm];
    const float g = out.acc ? 0.0f : out.gamma[0], sc = out.acc ? 1.0f : out.scale[gm];
    v4i v = {0, 0, 0, 0};
    for (int s0 = 0; s0 < splits; s0 += 4) {
        v4i p[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int sp = s0 + q < splits ? s0 + q : splits - 1;   // in bounds; masked below
            p[q] = *(const v4i *)(ws + sp * m * n + e);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (s0 + q < splits) v += p[q];
    }
    const v4i a = v - rs;
    if (out.acc) {
        int32_t *d = out.acc + gm * ldy + gn;
        if (vec) *(v4i *)d = a;
        else
            for (int j = 0; j < 4; ++j) d[j] = a[j];
    } else {
        const double gs = epi_gs(g, sc);
        float *d = out.y + gm * ldy + gn;
        const float f[4] = {epi_y(a[0], gs), epi_y(a[1], gs), epi_y(a[2], gs), epi_y(a[3], gs)};
        if (vec) *(float4 *)d = make_float4(f[0], f[1], f[2], f[3]);
        else
            for (int j = 0; j < 4; ++j) d[j] = f[j];
    }
}

}  // namespace

hipError_t launch_splitk_finish(const int32_t *ws, const int32_t *rowsum, int64_t m, int64_t n,
                                int splits, Out out, int64_t ldy, hipStream_t s)
{
    const int64_t total = m * n;
    if (n % 4 == 0 && ((uintptr_t)ws & 15) == 0) {
        const uintptr_t base = out.acc ? (uintptr_t)out.acc : (uintptr_t)out.y;
        const bool vec = (ldy % 4) == 0 && (base & 15) == 0;
        hipLaunchKernelGGL(splitk_finish4_kernel, dim3((unsigned)((total / 4 + 255) / 256)),
                           dim3(256), 0, s, ws, rowsum, m, n, splits, out, ldy, vec);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(splitk_finish_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                       s, ws, rowsum, m, n, splits, out, ldy);
    return hipGetLastError();
}

// Kernel configuration of the GEMM for (M, N, K): the square-ish tiles of
// gemm2 / gemm3 (wm x wn blocks of 64), or the wide-tile kernel.
struct GemmCfg { int wm, wn, splits; bool wide; };

GemmCfg gemm_config(int64_t m, int64_t n, int64_t k, int variant = GEMM_TILED)
{
    if (variant == GEMM_WIDE) return {0, 0, gemm_wide_splits(m, n, k), true};
    // Chosen from timings of every tile / split combination on the 2B-, 3B-
    // and 70B-class shapes.  M <= 64, or a product with few 64 x 64 tiles:
    // 64 x 64 tiles, the k range split (up to four ways, at least six stages
    // each) when there are few of them.
    // Larger: 128 x 128 tiles (one block per CU, its six-stage LDS ring takes
    // 120 KB) when they fill one round of the 256 CUs; 64 x 128 tiles (three
    // blocks per CU) when there are more, or when 128 x 128 ones are too few
    // and 64 x 128 ones still fill most of the chip; else 128 x 128 tiles with
    // the k range split.
    const int64_t nk = (k + BK - 1) / BK;
    auto tiles = [&](int wm, int wn) {
        return ((m + 64 * wm - 1) / (64 * wm)) * ((n + 64 * wn - 1) / (64 * wn));
    };
    const int64_t t11 = tiles(1, 1);
    if (m <= 64 || t11 < 192) {
        int64_t sp = t11 < 192 ? 256 / t11 : 1;   // splits: up to 4, >= 6 stages each
        if (sp > 4) sp = 4;
        if (sp > nk / 6) sp = nk / 6;
        return {1, 1, (int)(sp < 1 ? 1 : sp), false};
    }
    const int64_t t22 = tiles(2, 2);
    if (t22 >= 192 && t22 <= 256) return {2, 2, 1, false};
    if (t22 > 256) return {1, 2, 1, false};
    // 64 x 128 tiles that fill most of the chip beat 128 x 128 tiles with the
    // k range split (no partial sums to write, read back and add)
    if (tiles(1, 2) >= 192) return {1, 2, 1, false};
    int64_t sp = 256 / t22;
    if (sp > 8) sp = 8;
    if (sp > nk / 4) sp = nk / 4;
    return {2, 2, (int)(sp < 1 ? 1 : sp), false};
}

// Row / column blocks of a product whose operands exceed 32-bit offsets.
static void gemm_chunks(int64_t m, int64_t n, int64_t k, int64_t &mc, int64_t &nc)
{
    const int64_t lim = (int64_t)1 << 31;
    const int64_t pitch = pack2_pitch(k);
    mc = m;
    nc = n;
    if (mc * k >= lim) mc = ((lim - 1) / k) / 128 * 128;
    if (nc * pitch >= lim) nc = ((lim - 1) / pitch) / 128 * 128;
    if (mc < 1) mc = 1;
    if (nc < 1) nc = 1;
}

// The GEMM variant AUTO takes: the tiled kernel.  Timed against the wide
// tiles on the 3B-class M=512 and 70B-class M=128 products, it is as fast or
// faster on every one (the wide kernel stays available by explicit path).
int gemm_preferred_variant(int64_t, int64_t, int64_t)
{
    return GEMM_TILED;
}

// One int32 partial tile per split: splits x M x N (largest over the blocks).
int64_t gemm_workspace_bytes(int64_t m, int64_t n, int64_t k, int variant)
{
    int64_t mc, nc, need = 0;
    gemm_chunks(m, n, k, mc, nc);
    for (int64_t m0 = 0; m0 < m; m0 += mc)
        for (int64_t n0 = 0; n0 < n; n0 += nc) {
            const int64_t mb = m - m0 < mc ? m - m0 : mc;
            const int64_t nb = n - n0 < nc ? n - n0 : nc;
            const GemmCfg c = gemm_config(mb, nb, k, variant);
            const int64_t b = c.splits > 1 ? 4 * c.splits * mb * nb : 0;
            need = b > need ? b : need;
        }
    return need;
}

template <int WM, int WN>
hipError_t launch_gemm_cfg(const int8_t *xq, const int32_t *rowsum, int64_t m,
                           const uint8_t *packed, int64_t n, int64_t k, Out out, int splits,
                           int32_t *ws, hipStream_t s, int64_t ldy = -1, bool finish = true)
{
    constexpr int BM = 64 * WM, BN = 64 * WN;
    const int tiles_m = (int)((m + BM - 1) / BM);
    const int64_t tiles = (int64_t)tiles_m * ((n + BN - 1) / BN);
    const int64_t nk = (k + BK - 1) / BK;
    const int stages_per = (int)((nk + splits - 1) / splits);
    const int64_t units = tiles * splits;
    const int64_t per_xcd = (units + NXCD - 1) / NXCD;
    const dim3 grid((unsigned)(per_xcd * NXCD)), block(256);
    const int64_t pitch = pack2_pitch(k);
    if (ldy < 0) ldy = n;
    // the producer/consumer kernel pays off once a block has two weight-column
    // blocks per wave (WN >= 2); narrower tiles keep the single-role kernel
    bool specialised = false;
    if constexpr (WN >= 2) {
        if (k % 16 == 0 && GEMM_SPECIALISED) {
            bool deep = false;
            if constexpr (WN == 2) {
                if (units <= 256) {
                    // tiles that fit one round of the CUs (one block each):
                    // stages of 256 k in a four-stage ring (64 x 128 tiles:
                    // 96 KB; 128 x 128 tiles: all 160 KB, the epilogue's row
                    // operands held by the producers).  Paired steady-state
                    // timing: 512 x 3200 x 8640 (200 tiles) 25.3 -> 21.0 us
                    // (three stages 32.6 us); 128 x 28672 x 8192 35.6 -> 34.6
                    // us, 128 x 8192 x 28672 41.7 -> 40.0 us (three 256-k
                    // stages 45.6 / 48.5 us).
                    const int64_t nk2 = (k + 255) / 256;
                    const int sp2 = (int)((nk2 + splits - 1) / splits);
                    hipLaunchKernelGGL((gemm3_kernel<WM, WN, 4, 256>), grid, dim3(512), 0, s, xq,
                                       rowsum, m, k, packed, n, pitch, tiles_m, tiles, per_xcd,
                                       splits, sp2, out, ldy, ws);
                    deep = true;
                }
            }
            if (!deep)
                hipLaunchKernelGGL((gemm3_kernel<WM, WN, gemm3_ring<WM, WN>()>), grid, dim3(512),
                                   0, s, xq, rowsum, m, k, packed, n, pitch, tiles_m, tiles,
                                   per_xcd, splits, stages_per, out, ldy, ws);
            specialised = true;
        }
    }
    if (specialised)
        ;
    else if (k % 16 == 0)
        hipLaunchKernelGGL((gemm2_kernel<WM, WN, true>), grid, block, 0, s, xq, rowsum, m, k,
                           packed, n, pitch, tiles_m, tiles, per_xcd, splits, stages_per, out, ldy,
                           ws);
    else
        hipLaunchKernelGGL((gemm2_kernel<WM, WN, false>), grid, block, 0, s, xq, rowsum, m, k,
                           packed, n, pitch, tiles_m, tiles, per_xcd, splits, stages_per, out, ldy,
                           ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits == 1 || !finish) return e;
    return launch_splitk_finish(ws, rowsum, m, n, splits, out, ldy, s);
}

hipError_t launch_gemm_pack2(const int8_t *xq, const int32_t *rowsum, int64_t m,
                             const uint8_t *packed, int64_t n, int64_t k, Out out, void *ws,
                             hipStream_t s, int variant)
{
    // The kernel addresses each operand with 32-bit per-lane offsets: larger
    // operands are processed in blocks of rows of x and of weight rows.
    const int64_t pitch = pack2_pitch(k);
    int64_t mc, nc;
    gemm_chunks(m, n, k, mc, nc);
    for (int64_t m0 = 0; m0 < m; m0 += mc) {
        for (int64_t n0 = 0; n0 < n; n0 += nc) {
            const int64_t mb = m - m0 < mc ? m - m0 : mc;
            const int64_t nb = n - n0 < nc ? n - n0 : nc;
            Out o = out;
            if (o.scale) o.scale += m0;
            if (o.y) o.y += m0 * n + n0;
            if (o.acc) o.acc += m0 * n + n0;
            const GemmCfg c = gemm_config(mb, nb, k, variant);
            int32_t *w = (int32_t *)ws;
            const int8_t *x = xq + m0 * k;
            const int32_t *rs = rowsum + m0;
            const uint8_t *pk = packed + n0 * pitch;
            hipError_t e;
            if (c.wide)
                e = launch_gemm_wide(x, rs, mb, pk, nb, k, o, c.splits, w, s, n, true);
            else if (c.wm == 2 && c.wn == 2)
                e = launch_gemm_cfg<2, 2>(x, rs, mb, pk, nb, k, o, c.splits, w, s, n);
            else if (c.wm == 1 && c.wn == 2)
                e = launch_gemm_cfg<1, 2>(x, rs, mb, pk, nb, k, o, c.splits, w, s, n);
            else if (c.wm == 2 && c.wn == 1)
                e = launch_gemm_cfg<2, 1>(x, rs, mb, pk, nb, k, o, c.splits, w, s, n);
            else
                e = launch_gemm_cfg<1, 1>(x, rs, mb, pk, nb, k, o, c.splits, w, s, n);
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

// Tiles and k split of a product whose split partial sums the next kernel
// finishes (no finish launch to pay for).
static GemmCfg gemm_partial_config(int64_t m, int64_t n, int64_t k, int variant)
{
    return gemm_config(m, n, k, variant);
}

int gemm_partial_splits(int64_t m, int64_t n, int64_t k, int variant)
{
    int64_t mc, nc;
    gemm_chunks(m, n, k, mc, nc);
    if (mc < m || nc < n) return 0;
    const GemmCfg c = gemm_partial_config(m, n, k, variant);
    return c.splits > 1 ? c.splits : 0;
}

int64_t gemm_partial_workspace_bytes(int64_t m, int64_t n, int64_t k, int variant)
{
    const int sp = gemm_partial_splits(m, n, k, variant);
    return sp > 1 ? 4 * (int64_t)sp * m * n : 0;
}

hipError_t launch_gemm_pack2_partials(const int8_t *xq, const int32_t *rowsum, int64_t m,
                                      const uint8_t *packed, int64_t n, int64_t k, Out out,
                                      int32_t *ws, hipStream_t s, int variant)
{
    const GemmCfg c = gemm_partial_config(m, n, k, variant);
    if (c.wide) return launch_gemm_wide(xq, rowsum, m, packed, n, k, out, c.splits, ws, s, n, false);
    if (c.wm == 2 && c.wn == 2)
        return launch_gemm_cfg<2, 2>(xq, rowsum, m, packed, n, k, out, c.splits, ws, s, n, false);
    if (c.wm == 1 && c.wn == 2)
        return launch_gemm_cfg<1, 2>(xq, rowsum, m, packed, n, k, out, c.splits, ws, s, n, false);
    if (c.wm == 2 && c.wn == 1)
        return launch_gemm_cfg<2, 1>(xq, rowsum, m, packed, n, k, out, c.splits, ws, s, n, false);
    return launch_gemm_cfg<1, 1>(xq, rowsum, m, packed, n, k, out, c.splits, ws, s, n, false);
}

}  // namespace bl
