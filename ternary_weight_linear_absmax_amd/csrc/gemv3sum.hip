// Base-3 ternary GEMV for one token with partial-sum lookup tables.
//
// Source: news.hada.io topic 20406, the comment on ternary packing: five
// ternary digits fit in one byte (3^5 = 243 <= 256, log2 3 = 1.585 bits per
// weight).  A packed byte b holds the codes d_i = t_{5j+i} + 1 of five
// consecutive k as its base-3 digits, b = sum_i d_i 3^i.  For a fixed token,
// the group's contribution sum_i d_i q_{5j+i} depends only on b, so one table
// of 243 partial sums per group of five activations turns every packed byte
// into one table read and one add (the offset codes are corrected by the
// token's row sum in the epilogue, as on every other path).
//
// The tables of all groups of a row do not fit in LDS, so the k range is cut
// into slices of SLICE packed bytes (SLICE groups, 5 * SLICE trits).  Block
// (r, s) builds the SLICE tables of slice s in LDS (one group per thread, the
// 243 sums by adding one activation at a time, odometer order) and streams
// the slice's packed bytes of its rows: a wave takes four rows at once, 16
// lanes per row, 16 bytes per lane, so an instruction reads four contiguous
// 256-byte runs (eight waves per block, two per SIMD, share the tables).
// Each lane adds its 16 table entries, the row's 16 lanes (one DPP row) are
// summed, and the slice's partial sum of the row goes to its own slice of the
// workspace; the split-k finish adds the slices in order, subtracts the row
// sum and rescales.  One slice (K <= 1280) writes the outputs directly.
#include "internal.h"

namespace bl {
namespace {

constexpr int S3_SLICE = 256;      // packed bytes (groups) per slice
constexpr int S3_STRIDE = 246;     // int16 entries per table (243 used; an odd dword stride)
constexpr int S3_PF = 8;           // row quads of packed bytes in flight ahead, per wave
constexpr int S3_WAVES = 8;        // waves per block (two per SIMD share the tables)

__global__ __launch_bounds__(64 * S3_WAVES) void gemv3sum_kernel(const int8_t *__restrict__ xq,
                                                       const int32_t *__restrict__ rowsum,
                                                       int64_t k, const uint8_t *__restrict__ packed,
                                                       int64_t n, int64_t pitch, int64_t rows_per,
                                                       Out out, int32_t *__restrict__ part)
{
    __shared__ int16_t lut[S3_SLICE * S3_STRIDE];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t s = blockIdx.y;                     // slice
    const int64_t byte0 = s * S3_SLICE;               // first packed byte (group) of the slice
    const int64_t r0 = (int64_t)blockIdx.x * rows_per;
    int64_t r1 = r0 + rows_per;
    r1 = r1 < n ? r1 : n;
    const int64_t nquads = r1 > r0 ? (r1 - r0 + 3) / 4 : 0;

    // this lane's rows and chunk: row quad q covers rows r0 + 4q .. +3; lane
    // (sub = lane / 16, c = lane % 16) reads bytes byte0 + 16c .. +15 of its row
    const int sub = lane >> 4, c = lane & 15;
    const bool chunk_ok = byte0 + 16 * c < pitch;     // the last slice may be short
    const int64_t coff = chunk_ok ? byte0 + 16 * c : 0;
    auto row_of = [&](int64_t q) __attribute__((always_inline)) {
        int64_t row = r0 + 4 * q + sub;
        row = row < r1 ? row : r1 - 1;                // clamped: never stored
        return row;
    };
    // quads of this wave: wave, wave + S3_WAVES, ...; loads issued S3_PF
    // quads ahead (clamped to the wave's last quad, whose loads stay in bounds)
    const int64_t my_quads = nquads > wave ? (nquads - wave + S3_WAVES - 1) / S3_WAVES : 0;
    auto load = [&](int64_t j) __attribute__((always_inline)) {
        const int64_t jj = j < my_quads ? j : (my_quads > 0 ? my_quads - 1 : 0);
        return load_nt16(packed + row_of(wave + S3_WAVES * jj) * pitch + coff);
    };
    uint4 ring[S3_PF];
#pragma unroll
    for (int p = 0; p < S3_PF; ++p) ring[p] = load(p);

    // tables of the slice: thread t builds group t, entry b = sum_i d_i q_i
    // for the base-3 digits d_i of b (activations past K are zero)
    if (tid < S3_SLICE) {
        int q[5];
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            const int64_t kk = 5 * (byte0 + tid) + i;
            q[i] = kk < k ? (int)xq[kk] : 0;
        }
        int16_t *tab = lut + tid * S3_STRIDE;
        int b = 0;
        int s4 = 0;
#pragma unroll
        for (int d4 = 0; d4 < 3; ++d4) {
            int s3 = s4;
#pragma unroll
            for (int d3 = 0; d3 < 3; ++d3) {
                int s2 = s3;
#pragma unroll
                for (int d2 = 0; d2 < 3; ++d2) {
                    int s1 = s2;
#pragma unroll
                    for (int d1 = 0; d1 < 3; ++d1) {
                        int s0 = s1;
#pragma unroll
                        for (int d0 = 0; d0 < 3; ++d0) {
                            tab[b++] = (int16_t)s0;
                            s0 += q[0];
                        }
                        s1 += q[1];
                    }
                    s2 += q[2];
                }
                s3 += q[3];
            }
            s4 += q[4];
        }
    }
    __syncthreads();

    const int16_t *tbase = lut + 16 * c * S3_STRIDE;
    const int32_t e_rs = rowsum[0];
    const double e_gs = (part || out.acc) ? 0.0 : epi_gs(out.gamma[0], out.scale[0]);
    auto quad = [&](const uint4 &v, int64_t j) __attribute__((always_inline)) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        int acc = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t byte = (w[i >> 2] >> (8 * (i & 3))) & 0xFFu;
            acc += tbase[i * S3_STRIDE + byte];
        }
        acc = chunk_ok ? acc : 0;
        // sum over the 16 lanes of the row (a DPP row: pairs, quads, half
        // rows, rows; every lane of the row ends with the sum)
        acc += __builtin_amdgcn_update_dpp(0, acc, 0xB1, 0xF, 0xF, false);    // quad_perm [1,0,3,2]
        acc += __builtin_amdgcn_update_dpp(0, acc, 0x4E, 0xF, 0xF, false);    // quad_perm [2,3,0,1]
        acc += __builtin_amdgcn_update_dpp(0, acc, 0x141, 0xF, 0xF, false);   // row_half_mirror
        acc += __builtin_amdgcn_update_dpp(0, acc, 0x140, 0xF, 0xF, false);   // row_mirror
        const int64_t row = r0 + 4 * (wave + S3_WAVES * j) + sub;
        if (c == 0 && row < r1) {
            if (part) {
                part[s * n + row] = acc;
            } else if (out.acc) {
                out.acc[row] = acc - e_rs;
            } else {
                out.y[row] = epi_y(acc - e_rs, e_gs);
            }
        }
    };
    // ring slots fixed at compile time: quad j uses slot j % S3_PF, which is
    // refilled with quad j + S3_PF right after it is read
    int64_t j = 0;
    for (; j + S3_PF <= my_quads; j += S3_PF)
        static_for<S3_PF>([&](auto pc) __attribute__((always_inline)) {
            constexpr int P = decltype(pc)::value;
            const uint4 v = ring[P];
            ring[P] = load(j + P + S3_PF);
            quad(v, j + P);
        });
    static_for<S3_PF - 1>([&](auto pc) __attribute__((always_inline)) {
        constexpr int P = decltype(pc)::value;
        if (j + P < my_quads) quad(ring[P], j + P);
    });
}

}  // namespace

// Slices of the k range (0: the shape does not take this kernel).
int gemv3sum_slices(int64_t m, int64_t n, int64_t k)
{
    if (m != 1 || gemv3lut_supported(m, k)) return 0;
    const int64_t pitch = pack3_pitch(k);
    // the tables pay off once every block streams several hundred rows
    if (n < 4096) return 0;
    return (int)((pitch + S3_SLICE - 1) / S3_SLICE);
}

int64_t gemv3sum_workspace_bytes(int64_t m, int64_t n, int64_t k)
{
    const int sl = gemv3sum_slices(m, n, k);
    return sl > 1 ? 4 * (int64_t)sl * n : 0;
}

hipError_t launch_gemv3sum(const int8_t *xq, const int32_t *rowsum, const uint8_t *packed,
                           int64_t n, int64_t k, Out out, int32_t *ws, hipStream_t s)
{
    const int slices = gemv3sum_slices(1, n, k);
    // at most one block per CU in total (the tables take most of the LDS, so
    // a block more than the CUs would run in a second round on its own)
    int64_t rgroups = 256 / slices;
    rgroups = rgroups < 1 ? 1 : rgroups;
    int64_t rows_per = (n + rgroups - 1) / rgroups;
    rows_per = (rows_per + 15) / 16 * 16;
    rgroups = (n + rows_per - 1) / rows_per;
    hipLaunchKernelGGL(gemv3sum_kernel, dim3((unsigned)rgroups, (unsigned)slices),
                       dim3(64 * S3_WAVES), 0, s,
                       xq, rowsum, k, packed, n, pack3_pitch(k), rows_per, out,
                       slices > 1 ? ws : (int32_t *)nullptr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || slices == 1) return e;
    return launch_splitk_finish(ws, rowsum, 1, n, slices, out, n, s);
}

}  // namespace bl
