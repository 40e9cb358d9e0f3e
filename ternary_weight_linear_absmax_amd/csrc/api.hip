// C ABI of libbitlinear: host-side argument checks, kernel-path dispatch and
// launches.  Nothing here allocates, frees or synchronises.
#include <mutex>

#include "../../include/bitlinear.h"
#include "internal.h"

namespace {

constexpr int64_t kMaxElems = (int64_t)1 << 40;   // bound on N*K and M*K (grid sizes)

inline bool al16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
inline bool al4(const void *p) { return ((uintptr_t)p & 3u) == 0; }
inline bool good_dtype(int d) { return d == BL_F32 || d == BL_BF16; }
inline bool good_layout(int l) { return l == BL_PACK2 || l == BL_PACK3; }
inline bool good_k(int64_t k) { return k >= 1 && k <= BITLINEAR_MAX_K; }

inline int hip_status(hipError_t e) { return e == hipSuccess ? BL_OK : BL_ERR_HIP; }

inline bool known_path(int p)
{
    return p == BL_PATH_AUTO || p == BL_PATH_GEMV || p == BL_PATH_MFMA || p == BL_PATH_SKINNY ||
           p == BL_PATH_MFMA_WIDE;
}

// M = 1, 2: the vector kernel reads each weight word once per pass of up to
// four tokens and is the fastest; 3..16 tokens: the weight-streaming
// matrix-core kernel (one pass over the weights for all tokens), measured
// faster than the tiled GEMM on every 2B- and 70B-class matrix; 17..32 tokens
// (a second group of 16 token slots): still faster on matrices of up to 8192
// rows, slower on the 13824- and 28672-row ones; more: a tiled GEMM.
int choose_path(int64_t m, int64_t n, int64_t k, int layout)
{
    if (layout == BL_PACK3 || m <= 2) return BL_PATH_GEMV;
    if ((m <= 16 || (m <= 32 && n <= 8192)) && bl::skinny_supported(m, n, k))
        return BL_PATH_SKINNY;
    if (m <= 4) return BL_PATH_GEMV;
    return bl::gemm_preferred_variant(m, n, k) == bl::GEMM_WIDE ? BL_PATH_MFMA_WIDE : BL_PATH_MFMA;
}

// Whether an explicitly requested path can run the shape and layout.
bool path_runs(int path, int64_t m, int64_t n, int64_t k, int layout)
{
    if (layout == BL_PACK3) return path == BL_PATH_GEMV;
    if (path == BL_PATH_SKINNY) return bl::skinny_supported(m, n, k);
    if (path == BL_PATH_MFMA_WIDE) return k % 16 == 0;
    return true;
}

// Workspace bytes the chosen path needs (partial sums of a split k range).
int64_t workspace_need(int path, int64_t m, int64_t n, int64_t k, int layout = BL_PACK2)
{
    if (layout == BL_PACK3) return bl::gemv3_workspace_bytes(m, n, k);
    if (path == BL_PATH_MFMA) return bl::gemm_workspace_bytes(m, n, k, bl::GEMM_TILED);
    if (path == BL_PATH_MFMA_WIDE) return bl::gemm_workspace_bytes(m, n, k, bl::GEMM_WIDE);
    if (path == BL_PATH_SKINNY) return bl::skinny_workspace_bytes(m, n, k);
    return 0;
}

// One product on a resolved path (arguments already checked).
hipError_t launch_product(int path, int layout, const int8_t *xq, const int32_t *rowsum,
                          int64_t m, const uint8_t *packed, int64_t n, int64_t k, bl::Out out,
                          void *workspace, hipStream_t stream)
{
    if (layout == BL_PACK3)
        return bl::launch_gemv_pack3(xq, rowsum, m, packed, n, k, out, workspace, stream);
    if (path == BL_PATH_GEMV) return bl::launch_gemv_pack2(xq, rowsum, m, packed, n, k, out, stream);
    if (path == BL_PATH_SKINNY)
        return bl::launch_skinny_pack2(xq, rowsum, m, packed, n, k, out, workspace, stream);
    return bl::launch_gemm_pack2(xq, rowsum, m, packed, n, k, out, workspace, stream,
                                 path == BL_PATH_MFMA_WIDE ? bl::GEMM_WIDE : bl::GEMM_TILED);
}

// Shared body of bitlinear_forward_ex and bitlinear_matmul_i32.
int run_product(const int8_t *xq, const float *scale, const int32_t *rowsum, int64_t m,
                const uint8_t *packed, int layout, const float *gamma, int64_t n, int64_t k,
                float *y, int32_t *acc, void *workspace, int64_t workspace_bytes, int path,
                hipStream_t stream)
{
    if (!good_layout(layout)) return BL_ERR_LAYOUT;
    if (!known_path(path)) return BL_ERR_PATH;
    if (m < 0 || n < 0 || !good_k(k)) return BL_ERR_SHAPE;
    if (m > 0 && k > kMaxElems / m) return BL_ERR_SHAPE;
    if (n > 0 && k > kMaxElems / n) return BL_ERR_SHAPE;
    if (m > 0 && n > kMaxElems / m) return BL_ERR_SHAPE;
    if (path == BL_PATH_AUTO) path = choose_path(m, n, k, layout);
    if (layout == BL_PACK3 && path != BL_PATH_GEMV) return BL_ERR_PATH;
    if (m > 0 && n > 0 && !path_runs(path, m, n, k, layout)) return BL_ERR_PATH;
    if (m == 0 || n == 0) return BL_OK;    // empty product: buffers may be NULL
    if (!xq || !rowsum || !packed || (!y && !acc)) return BL_ERR_NULL;
    if (y && (!scale || !gamma)) return BL_ERR_NULL;
    if (!al16(xq) || !al16(packed) || !al4(rowsum)) return BL_ERR_ALIGN;
    if (y && (!al4(y) || !al4(scale) || !al4(gamma))) return BL_ERR_ALIGN;
    if (acc && !al4(acc)) return BL_ERR_ALIGN;
    const int64_t need = workspace_need(path, m, n, k, layout);
    if (need > 0 && (!workspace || workspace_bytes < need)) return BL_ERR_WORKSPACE;
    if (need > 0 && !al16(workspace)) return BL_ERR_ALIGN;

    bl::Out out{scale, gamma, y, acc};
    return hip_status(launch_product(path, layout, xq, rowsum, m, packed, n, k, out, workspace,
                                     stream));
}

}  // namespace

extern "C" {

int64_t bitlinear_packed_row_bytes(int64_t K, int layout)
{
    if (K < 1 || !good_layout(layout)) return 0;
    return layout == BL_PACK2 ? bl::pack2_pitch(K) : bl::pack3_pitch(K);
}

int64_t bitlinear_packed_bytes(int64_t N, int64_t K, int layout)
{
    if (N < 0) return 0;
    return N * bitlinear_packed_row_bytes(K, layout);
}

int64_t bitlinear_quantize_weights_workspace_bytes(int64_t N, int64_t K)
{
    if (N < 1 || K < 1 || K > kMaxElems / N) return 0;
    return bl::gamma_workspace_bytes(N * K);
}

int64_t bitlinear_forward_workspace_bytes(int64_t M, int64_t N, int64_t K, int layout)
{
    if (M < 1 || N < 1 || !good_k(K) || !good_layout(layout)) return 0;
    if (layout == BL_PACK3) return bl::gemv3_workspace_bytes(M, N, K);
    // the largest need over the paths the caller may force
    int64_t need = bl::skinny_workspace_bytes(M, N, K);
    const int64_t g = bl::gemm_workspace_bytes(M, N, K, bl::GEMM_TILED);
    need = g > need ? g : need;
    if (K % 16 == 0) {
        const int64_t w = bl::gemm_workspace_bytes(M, N, K, bl::GEMM_WIDE);
        need = w > need ? w : need;
    }
    return need;
}

int bitlinear_forward_path(int64_t M, int64_t N, int64_t K, int layout)
{
    return choose_path(M, N, K, layout);
}

const char *bitlinear_status_string(int status)
{
    switch (status) {
    case BL_OK: return "ok";
    case BL_ERR_NULL: return "a required pointer is NULL";
    case BL_ERR_SHAPE: return "invalid size (negative, zero where not allowed, or too large)";
    case BL_ERR_ALIGN: return "a device pointer is not suitably aligned (16 bytes for data)";
    case BL_ERR_DTYPE: return "unknown element type";
    case BL_ERR_LAYOUT: return "unknown packed layout";
    case BL_ERR_WORKSPACE: return "workspace smaller than the size query returned";
    case BL_ERR_HIP: return "a HIP launch or runtime call failed";
    case BL_ERR_PATH: return "the requested kernel path cannot run this shape or layout";
    case BL_ERR_SCRATCH:
        return "the product needs more scratch than the library's static buffer holds "
               "(BITLINEAR_NOALLOC_SCRATCH_BYTES); call bitlinear_forward_ex with a workspace";
    default: return "unknown status";
    }
}

int bitlinear_quantize_weights(const void *W, int dtype, int64_t N, int64_t K, int layout,
                               uint8_t *packed, float *gamma, void *workspace,
                               int64_t workspace_bytes, hipStream_t stream)
{
    if (!W || !packed || !gamma || !workspace) return BL_ERR_NULL;
    if (!good_dtype(dtype)) return BL_ERR_DTYPE;
    if (!good_layout(layout)) return BL_ERR_LAYOUT;
    if (N < 1 || !good_k(K) || K > kMaxElems / N) return BL_ERR_SHAPE;
    if (!al16(W) || !al16(packed) || !al16(workspace) || !al4(gamma)) return BL_ERR_ALIGN;
    if (workspace_bytes < bitlinear_quantize_weights_workspace_bytes(N, K)) return BL_ERR_WORKSPACE;
    hipError_t e = bl::launch_gamma(W, dtype, N, K, workspace, gamma, stream);
    if (e == hipSuccess) e = bl::launch_pack(W, dtype, N, K, layout, gamma, packed, stream);
    return hip_status(e);
}

int bitlinear_quantize_weights_binary(const void *W, int dtype, int64_t N, int64_t K, int layout,
                                      uint8_t *packed, float *beta, void *workspace,
                                      int64_t workspace_bytes, hipStream_t stream)
{
    if (!W || !packed || !beta || !workspace) return BL_ERR_NULL;
    if (!good_dtype(dtype)) return BL_ERR_DTYPE;
    if (!good_layout(layout)) return BL_ERR_LAYOUT;
    if (N < 1 || !good_k(K) || K > kMaxElems / N) return BL_ERR_SHAPE;
    if (!al16(W) || !al16(packed) || !al16(workspace) || !al4(beta)) return BL_ERR_ALIGN;
    if (workspace_bytes < bitlinear_quantize_weights_workspace_bytes(N, K)) return BL_ERR_WORKSPACE;
    hipError_t e = bl::launch_gamma(W, dtype, N, K, workspace, beta, stream);
    if (e == hipSuccess) e = bl::launch_pack(W, dtype, N, K, layout, beta, packed, stream, true);
    return hip_status(e);
}

int bitlinear_quantize_weights_binary_groups(const void *W, int dtype, int64_t N, int64_t K,
                                             int64_t groups, int layout, uint8_t *packed,
                                             float *beta, void *workspace,
                                             int64_t workspace_bytes, hipStream_t stream)
{
    if (!W || !packed || !beta || !workspace) return BL_ERR_NULL;
    if (!good_dtype(dtype)) return BL_ERR_DTYPE;
    if (!good_layout(layout)) return BL_ERR_LAYOUT;
    if (N < 1 || !good_k(K) || K > kMaxElems / N) return BL_ERR_SHAPE;
    if (groups < 1 || groups > N || N % groups != 0) return BL_ERR_SHAPE;
    const int64_t rows = N / groups;
    const int64_t esz = dtype == BL_BF16 ? 2 : 4;
    if (!al16(W) || !al16(packed) || !al16(workspace) || !al4(beta)) return BL_ERR_ALIGN;
    if (groups > 1 && (rows * K * esz) % 16 != 0) return BL_ERR_ALIGN;   // each group's start
    if (workspace_bytes < bitlinear_quantize_weights_workspace_bytes(N, K)) return BL_ERR_WORKSPACE;
    // groups one after another on the stream share the workspace
    hipError_t e = hipSuccess;
    for (int64_t g = 0; g < groups && e == hipSuccess; ++g)
        e = bl::launch_gamma((const uint8_t *)W + g * rows * K * esz, dtype, rows, K, workspace,
                             beta + g, stream);
    if (e == hipSuccess) e = bl::launch_pack(W, dtype, N, K, layout, beta, packed, stream, true);
    return hip_status(e);
}

int bitlinear_quantize_act_bits(const void *x, int dtype, int64_t M, int64_t K, int bits,
                                int8_t *xq, float *scale, int32_t *rowsum, hipStream_t stream)
{
    if (!good_dtype(dtype)) return BL_ERR_DTYPE;
    if (bits < 2 || bits > 8) return BL_ERR_SHAPE;
    if (M < 0 || !good_k(K) || (M > 0 && K > kMaxElems / M) || M > 0x7FFFFFFF)
        return BL_ERR_SHAPE;
    if (M == 0) return BL_OK;
    if (!x || !xq || !scale) return BL_ERR_NULL;
    if (!al16(x) || !al16(xq) || !al4(scale) || (rowsum && !al4(rowsum))) return BL_ERR_ALIGN;
    return hip_status(
        bl::launch_quant_act(x, dtype, M, K, xq, scale, rowsum, stream, (1 << (bits - 1)) - 1));
}

int bitlinear_backward_input(const void *grad_y, int dtype, int64_t M, int64_t N,
                             const uint8_t *packed, int layout, const float *gamma, int64_t K,
                             float *grad_x, hipStream_t stream)
{
    if (!good_dtype(dtype)) return BL_ERR_DTYPE;
    if (!good_layout(layout)) return BL_ERR_LAYOUT;
    if (layout != BL_PACK2) return BL_ERR_LAYOUT;
    if (M < 0 || N < 0 || !good_k(K)) return BL_ERR_SHAPE;
    if ((M > 0 && N > kMaxElems / M) || (M > 0 && K > kMaxElems / M) ||
        (N > 0 && K > kMaxElems / N) || M > (int64_t)65535 * 64)
        return BL_ERR_SHAPE;
    if (M == 0) return BL_OK;
    if (!grad_x || !gamma || (N > 0 && (!grad_y || !packed))) return BL_ERR_NULL;
    if ((grad_y && !al4(grad_y)) || !al4(grad_x) || !al4(gamma) || (packed && !al16(packed)))
        return BL_ERR_ALIGN;
    return hip_status(
        bl::launch_backward_input(grad_y, dtype, M, N, packed, K, gamma, grad_x, stream));
}

int bitlinear_quantize_act(const void *x, int dtype, int64_t M, int64_t K, int8_t *xq,
                           float *scale, int32_t *rowsum, hipStream_t stream)
{
    if (!good_dtype(dtype)) return BL_ERR_DTYPE;
    if (M < 0 || !good_k(K) || (M > 0 && K > kMaxElems / M) || M > 0x7FFFFFFF)
        return BL_ERR_SHAPE;
    if (M == 0) return BL_OK;              // empty batch: buffers may be NULL
    if (!x || !xq || !scale) return BL_ERR_NULL;
    if (!al16(x) || !al16(xq) || !al4(scale) || (rowsum && !al4(rowsum))) return BL_ERR_ALIGN;
    return hip_status(bl::launch_quant_act(x, dtype, M, K, xq, scale, rowsum, stream));
}

int bitlinear_forward(const int8_t *xq, const float *scale, const int32_t *rowsum, int64_t M,
                      const uint8_t *packed, int layout, const float *gamma, int64_t N,
                      int64_t K, float *y, void *workspace, int64_t workspace_bytes,
                      hipStream_t stream)
{
    return run_product(xq, scale, rowsum, M, packed, layout, gamma, N, K, y, nullptr, workspace,
                       workspace_bytes, BL_PATH_AUTO, stream);
}

int bitlinear_forward_ex(const int8_t *xq, const float *scale, const int32_t *rowsum,
                         int64_t M, const uint8_t *packed, int layout, const float *gamma,
                         int64_t N, int64_t K, float *y, void *workspace,
                         int64_t workspace_bytes, int path, hipStream_t stream)
{
    return run_product(xq, scale, rowsum, M, packed, layout, gamma, N, K, y, nullptr, workspace,
                       workspace_bytes, path, stream);
}

}  // extern "C"

namespace {

// Scratch of the allocation-free forward: one array per GPU, held for the
// life of the process.  Host code never passes the array's name to a kernel
// (in host code it is a stand-in, not a device address): the device address
// is looked up once per device, with that device current, and kept.
__device__ __attribute__((aligned(256))) uint8_t scratch[BITLINEAR_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void *g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of the current device's scratch array.
hipError_t scratch_address(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(g_scratch_once[dev], [dev] {
        void *p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
    });
    *out = g_scratch_ptr[dev];
    return g_scratch_err[dev];
}

}  // namespace

extern "C" {

int bitlinear_forward_noalloc(const int8_t *xq, const float *scale, const int32_t *rowsum,
                              int64_t M, const uint8_t *packed, int layout, const float *gamma,
                              int64_t N, int64_t K, float *y, int path, hipStream_t stream)
{
    // shape, layout and path checks first (no HIP call for a rejected call)
    if (!good_layout(layout)) return BL_ERR_LAYOUT;
    if (!known_path(path)) return BL_ERR_PATH;
    if (M < 0 || N < 0 || !good_k(K)) return BL_ERR_SHAPE;
    if ((M > 0 && K > kMaxElems / M) || (N > 0 && K > kMaxElems / N) ||
        (M > 0 && N > kMaxElems / M))
        return BL_ERR_SHAPE;
    const int p = path == BL_PATH_AUTO ? choose_path(M, N, K, layout) : path;
    if (M > 0 && N > 0 && path_runs(p, M, N, K, layout) &&
        workspace_need(p, M, N, K, layout) > (int64_t)BITLINEAR_NOALLOC_SCRATCH_BYTES)
        return BL_ERR_SCRATCH;
    void *ws = nullptr;
    if (M > 0 && N > 0 && workspace_need(p, M, N, K, layout) > 0 &&
        scratch_address(&ws) != hipSuccess)
        return BL_ERR_HIP;
    return run_product(xq, scale, rowsum, M, packed, layout, gamma, N, K, y, nullptr, ws,
                       ws ? (int64_t)BITLINEAR_NOALLOC_SCRATCH_BYTES : 0, path, stream);
}

int bitlinear_forward_groups(const int8_t *xq, const float *scale, const int32_t *rowsum,
                             int64_t M, const uint8_t *packed, int layout, const float *beta,
                             int64_t groups, int64_t N, int64_t K, float *y, void *workspace,
                             int64_t workspace_bytes, int path, hipStream_t stream)
{
    if (groups < 1 || (N > 0 && (groups > N || N % groups != 0))) return BL_ERR_SHAPE;
    if (M > 0 && N > 0) {
        if (!scale || !beta || !y) return BL_ERR_NULL;
        if (!al4(scale) || !al4(beta) || !al4(y)) return BL_ERR_ALIGN;
    }
    // the exact int32 accumulators into y's memory, then rescaled in place
    const int r = run_product(xq, nullptr, rowsum, M, packed, layout, nullptr, N, K, nullptr,
                              (int32_t *)y, workspace, workspace_bytes, path, stream);
    if (r != BL_OK || M == 0 || N == 0) return r;
    return hip_status(bl::launch_group_rescale(y, scale, beta, M, N, N / groups, stream));
}

int bitlinear_matmul_i32(const int8_t *xq, const int32_t *rowsum, int64_t M,
                         const uint8_t *packed, int layout, int64_t N, int64_t K, int32_t *acc,
                         void *workspace, int64_t workspace_bytes, int path, hipStream_t stream)
{
    return run_product(xq, nullptr, rowsum, M, packed, layout, nullptr, N, K, nullptr, acc,
                       workspace, workspace_bytes, path, stream);
}

int bitlinear_quantize_forward(const void *x, int dtype, int64_t M, int64_t K, int8_t *xq,
                               float *scale, int32_t *rowsum, const uint8_t *packed, int layout,
                               const float *gamma, int64_t N, float *y, void *workspace,
                               int64_t workspace_bytes, int path, hipStream_t stream)
{
    if (!good_dtype(dtype)) return BL_ERR_DTYPE;
    if (!good_layout(layout)) return BL_ERR_LAYOUT;
    if (!known_path(path)) return BL_ERR_PATH;
    if (M < 0 || N < 0 || !good_k(K) || M > 0x7FFFFFFF) return BL_ERR_SHAPE;
    if ((M > 0 && K > kMaxElems / M) || (N > 0 && K > kMaxElems / N) ||
        (M > 0 && N > kMaxElems / M))
        return BL_ERR_SHAPE;
    if (path == BL_PATH_AUTO) path = choose_path(M, N, K, layout);
    if (layout == BL_PACK3 && path != BL_PATH_GEMV) return BL_ERR_PATH;
    if (M > 0 && N > 0 && !path_runs(path, M, N, K, layout)) return BL_ERR_PATH;
    if (M == 0) return BL_OK;
    if (!x || !xq || !scale || !rowsum) return BL_ERR_NULL;
    if (!al16(x) || !al16(xq) || !al4(scale) || !al4(rowsum)) return BL_ERR_ALIGN;
    if (N == 0) return hip_status(bl::launch_quant_act(x, dtype, M, K, xq, scale, rowsum, stream));
    if (!packed || !gamma || !y) return BL_ERR_NULL;
    if (!al16(packed) || !al4(gamma) || !al4(y)) return BL_ERR_ALIGN;
    const int64_t need = workspace_need(path, M, N, K, layout);
    if (need > 0 && (!workspace || workspace_bytes < need)) return BL_ERR_WORKSPACE;
    if (need > 0 && !al16(workspace)) return BL_ERR_ALIGN;

    bl::Out out{scale, gamma, y, nullptr};
    if (layout == BL_PACK2 && path == BL_PATH_GEMV && bl::gemv_fused_supported(M, N, K, dtype))
        return hip_status(bl::launch_gemv_pack2_fused(x, dtype, xq, scale, rowsum, packed, N, K,
                                                      out, stream));
    hipError_t e = bl::launch_quant_act(x, dtype, M, K, xq, scale, rowsum, stream);
    if (e != hipSuccess) return BL_ERR_HIP;
    return hip_status(launch_product(path, layout, xq, rowsum, M, packed, N, K, out, workspace,
                                     stream));
}

namespace {

int glue_common(int64_t M, int64_t K, float eps, int8_t *xq, float *scale, int32_t *rowsum)
{
    if (M < 0 || K < 1 || K > bl::GLUE_MAX_K || M > 0x7FFFFFFF) return BL_ERR_SHAPE;
    if (!(eps >= 0.0f)) return BL_ERR_SHAPE;
    if (M == 0) return BL_OK;
    if (!xq || !scale || !rowsum) return BL_ERR_NULL;
    if (!al16(xq) || !al4(scale) || !al4(rowsum)) return BL_ERR_ALIGN;
    return 1;   // proceed
}

}  // namespace

int bitlinear_residual_rmsnorm_quantize(float *x, const float *add, int64_t M, int64_t K,
                                        float eps, int8_t *xq, float *scale, int32_t *rowsum,
                                        hipStream_t stream)
{
    const int c = glue_common(M, K, eps, xq, scale, rowsum);
    if (c != 1) return c;
    if (!x) return BL_ERR_NULL;
    if (!al4(x) || (add && !al4(add))) return BL_ERR_ALIGN;
    bl::GlueArgs a{x, add, nullptr, 0, 0, 1, 1};
    return hip_status(bl::launch_glue(bl::GLUE_RESIDUAL, a, M, K, eps, xq, scale, rowsum, stream));
}

int bitlinear_gqa_rmsnorm_quantize(const float *qkv, int64_t M, int64_t ld, int64_t v_col,
                                   int64_t heads, int64_t kv_heads, int64_t head_dim, float eps,
                                   int8_t *xq, float *scale, int32_t *rowsum, hipStream_t stream)
{
    if (heads < 1 || kv_heads < 1 || head_dim < 1 || heads % kv_heads != 0) return BL_ERR_SHAPE;
    if (heads > bl::GLUE_MAX_K || head_dim > bl::GLUE_MAX_K) return BL_ERR_SHAPE;
    if (v_col < 0 || ld < 1 || v_col + kv_heads * head_dim > ld) return BL_ERR_SHAPE;
    const int c = glue_common(M, heads * head_dim, eps, xq, scale, rowsum);
    if (c != 1) return c;
    if (!qkv) return BL_ERR_NULL;
    if (!al4(qkv)) return BL_ERR_ALIGN;
    bl::GlueArgs a{nullptr, nullptr, qkv, ld, v_col, heads / kv_heads, head_dim};
    return hip_status(bl::launch_glue(bl::GLUE_GQA, a, M, heads * head_dim, eps, xq, scale,
                                      rowsum, stream));
}

int bitlinear_relu2_rmsnorm_quantize(const float *gate_up, int64_t M, int64_t ld, int64_t F,
                                     float eps, int8_t *xq, float *scale, int32_t *rowsum,
                                     hipStream_t stream)
{
    if (F < 1 || ld < 2 * F) return BL_ERR_SHAPE;
    const int c = glue_common(M, F, eps, xq, scale, rowsum);
    if (c != 1) return c;
    if (!gate_up) return BL_ERR_NULL;
    if (!al4(gate_up)) return BL_ERR_ALIGN;
    bl::GlueArgs a{nullptr, nullptr, gate_up, ld, F, 1, 1};
    return hip_status(bl::launch_glue(bl::GLUE_RELU2, a, M, F, eps, xq, scale, rowsum, stream));
}

namespace {

// Bytes of the product's own workspace (its split partial sums, whether the
// product or the glue finishes them), rounded up so that the float output
// that follows it stays 256-byte aligned.
int gemm_variant_of(int path)
{
    return path == BL_PATH_MFMA_WIDE ? bl::GEMM_WIDE : bl::GEMM_TILED;
}

int64_t fused_product_ws(int64_t m, int64_t n, int64_t k)
{
    int64_t p = bitlinear_forward_workspace_bytes(m, n, k, BL_PACK2);
    const int path = choose_path(m, n, k, BL_PACK2);
    const int64_t part = bl::gemm_partial_workspace_bytes(m, n, k, gemm_variant_of(path));
    p = part > p ? part : p;
    return (p + 255) / 256 * 256;
}

// BitLinear product of 2-bit weights followed by one of the glue forms.  When
// the tiled GEMM splits the k range, its int32 slices stay in the workspace
// and the glue kernel finishes them (no finish launch); otherwise the product
// writes its float output into the workspace and the glue reads it.
int forward_glue(int mode, const int8_t *xq, const float *scale, const int32_t *rowsum,
                 int64_t M, int64_t K, const uint8_t *packed, const float *gamma, int64_t N,
                 bl::GlueArgs a, int64_t gk, float eps, int8_t *xq_out, float *scale_out,
                 int32_t *rowsum_out, void *workspace, int64_t workspace_bytes,
                 hipStream_t stream)
{
    if (N < 1 || !good_k(K) || M > 0x7FFFFFFF) return BL_ERR_SHAPE;
    if (M > 0 && (K > kMaxElems / M || N > kMaxElems / M)) return BL_ERR_SHAPE;
    if (K > kMaxElems / N) return BL_ERR_SHAPE;
    const int c = glue_common(M, gk, eps, xq_out, scale_out, rowsum_out);
    if (c != 1) return c;
    if (!xq || !scale || !rowsum || !packed || !gamma || !workspace) return BL_ERR_NULL;
    if (!al16(xq) || !al16(packed) || !al4(scale) || !al4(rowsum) || !al4(gamma) ||
        !al16(workspace))
        return BL_ERR_ALIGN;
    const int64_t pws = fused_product_ws(M, N, K);
    if (workspace_bytes < pws + 4 * M * N) return BL_ERR_WORKSPACE;

    const int path = choose_path(M, N, K, BL_PACK2);
    const bool gemm = path == BL_PATH_MFMA || path == BL_PATH_MFMA_WIDE;
    const int splits = gemm ? bl::gemm_partial_splits(M, N, K, gemm_variant_of(path)) : 0;
    if (splits > 1) {
        bl::Out out{scale, gamma, nullptr, nullptr};
        hipError_t e = bl::launch_gemm_pack2_partials(xq, rowsum, M, packed, N, K, out,
                                                      (int32_t *)workspace, stream,
                                                      gemm_variant_of(path));
        if (e != hipSuccess) return BL_ERR_HIP;
        a.part = (const int32_t *)workspace;
        a.splits = splits;
        a.pm = M;
        a.p_rowsum = rowsum;
        a.p_scale = scale;
        a.p_gamma = gamma;
        if (mode == bl::GLUE_RESIDUAL) a.ld = N;
    } else {
        float *y = (float *)((uint8_t *)workspace + pws);
        const int r = run_product(xq, scale, rowsum, M, packed, BL_PACK2, gamma, N, K, y, nullptr,
                                  workspace, pws, path, stream);
        if (r != BL_OK) return r;
        if (mode == bl::GLUE_RESIDUAL) a.add = y;
        else a.src = y;
    }
    return hip_status(bl::launch_glue(mode, a, M, gk, eps, xq_out, scale_out, rowsum_out, stream));
}

}  // namespace

int64_t bitlinear_forward_glue_workspace_bytes(int64_t M, int64_t N, int64_t K)
{
    if (M < 1 || N < 1 || !good_k(K) || M > 0x7FFFFFFF) return 0;
    if (K > kMaxElems / M || N > kMaxElems / M || K > kMaxElems / N) return 0;
    return fused_product_ws(M, N, K) + 4 * M * N;
}

int bitlinear_forward_residual_rmsnorm_quantize(const int8_t *xq, const float *scale,
                                                const int32_t *rowsum, int64_t M, int64_t K,
                                                const uint8_t *packed, const float *gamma,
                                                int64_t N, float *x, float eps, int8_t *xq_out,
                                                float *scale_out, int32_t *rowsum_out,
                                                void *workspace, int64_t workspace_bytes,
                                                hipStream_t stream)
{
    if (M > 0 && !x) return BL_ERR_NULL;
    if (!al4(x)) return BL_ERR_ALIGN;
    bl::GlueArgs a{x, nullptr, nullptr, 0, 0, 1, 1};
    return forward_glue(bl::GLUE_RESIDUAL, xq, scale, rowsum, M, K, packed, gamma, N, a, N, eps,
                        xq_out, scale_out, rowsum_out, workspace, workspace_bytes, stream);
}

int bitlinear_forward_gqa_rmsnorm_quantize(const int8_t *xq, const float *scale,
                                           const int32_t *rowsum, int64_t M, int64_t K,
                                           const uint8_t *packed, const float *gamma, int64_t N,
                                           int64_t v_col, int64_t heads, int64_t kv_heads,
                                           int64_t head_dim, float eps, int8_t *xq_out,
                                           float *scale_out, int32_t *rowsum_out,
                                           void *workspace, int64_t workspace_bytes,
                                           hipStream_t stream)
{
    if (heads < 1 || kv_heads < 1 || head_dim < 1 || heads % kv_heads != 0) return BL_ERR_SHAPE;
    if (heads > bl::GLUE_MAX_K || head_dim > bl::GLUE_MAX_K) return BL_ERR_SHAPE;
    if (v_col < 0 || N < 1 || v_col + kv_heads * head_dim > N) return BL_ERR_SHAPE;
    bl::GlueArgs a{nullptr, nullptr, nullptr, N, v_col, heads / kv_heads, head_dim};
    return forward_glue(bl::GLUE_GQA, xq, scale, rowsum, M, K, packed, gamma, N, a,
                        heads * head_dim, eps, xq_out, scale_out, rowsum_out, workspace,
                        workspace_bytes, stream);
}

int bitlinear_forward_relu2_rmsnorm_quantize(const int8_t *xq, const float *scale,
                                             const int32_t *rowsum, int64_t M, int64_t K,
                                             const uint8_t *packed, const float *gamma,
                                             int64_t N, int64_t F, float eps, int8_t *xq_out,
                                             float *scale_out, int32_t *rowsum_out,
                                             void *workspace, int64_t workspace_bytes,
                                             hipStream_t stream)
{
    if (F < 1 || N < 2 * F) return BL_ERR_SHAPE;
    bl::GlueArgs a{nullptr, nullptr, nullptr, N, F, 1, 1};
    return forward_glue(bl::GLUE_RELU2, xq, scale, rowsum, M, K, packed, gamma, N, a, F, eps,
                        xq_out, scale_out, rowsum_out, workspace, workspace_bytes, stream);
}

int bitlinear_norm_forward(int input, const void *src, const float *add, float *x_out,
                           int64_t v_col, int64_t heads, int64_t kv_heads, int64_t head_dim,
                           int64_t K, float eps, const uint8_t *packed, const float *gamma,
                           int64_t N, int relu2, void *out, int8_t *xq, float *scale,
                           int32_t *rowsum, hipStream_t stream)
{
    if (input != BL_NORM_RESIDUAL && input != BL_NORM_GQA && input != BL_NORM_F64)
        return BL_ERR_DTYPE;
    if (relu2 != 0 && relu2 != 1) return BL_ERR_SHAPE;
    if (!(eps >= 0.0f)) return BL_ERR_SHAPE;
    if (input == BL_NORM_GQA) {
        if (heads < 1 || kv_heads < 1 || head_dim < 1 || heads % kv_heads != 0) return BL_ERR_SHAPE;
        if (heads > bl::NORM_MAX_K || head_dim > bl::NORM_MAX_K || v_col < 0) return BL_ERR_SHAPE;
        if (heads * head_dim != K) return BL_ERR_SHAPE;
    }
    if (K < 1 || K > bl::NORM_MAX_K || N < 1 || K > kMaxElems / N) return BL_ERR_SHAPE;
    if (relu2 && N % 2 != 0) return BL_ERR_SHAPE;
    if (!bl::gemv_norm_supported(N, K)) return BL_ERR_SHAPE;
    if (!src || !packed || !gamma || !out) return BL_ERR_NULL;
    if (input == BL_NORM_RESIDUAL && add && !x_out) return BL_ERR_NULL;
    const bool f64 = input == BL_NORM_F64;
    if ((uintptr_t)src & (f64 ? 7u : 3u)) return BL_ERR_ALIGN;
    if ((add && !al4(add)) || (x_out && !al4(x_out)) || !al16(packed) || !al4(gamma))
        return BL_ERR_ALIGN;
    if ((uintptr_t)out & (relu2 ? 7u : 3u)) return BL_ERR_ALIGN;
    if ((scale && !al4(scale)) || (rowsum && !al4(rowsum))) return BL_ERR_ALIGN;
    bl::NormArgs a{};
    a.pro = input == BL_NORM_RESIDUAL ? bl::NORM_RESIDUAL
            : input == BL_NORM_GQA    ? bl::NORM_GQA
                                      : bl::NORM_F64;
    a.src = src;
    a.add = input == BL_NORM_RESIDUAL ? add : nullptr;
    a.x_out = x_out;
    a.col = v_col;
    a.group = input == BL_NORM_GQA ? heads / kv_heads : 1;
    a.head_dim = input == BL_NORM_GQA ? head_dim : 1;
    a.eps = eps;
    a.xq = xq;
    a.scale = scale;
    a.rowsum = rowsum;
    a.f = N / 2;
    a.v = relu2 ? (double *)out : nullptr;
    bl::Out o{nullptr, gamma, relu2 ? nullptr : (float *)out, nullptr};
    return hip_status(bl::launch_gemv_norm(a, N, K, packed, o, relu2 != 0, stream));
}

int bitlinear_unpack_weights(const uint8_t *packed, int layout, int64_t N, int64_t K,
                             int8_t *trits, hipStream_t stream)
{
    if (!good_layout(layout)) return BL_ERR_LAYOUT;
    if (N < 0 || !good_k(K) || (N > 0 && K > kMaxElems / N)) return BL_ERR_SHAPE;
    if (N == 0) return BL_OK;
    if (!packed || !trits) return BL_ERR_NULL;
    if (!al16(packed)) return BL_ERR_ALIGN;
    return hip_status(bl::launch_unpack(packed, layout, N, K, trits, stream));
}

}  // extern "C"
