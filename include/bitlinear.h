/*
 * bitlinear.h - C ABI of the BitNet b1.58 BitLinear layer for AMD Instinct
 * MI355X (gfx950).
 *
 * The layer replaces a linear layer y = x W^T (no bias) with
 *   - weights quantised by their absolute mean gamma = mean|W| to ternary
 *     values t = clip(round(W / gamma), -1, 1);
 *   - activations quantised per token to 8 bits by their absolute maximum,
 *     q = round(x * s) with s = 127 / max|x|;
 *   - an exact integer product acc = q t^T, rescaled to y = acc * gamma / s.
 * Sources: "1-bit LLM era: Microsoft introduces BitNet b1.58" (cheatsheet.md),
 * section "What is BitNet b1.58?" (absmean weights, per-token activation
 * scaling, BitLinear in place of nn.Linear, no bias); the asi.tokyo article on
 * BitNet b1.58 2B4T (8-bit activations; four trits packed per byte, unpacked
 * next to the arithmetic units and multiplied with the 8-bit values); the
 * news.hada.io topic 20406 comment on ternary packing (five trits per byte).
 *
 * Conventions shared by every call
 *   - Shapes follow nn.Linear: x is [M, K] (M tokens), W is [N, K] (N output
 *     features), y is [M, N]; all row-major and dense.
 *   - Pointers marked "device" are HIP device pointers (or host-coherent memory
 *     a kernel may read); the caller owns every buffer.  The library never
 *     allocates, frees or keeps a pointer after the call returns.
 *   - Calls are asynchronous on `stream` (0 = the null stream).  Arguments are
 *     checked on the host before anything is launched; a failed check returns
 *     a negative bl_status and launches nothing.  A failed launch returns
 *     BL_ERR_HIP.  No host synchronisation happens inside any call.
 *   - Device pointers must be 16-byte aligned.  Sizes are element counts.
 *   - Inputs must be finite; NaN or infinite inputs give unspecified results.
 *   - M == 0 or N == 0 is an empty product and returns BL_OK without a
 *     launch (the buffers of an empty product may be NULL); K must be in
 *     [1, BITLINEAR_MAX_K].  Other size and layout checks come first.
 *   - Every call is stateless and re-entrant; calls on different streams may
 *     overlap if their buffers do not.  The one exception is
 *     bitlinear_forward_noalloc, whose calls on one GPU share a static
 *     scratch array.
 */
#ifndef BITLINEAR_H
#define BITLINEAR_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    BL_OK = 0,
    BL_ERR_NULL = -1,        /* a required pointer is NULL */
    BL_ERR_SHAPE = -2,       /* a size is negative, zero where it may not be, or too large */
    BL_ERR_ALIGN = -3,       /* a device pointer is not 16-byte aligned */
    BL_ERR_DTYPE = -4,       /* unknown bl_dtype */
    BL_ERR_LAYOUT = -5,      /* unknown bl_layout */
    BL_ERR_WORKSPACE = -6,   /* workspace smaller than the size query returned */
    BL_ERR_HIP = -7,         /* a HIP launch or runtime call failed */
    BL_ERR_PATH = -8,        /* the requested kernel path cannot run this shape */
    BL_ERR_SCRATCH = -9      /* the allocation-free call needs more scratch than it has */
} bl_status;

typedef enum {
    BL_F32 = 0,              /* IEEE binary32 */
    BL_BF16 = 1              /* bfloat16, stored as 16-bit words */
} bl_dtype;

typedef enum {
    /* Four trits per byte.  Row n of an [N, K] matrix occupies
     * bitlinear_packed_row_bytes(K, BL_PACK2) = 16 * ceil(K / 64) bytes.  Read
     * as little-endian 32-bit words, word g of a row holds k = 16g .. 16g+15:
     * trit k = 16g + 4i + j is stored in byte j of the word at bits 2i..2i+1
     * as the code t + 1 (0 for -1, 1 for 0, 2 for +1; code 3 never occurs).
     * So (word >> 2i) & 0x03030303 yields the codes of four consecutive k in
     * its four bytes.  Positions k >= K hold code 1 (trit 0). */
    BL_PACK2 = 0,
    /* Five trits per byte (base 3).  Byte j of a row is
     * sum_{i=0..4} (t[5j+i] + 1) * 3^i, the lowest k being the least
     * significant digit; positions k >= K are trit 0, and the row is padded to
     * bitlinear_packed_row_bytes(K, BL_PACK3) = 16 * ceil(ceil(K / 5) / 16)
     * bytes with the byte 121 (five zero trits). */
    BL_PACK3 = 1
} bl_layout;

typedef enum {
    BL_PATH_AUTO = 0,        /* choose by M, N, K and layout (the default): GEMV
                                for PACK3 and M <= 2; SKINNY for M <= 32 when it
                                can run the shape; else GEMV for M <= 4, above
                                that MFMA_WIDE for M >= 128 and N >= 512 with K
                                a multiple of 16, MFMA otherwise */
    BL_PATH_GEMV = 1,        /* vector dot-product kernel, tokens in passes of 4 */
    BL_PATH_MFMA = 2,        /* int8 matrix-core kernel with square-ish block
                                tiles, any M and K (PACK2 only) */
    BL_PATH_SKINNY = 3,      /* int8 matrix-core weight-streaming kernel for
                                1 <= M <= 64 and K a multiple of 256 (PACK2 only) */
    BL_PATH_MFMA_WIDE = 4    /* int8 matrix-core kernel with 64 x 512 block tiles,
                                any M, K a multiple of 16 (PACK2 only) */
} bl_path;

#define BITLINEAR_MAX_K (1 << 20)

/* ---- host-only size queries (pure; no HIP calls) ---------------------------- */

/* Bytes of one packed row; 0 for an unknown layout or K < 1. */
int64_t bitlinear_packed_row_bytes(int64_t K, int layout);

/* Bytes of a packed [N, K] matrix: N * bitlinear_packed_row_bytes(K, layout). */
int64_t bitlinear_packed_bytes(int64_t N, int64_t K, int layout);

/* Workspace that bitlinear_quantize_weights needs: 128 bytes per summing block,
 * min(2048, max(1, ceil(N*K / 8192))) blocks (partial sums of |w| as exact
 * multi-word integers; no initial contents needed); 0 for N < 1 or K < 1. */
int64_t bitlinear_quantize_weights_workspace_bytes(int64_t N, int64_t K);

/* Workspace that bitlinear_forward / bitlinear_matmul_i32 need for this shape
 * on any path (0 when none; then workspace may be NULL).  A non-empty
 * workspace is scratch for the int32 partial sums of the GEMM path, or of the
 * skinny path (M <= 16), when it splits the k range (one [M, N] int32 slice
 * per split, added in split order): it needs no initial contents, and calls
 * that share one workspace must not overlap. */
int64_t bitlinear_forward_workspace_bytes(int64_t M, int64_t N, int64_t K, int layout);

/* Kernel path that BL_PATH_AUTO selects for this shape (a bl_path value). */
int bitlinear_forward_path(int64_t M, int64_t N, int64_t K, int layout);

/* Static description of a status code. */
const char *bitlinear_status_string(int status);

/* ---- weights: absmean quantiser and packing (offline, once per matrix) ------
 * [cheatsheet.md BitNet b1.58 summary, "What is BitNet b1.58?", weight bullet;
 *  asi.tokyo 2B4T article, packing paragraph; news.hada.io 20406, packing
 *  comment]
 *
 * W       device, [N, K] of `dtype`.
 * packed  device, bitlinear_packed_bytes(N, K, layout) bytes, written.
 * gamma   device, one float, written: gamma = mean|W|: the sum of |w| is formed
 *         exactly (independent of element order) and rounded once to double,
 *         divided by N*K in double precision and rounded to float.  A NaN
 *         element gives gamma = NaN, else an infinite one gives +inf.
 * t       t = sign(w) when 2|w| > gamma, else 0: round-half-to-even of the
 *         exact quotient w / gamma, clipped to [-1, 1].
 * workspace  device, >= bitlinear_quantize_weights_workspace_bytes(N, K).
 * Requires N >= 1 (the mean of an empty matrix is undefined). */
int bitlinear_quantize_weights(const void *W, int dtype, int64_t N, int64_t K, int layout,
                               uint8_t *packed, float *gamma, void *workspace,
                               int64_t workspace_bytes, hipStream_t stream);

/* ---- weights, 1-bit variant: sign binariser (offline) ----------------------
 * [lumen-it.ai article on the original 1-bit BitNet: weights binarised to +1
 *  or -1 with the signum function; group quantisation for model parallelism]
 *
 * Same arguments, layout, packing and errors as bitlinear_quantize_weights,
 * with t = -1 for w < 0 and t = +1 otherwise (a zero weight of either sign
 * maps to +1; the pages give no tie rule), so the packed matrix holds no zero
 * trits and every product kernel runs it unchanged.
 * beta    device, one float, written: the scale of the binary weights, mean|W|
 *         computed exactly as gamma above (one group: the whole matrix on one
 *         device).  Pass it where the products take gamma. */
int bitlinear_quantize_weights_binary(const void *W, int dtype, int64_t N, int64_t K, int layout,
                                      uint8_t *packed, float *beta, void *workspace,
                                      int64_t workspace_bytes, hipStream_t stream);

/* ---- weights, 1-bit variant with group quantisation (offline) ----------------
 * [lumen-it.ai article on the original 1-bit BitNet: group quantisation and
 *  normalisation, so that the layer splits over devices with little
 *  communication]
 *
 * bitlinear_quantize_weights_binary with one scale per group: the N rows are
 * cut into `groups` equal groups of consecutive rows (the output features a
 * device would hold), and group g gets beta[g] = mean |W| over its rows,
 * computed exactly as gamma.  The packed trits are those of
 * bitlinear_quantize_weights_binary (the sign does not depend on the scale).
 * groups   1 <= groups <= N, groups divides N (BL_ERR_SHAPE otherwise).
 * beta     device, [groups] float, written.
 * Each group's rows must start 16-byte aligned: (N / groups) * K * element
 * size a multiple of 16 when groups > 1 (BL_ERR_ALIGN otherwise).  Same
 * workspace as bitlinear_quantize_weights (the groups reuse it in turn). */
int bitlinear_quantize_weights_binary_groups(const void *W, int dtype, int64_t N, int64_t K,
                                             int64_t groups, int layout, uint8_t *packed,
                                             float *beta, void *workspace,
                                             int64_t workspace_bytes, hipStream_t stream);

/* ---- activations: per-token absmax to int8 -----------------------------------
 * [cheatsheet.md BitNet b1.58 summary, "What is BitNet b1.58?", activation
 *  bullet; asi.tokyo 2B4T article, 8-bit messages; lumen-it.ai BitNet, absmax]
 *
 * x       device, [M, K] of `dtype`.
 * xq      device, [M, K] int8, written: clamp(rint(x * s), -127, 127) with
 *         float multiply and round-half-to-even.
 * scale   device, [M] float, written: s = 127 / max_k |x[m, k]| (IEEE float
 *         division), or 1 for an all-zero token (then xq is 0).
 * rowsum  device, [M] int32, written if not NULL: sum_k xq[m, k].
 */
int bitlinear_quantize_act(const void *x, int dtype, int64_t M, int64_t K, int8_t *xq,
                           float *scale, int32_t *rowsum, hipStream_t stream);

/* ---- activations with fewer bits ------------------------------------------------
 * [cheatsheet.md BitNet b1.58 summary, outlook: activations compressed below
 *  8 bits, to 4 bits or fewer]
 *
 * bitlinear_quantize_act with Q = 2^(bits-1) - 1 in place of 127:
 * s = Q / max_k |x[m, k]| (IEEE float division; 1 for an all-zero token) and
 * xq = clamp(rint(x * s), -Q, Q), stored as int8.  bits in [2, 8]
 * (BL_ERR_SHAPE otherwise); bits = 8 is bitlinear_quantize_act.  The products
 * take the result unchanged (y = acc * gamma / s). */
int bitlinear_quantize_act_bits(const void *x, int dtype, int64_t M, int64_t K, int bits,
                                int8_t *xq, float *scale, int32_t *rowsum, hipStream_t stream);

/* ---- forward: exact integer product and rescale ---------------------------------
 * [asi.tokyo 2B4T article, packing paragraph: unpack next to the arithmetic
 *  units and multiply with the 8-bit activations; cheatsheet.md summary:
 *  both quantiser scalings are undone at the output]
 *
 * xq, scale, rowsum  device, as written by bitlinear_quantize_act (rowsum is
 *         required and must equal sum_k xq[m, k]).
 * packed, gamma      device, as written by bitlinear_quantize_weights.
 * y       device, [M, N] float, written:
 *         y[m, n] = acc[m, n] * (gamma / scale[m]), the factor gamma / scale[m]
 *         formed in double precision and the product rounded once to float,
 *         acc[m, n] = sum_k t[n, k] * xq[m, k] computed exactly in int32.
 * workspace  device, >= bitlinear_forward_workspace_bytes(M, N, K, layout).
 */
int bitlinear_forward(const int8_t *xq, const float *scale, const int32_t *rowsum, int64_t M,
                      const uint8_t *packed, int layout, const float *gamma, int64_t N,
                      int64_t K, float *y, void *workspace, int64_t workspace_bytes,
                      hipStream_t stream);

/* bitlinear_forward with an explicit kernel path (bl_path); BL_ERR_PATH if that
 * path cannot run the shape or layout. */
int bitlinear_forward_ex(const int8_t *xq, const float *scale, const int32_t *rowsum,
                         int64_t M, const uint8_t *packed, int layout, const float *gamma,
                         int64_t N, int64_t K, float *y, void *workspace,
                         int64_t workspace_bytes, int path, hipStream_t stream);

/* bitlinear_forward_ex with one weight scale per group of N / groups
 * consecutive output features (bitlinear_quantize_weights_binary_groups):
 *   y[m, n] = acc[m, n] * (beta[n / (N / groups)] / scale[m]) (the factor in
 *   double precision, the product rounded once to float).
 * beta     device, [groups] float; groups divides N (BL_ERR_SHAPE otherwise).
 * The product writes the exact int32 accumulators into y's memory and a
 * second kernel rescales them in place (two launches).  Other arguments,
 * workspace and errors as for bitlinear_forward_ex. */
int bitlinear_forward_groups(const int8_t *xq, const float *scale, const int32_t *rowsum,
                             int64_t M, const uint8_t *packed, int layout, const float *beta,
                             int64_t groups, int64_t N, int64_t K, float *y, void *workspace,
                             int64_t workspace_bytes, int path, hipStream_t stream);

/* The same kernels without the rescale: acc[m, n] = sum_k t[n, k] * xq[m, k]
 * as int32 (device, [M, N]).  path as in bitlinear_forward_ex. */
int bitlinear_matmul_i32(const int8_t *xq, const int32_t *rowsum, int64_t M,
                         const uint8_t *packed, int layout, int64_t N, int64_t K,
                         int32_t *acc, void *workspace, int64_t workspace_bytes, int path,
                         hipStream_t stream);

/* ---- forward without any allocation ------------------------------------------------
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Same arguments, results and errors as bitlinear_forward_ex without the
 * workspace: the split-k partial sums go to a static scratch array of
 * BITLINEAR_NOALLOC_SCRATCH_BYTES in the library, one per GPU, which the GPU
 * holds until the process ends.  The call allocates and frees nothing.
 * Returns BL_ERR_SCRATCH, and launches nothing, when the shape needs more
 * scratch than that (bitlinear_forward_workspace_bytes tells how much a shape
 * needs on its path).  The scratch needs no initial contents and keeps the
 * last call's partial sums; calls that overlap on one GPU (other streams,
 * other host threads) share it and race, so serialise them.  The first call
 * on a device looks up the array's device address (hipGetSymbolAddress). */
#define BITLINEAR_NOALLOC_SCRATCH_BYTES ((size_t)14 << 20)

int bitlinear_forward_noalloc(const int8_t *xq, const float *scale, const int32_t *rowsum,
                              int64_t M, const uint8_t *packed, int layout, const float *gamma,
                              int64_t N, int64_t K, float *y, int path, hipStream_t stream);

/* ---- backward through BitLinear: input gradient -------------------------------
 * [lumen-it.ai BitNet article, training paragraph: straight-through estimators
 *  carry the gradient through the quantisers]
 *
 * With both quantisers passed straight through, the layer acts on x as the
 * matrix gamma * t, so
 *     grad_x[m, k] = gamma * sum_n grad_y[m, n] * t[n, k]
 * over the same packed weights (2-bit layout only; BL_ERR_LAYOUT for base-3),
 * in fp32 arithmetic.  The weight gradient passes straight through to the
 * latent weights (a dense product of grad_y and the activations) and is not
 * part of this library.
 * grad_y  device, [M, N] of `dtype` (bf16 or fp32), row-major, 4-byte aligned
 *         (may be NULL when N == 0).
 * packed  device, bitlinear_packed_bytes(N, K, BL_PACK2) bytes (may be NULL
 *         when N == 0: then grad_x is all zero).
 * gamma   device, one float: the scale the weights were quantised with.
 * grad_x  device, [M, K] float32, written.
 * M == 0: nothing to do.  M <= 65535 * 64. */
int bitlinear_backward_input(const void *grad_y, int dtype, int64_t M, int64_t N,
                             const uint8_t *packed, int layout, const float *gamma, int64_t K,
                             float *grad_x, hipStream_t stream);

/* ---- quantise and multiply in one call ---------------------------------------
 * [cheatsheet.md summary, "What is BitNet b1.58?": activations scaled per token
 *  in front of every BitLinear; asi.tokyo 2B4T article, packing paragraph]
 *
 * Same results as bitlinear_quantize_act(x, dtype, M, K, xq, scale, rowsum)
 * followed by bitlinear_forward_ex(xq, scale, rowsum, M, packed, layout,
 * gamma, N, K, y, workspace, workspace_bytes, path), after all arguments of
 * both have been checked: xq, scale and rowsum (all required) are written, and
 * y is bit-identical to the two calls.  N == 0 only quantises.  One token on
 * the vector path with the 2-bit layout (M == 1, K % 16 == 0, K <= 16384;
 * fp32 tokens longer than 8192 on matrices of few rows excepted) is one
 * launch: every block of the product quantises the token itself (same
 * arithmetic) and the first block also stores xq, scale and rowsum; other
 * shapes are two launches back to back on `stream`.  x must not overlap xq. */
int bitlinear_quantize_forward(const void *x, int dtype, int64_t M, int64_t K, int8_t *xq,
                               float *scale, int32_t *rowsum, const uint8_t *packed, int layout,
                               const float *gamma, int64_t N, float *y, void *workspace,
                               int64_t workspace_bytes, int path, hipStream_t stream);

/* ---- decoder-block glue of the layer-stack workload ------------------------------
 * [asi.tokyo 2B4T article, stabiliser paragraph: a norm in front of the
 *  sub-layers, squared ReLU in the feed-forward block; cheatsheet.md summary,
 *  "What is BitNet b1.58?": RMSNorm, no bias, activations scaled per token]
 *
 * Each call forms a [M, K] block of values v (device, float inputs), applies
 * RMSNorm with unit gain in double precision, h = v / sqrt(mean_k v^2 + eps)
 * rounded to float, and quantises h per token with the arithmetic of
 * bitlinear_quantize_act: xq [M, K] int8, scale [M] float and rowsum [M] int32
 * (device, all required, written).  1 <= K <= 8192; eps >= 0.  M == 0 is a
 * no-op.  The double-precision sum of squares is reduced in a different order
 * than a sequential loop, so h can differ from such a loop in the last bit in
 * rare cases; every later step is exact. */

/* v = x after x += add: x device [M, K] float, updated in place (the residual
 * stream); add device [M, K] float, or NULL for no addition. */
int bitlinear_residual_rmsnorm_quantize(float *x, const float *add, int64_t M, int64_t K,
                                        float eps, int8_t *xq, float *scale, int32_t *rowsum,
                                        hipStream_t stream);

/* Attention output of the first token (sequence position 0: a single key, so
 * the softmax weight is 1) under grouped-query attention:
 * v[m, h * head_dim + d] = qkv[m * ld + v_col + (h / (heads / kv_heads)) * head_dim + d],
 * K = heads * head_dim.  qkv: device, M rows of ld floats (the QKV product). */
int bitlinear_gqa_rmsnorm_quantize(const float *qkv, int64_t M, int64_t ld, int64_t v_col,
                                   int64_t heads, int64_t kv_heads, int64_t head_dim, float eps,
                                   int8_t *xq, float *scale, int32_t *rowsum, hipStream_t stream);

/* Squared-ReLU gate: v[m, i] = relu(g)^2 * u in double precision, with
 * g = gate_up[m * ld + i] and u = gate_up[m * ld + F + i]; K = F.  gate_up:
 * device, M rows of ld >= 2F floats (the fused up/gate product). */
int bitlinear_relu2_rmsnorm_quantize(const float *gate_up, int64_t M, int64_t ld, int64_t F,
                                     float eps, int8_t *xq, float *scale, int32_t *rowsum,
                                     hipStream_t stream);

/* ---- a BitLinear product followed by the next BitLinear's input glue --------------
 * [same passages as the glue above, and the BitLinear product of
 *  bitlinear_forward_ex]
 *
 * Same results, bit for bit, as bitlinear_forward_ex(xq, scale, rowsum, M,
 * packed, BL_PACK2, gamma, N, K, y, ..., BL_PATH_AUTO) into a [M, N] float
 * y, followed by the glue call named after it on y, with its outputs written
 * to xq_out [M, K'], scale_out [M] and rowsum_out [M] (K' = the glue's width).
 * The first input is the product's (xq, scale, rowsum: device, required, as
 * for bitlinear_forward_ex; the 2-bit layout only).  y itself is not
 * returned: where the tiled GEMM splits the k range, the glue kernel adds the
 * split partial products itself, which saves the separate finishing launch.
 * The outputs may be the same buffers as the inputs xq, scale and rowsum (the
 * product has read them first); nothing else may overlap.  workspace: device,
 * 16-byte aligned, at least bitlinear_forward_glue_workspace_bytes(M, N, K)
 * bytes, any contents; it holds the product's partial sums or its output.
 * N >= 1 (the glue reads columns of y).  M == 0 is a no-op.  Errors as for
 * bitlinear_forward_ex and the glue calls; nothing is launched when a check
 * fails. */
int64_t bitlinear_forward_glue_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* x [M, N] (device, float, updated in place) += y; then the residual glue on
 * x with K' = N. */
int bitlinear_forward_residual_rmsnorm_quantize(const int8_t *xq, const float *scale,
                                                const int32_t *rowsum, int64_t M, int64_t K,
                                                const uint8_t *packed, const float *gamma,
                                                int64_t N, float *x, float eps, int8_t *xq_out,
                                                float *scale_out, int32_t *rowsum_out,
                                                void *workspace, int64_t workspace_bytes,
                                                hipStream_t stream);

/* The grouped-query glue on y (qkv = y, ld = N); K' = heads * head_dim. */
int bitlinear_forward_gqa_rmsnorm_quantize(const int8_t *xq, const float *scale,
                                           const int32_t *rowsum, int64_t M, int64_t K,
                                           const uint8_t *packed, const float *gamma, int64_t N,
                                           int64_t v_col, int64_t heads, int64_t kv_heads,
                                           int64_t head_dim, float eps, int8_t *xq_out,
                                           float *scale_out, int32_t *rowsum_out,
                                           void *workspace, int64_t workspace_bytes,
                                           hipStream_t stream);

/* The squared-ReLU glue on y (gate_up = y, ld = N >= 2F); K' = F. */
int bitlinear_forward_relu2_rmsnorm_quantize(const int8_t *xq, const float *scale,
                                             const int32_t *rowsum, int64_t M, int64_t K,
                                             const uint8_t *packed, const float *gamma,
                                             int64_t N, int64_t F, float eps, int8_t *xq_out,
                                             float *scale_out, int32_t *rowsum_out,
                                             void *workspace, int64_t workspace_bytes,
                                             hipStream_t stream);

/* ---- one token: the next BitLinear's input glue and product in one launch -------
 * [asi.tokyo 2B4T article, stabiliser paragraph: a norm in front of the
 *  sub-layers, squared ReLU in the feed-forward block; cheatsheet.md summary,
 *  "What is BitNet b1.58?": RMSNorm, no bias, activations scaled per token;
 *  asi.tokyo packing paragraph: the 2-bit product]
 *
 * For one token (decode) every block of the 2-bit vector product forms the
 * token's pre-norm values v itself, applies RMSNorm with unit gain in double
 * precision (h = v / sqrt(mean v^2 + eps) rounded to float; the sum of squares
 * is reduced in another order than a sequential loop, as in the glue calls),
 * quantises h with the arithmetic of bitlinear_quantize_act into an on-chip
 * int8 copy, and multiplies: no int8 token goes through memory.
 *
 * input    BL_NORM_RESIDUAL: src is the float residual stream [K]; with add
 *          (float [K]) not NULL, v = src + add in float, stored to x_out
 *          (float [K], required then; it must not overlap src or add: the
 *          launch's blocks all read src); with add NULL, v = src.
 *          BL_NORM_GQA: v is the first token's attention output under
 *          grouped-query attention, v[h * head_dim + d] =
 *          src[v_col + (h / (heads / kv_heads)) * head_dim + d] (src: the float
 *          QKV output row), K = heads * head_dim.
 *          BL_NORM_F64: src is a double [K] (the relu2 output below).
 * packed, gamma  the 2-bit weights [N, K] and their gamma (BL_PACK2 layout).
 * relu2 = 0: out is float [N], out[n] = acc[n] * (gamma / s) as in
 *          bitlinear_forward.
 * relu2 = 1: packed is a fused up/gate matrix, gate rows [0, F) and up rows
 *          [F, 2F), N = 2F; out is double [F], out[i] = relu(y_gate)^2 * y_up
 *          in double, with y_gate = y[i] and y_up = y[F + i] rounded to float
 *          as the product stores them.
 * xq, scale, rowsum  optional outputs (may be NULL): the quantised token
 *          [K], its scale and row sum, as bitlinear_quantize_act writes them.
 * 1 <= K <= 16384, N >= 1, eps >= 0; float pointers 4-byte aligned, double
 * pointers 8-byte aligned, packed 16-byte aligned.  One launch. */
typedef enum { BL_NORM_RESIDUAL = 0, BL_NORM_GQA = 1, BL_NORM_F64 = 2 } bl_norm_input;

int bitlinear_norm_forward(int input, const void *src, const float *add, float *x_out,
                           int64_t v_col, int64_t heads, int64_t kv_heads, int64_t head_dim,
                           int64_t K, float eps, const uint8_t *packed, const float *gamma,
                           int64_t N, int relu2, void *out, int8_t *xq, float *scale,
                           int32_t *rowsum, hipStream_t stream);

/* Decode packed weights to int8 trits in {-1, 0, 1} (device, [N, K]). */
int bitlinear_unpack_weights(const uint8_t *packed, int layout, int64_t N, int64_t K,
                             int8_t *trits, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* BITLINEAR_H */
