/*
 * CPU oracle for the BitNet b1.58 BitLinear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this file: only the tests, the smoke check and the benchmark's CPU-baseline leg
 * do.  It shares no code, header, table or constant with the HIP library.
 *
 * Every function is the plain definition of one step, written as slow scalar
 * loops so that it can be checked against the sources by eye:
 *
 *   [CS]    "1-bit LLM era: Microsoft introduces BitNet b1.58" (cheatsheet.md),
 *           section "What is BitNet b1.58?": BitLinear replaces nn.Linear; the
 *           weight quantiser scales by the mean absolute value, rounds to the
 *           nearest integer and constrains to {-1,0,1}; activations are scaled
 *           per token; no bias.
 *   [ASI]   asi.tokyo article on BitNet b1.58 2B4T (2025-04-27), the paragraphs
 *           on the absmean quantiser, the 8-bit messages between layers and the
 *           custom GPU software that packs four weights into one byte.
 *   [LUMEN] lumen-it.ai article on BitNet (original 1-bit BitNet): absmax
 *           quantisation of activations.
 *   [HADA]  news.hada.io topic 20406 (vi and pt editions), comment on ternary
 *           packing: five ternary digits in one byte, log2(3) = 1.58 bits.
 *
 * Readings taken where the sources are silent (each is listed with its reason
 * in the design notes):
 *   - gamma is one scalar per weight matrix: the sum of |w| is formed exactly
 *     and rounded once to double, divided by N*K in double precision and
 *     rounded once to float (so it does not depend on any summation order).
 *   - "round to the nearest integer" is round-half-to-even on the exact
 *     quotient w/gamma; the result is clipped to [-1, 1].
 *   - activation quantisation is symmetric 8-bit: s = 127 / max|x| per token,
 *     q = clamp(rint(x * s), -127, 127), computed in float (the precision of
 *     the GPU kernel, since this decides an integer); an all-zero token gets
 *     s = 1 and q = 0.  When 127 / max|x| overflows the float range (a token
 *     whose largest magnitude is below about 3.7e-37), s is the largest
 *     finite float instead of infinity, so q stays defined (zeros map to 0)
 *     and acc * gamma / s stays finite.
 *   - a NaN quotient w / gamma (gamma NaN, or w and gamma both infinite)
 *     gives the trit 0: the comparison 2|w| > gamma it stands for is false.
 *   - accumulation is exact integer arithmetic; the output is acc * gamma / s,
 *     evaluated here in double precision.
 *   - packed layouts are the ones the library header documents (2-bit codes
 *     t+1 in 32-bit words of 16 trits; base-3 bytes of 5 trits).
 *   - variants: sign binarisation maps w < 0 to -1 and everything else (zero
 *     included) to +1, with the absmean scale of the whole matrix, or one
 *     absmean scale per group of consecutive weight rows (group quantisation:
 *     G equal shards of the output features, each scaled on its own); b-bit
 *     activations use Q = 2^(b-1) - 1 in place of 127.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ---- input element types --------------------------------------------- */

enum { ORC_F32 = 0, ORC_BF16 = 1 };

/* bfloat16 is the upper half of a binary32: widening is a 16-bit shift. */
float orc_bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static float load_elem(const void *p, int dtype, int64_t i)
{
    if (dtype == ORC_BF16)
        return orc_bf16_to_f32(((const uint16_t *)p)[i]);
    return ((const float *)p)[i];
}

/* ---- weights: absmean quantiser [CS "What is BitNet b1.58?", first bullet;
 *      ASI, absmean-quantiser paragraph] --------------------------------- */

/* Sum of |w| over `count` elements without any rounding, then rounded once to
 * the nearest double (ties to even).  A finite binary32 magnitude is an integer
 * significand m < 2^24 times 2^(e - 150), with e = max(biased exponent, 1) and
 * the implicit leading bit included for e >= 1.  The significands are added
 * per exponent in 64-bit integers (fewer than 2^40 terms of less than 2^24
 * each, so no overflow), the per-exponent totals are added, shifted, into one
 * multi-word binary integer B, and B * 2^-150 is rounded to a double.
 * *nonfinite is set to 2 if an element is NaN, else 1 if one is infinite,
 * else 0. */
double orc_abs_sum(const void *w, int dtype, int64_t count, int *nonfinite)
{
    uint64_t per_exp[256];
    memset(per_exp, 0, sizeof per_exp);
    int nan_seen = 0, inf_seen = 0;
    for (int64_t i = 0; i < count; ++i) {
        float f = load_elem(w, dtype, i);
        uint32_t u;
        memcpy(&u, &f, sizeof u);
        uint32_t e = (u >> 23) & 0xffu, frac = u & 0x7fffffu;
        if (e == 255u) {
            if (frac) nan_seen = 1;
            else inf_seen = 1;
            continue;
        }
        uint32_t m = e ? (frac | 0x800000u) : frac;
        per_exp[e ? e : 1] += m;
    }
    *nonfinite = nan_seen ? 2 : (inf_seen ? 1 : 0);

    /* B = sum_e per_exp[e] * 2^e as 16 little-endian 32-bit digits. */
    uint32_t digit[16];
    memset(digit, 0, sizeof digit);
    for (int e = 1; e < 255; ++e) {
        uint64_t v = per_exp[e];
        int pos = e / 32, sh = e % 32;
        /* v << sh spans at most three digits; add them with carry */
        uint32_t part[3];
        part[0] = (uint32_t)(v << sh);
        part[1] = (uint32_t)(sh ? (v >> (32 - sh)) : (v >> 32));
        part[2] = (uint32_t)(sh ? (v >> (64 - sh)) : 0);
        uint64_t carry = 0;
        for (int d = pos; d < 16; ++d) {
            uint64_t add = (d - pos < 3) ? part[d - pos] : 0;
            uint64_t t = (uint64_t)digit[d] + add + carry;
            digit[d] = (uint32_t)t;
            carry = t >> 32;
            if (d - pos >= 2 && carry == 0) break;
        }
    }

    /* highest set bit of B */
    int top = -1;
    for (int d = 15; d >= 0 && top < 0; --d)
        for (int b = 31; b >= 0; --b)
            if ((digit[d] >> b) & 1u) {
                top = 32 * d + b;
                break;
            }
    if (top < 0) return 0.0;
#define ORC_BIT(pos) ((digit[(pos) / 32] >> ((pos) % 32)) & 1u)
    /* keep the 53 bits top-52 .. top, round on the rest */
    int low = top - 52;
    uint64_t mant = 0;
    for (int b = top; b >= (low > 0 ? low : 0); --b) mant = (mant << 1) | ORC_BIT(b);
    if (low <= 0) return ldexp((double)mant, -150);      /* B < 2^53: exact */
    int half = ORC_BIT(low - 1);
    int sticky = 0;
    for (int b = 0; b < low - 1; ++b) sticky |= ORC_BIT(b);
#undef ORC_BIT
    if (half && (sticky || (mant & 1u))) mant += 1;      /* may reach 2^53: still exact */
    return ldexp((double)mant, low - 150);
}

/* gamma = mean |W| over the whole N x K matrix: the exact sum of |w| rounded
 * once to double, divided by N*K in double precision, rounded to float.  A NaN
 * element makes gamma NaN; otherwise an infinite one makes it +inf. */
float orc_absmean_gamma(const void *w, int dtype, int64_t n_rows, int64_t k_cols)
{
    int nonfinite = 0;
    double total = orc_abs_sum(w, dtype, n_rows * k_cols, &nonfinite);
    if (nonfinite == 2) return NAN;
    if (nonfinite == 1) return INFINITY;
    return (float)(total / ((double)n_rows * (double)k_cols));
}

/* t = clip(round(w / gamma), -1, 1), round half to even. */
void orc_absmean_trits(const void *w, int dtype, int64_t n_rows, int64_t k_cols,
                       float gamma, int8_t *t)
{
    for (int64_t i = 0; i < n_rows * k_cols; ++i) {
        double v = (double)load_elem(w, dtype, i);
        if (v == 0.0) {           /* zero scales to zero, whatever gamma is */
            t[i] = 0;
            continue;
        }
        double r = rint(v / (double)gamma);  /* gamma == 0 gives +-inf */
        if (r != r) r = 0.0;                 /* NaN quotient: 2|w| > gamma is false */
        if (r > 1.0) r = 1.0;
        if (r < -1.0) r = -1.0;
        t[i] = (int8_t)r;
    }
}

/* ---- weights, 1-bit variant [LUMEN: binary weights +1 / -1 by the signum
 *      function]: t = -1 for w < 0, +1 otherwise (zero maps to +1; its scale
 *      is orc_absmean_gamma, one group per matrix). -------------------------- */
void orc_sign_trits(const void *w, int dtype, int64_t n_rows, int64_t k_cols, int8_t *t)
{
    for (int64_t i = 0; i < n_rows * k_cols; ++i)
        t[i] = load_elem(w, dtype, i) < 0.0f ? -1 : 1;
}

/* Group quantisation [LUMEN: group quantisation and normalisation let the
 * layer be split over devices with little communication]: the N rows are cut
 * into `groups` equal, consecutive groups (groups divides N), and group g gets
 * its own scale beta[g] = mean |w| over its rows, formed exactly as gamma. */
void orc_group_absmean(const void *w, int dtype, int64_t n_rows, int64_t k_cols, int64_t groups,
                       float *beta)
{
    const int64_t rows = n_rows / groups;
    const size_t esize = dtype == ORC_BF16 ? 2 : 4;
    for (int64_t g = 0; g < groups; ++g)
        beta[g] = orc_absmean_gamma((const char *)w + (size_t)(g * rows * k_cols) * esize, dtype,
                                    rows, k_cols);
}

/* ---- 2-bit packing, four trits per byte [ASI, custom-software paragraph] --
 * Row n occupies pitch2(K) bytes, a whole number of 16-byte groups of 64 trits.
 * Inside a row, 32-bit little-endian word g holds trits k = 16g .. 16g+15: the
 * trit k = 16g + 4i + j sits in byte j of the word, bits 2i..2i+1, as the code
 * t + 1 in {0,1,2}.  Positions past K hold code 1 (trit 0). */

int64_t orc_pack2_pitch(int64_t k_cols)
{
    return ((k_cols + 63) / 64) * 16;
}

void orc_pack2(const int8_t *t, int64_t n_rows, int64_t k_cols, uint8_t *packed)
{
    int64_t pitch = orc_pack2_pitch(k_cols);
    for (int64_t n = 0; n < n_rows; ++n) {
        for (int64_t b = 0; b < pitch; ++b) {
            /* byte b of the row is byte j of word g */
            int64_t g = b / 4, j = b % 4;
            unsigned byte = 0;
            for (int i = 0; i < 4; ++i) {
                int64_t k = 16 * g + 4 * i + j;
                int code = 1;
                if (k < k_cols)
                    code = t[n * k_cols + k] + 1;
                byte |= (unsigned)code << (2 * i);
            }
            packed[n * pitch + b] = (uint8_t)byte;
        }
    }
}

void orc_unpack2(const uint8_t *packed, int64_t n_rows, int64_t k_cols, int8_t *t)
{
    int64_t pitch = orc_pack2_pitch(k_cols);
    for (int64_t n = 0; n < n_rows; ++n) {
        for (int64_t k = 0; k < k_cols; ++k) {
            int64_t g = k / 16, i = (k % 16) / 4, j = k % 4;
            unsigned byte = packed[n * pitch + 4 * g + j];
            int code = (int)((byte >> (2 * i)) & 3u);
            t[n * k_cols + k] = (int8_t)(code - 1);
        }
    }
}

/* ---- base-3 packing, five trits per byte [HADA, ternary-packing comment] --
 * Byte j of row n is sum_{i=0..4} (t[n][5j+i] + 1) * 3^i, so the lowest k is
 * the least significant digit.  Trits past K are 0 (digit 1); the row pitch is
 * ceil(K/5) rounded up to 16 bytes and the filler bytes are 121 (= 11111 in
 * base 3, five zero trits). */

int64_t orc_pack3_pitch(int64_t k_cols)
{
    int64_t nbytes = (k_cols + 4) / 5;
    return ((nbytes + 15) / 16) * 16;
}

void orc_pack3(const int8_t *t, int64_t n_rows, int64_t k_cols, uint8_t *packed)
{
    int64_t pitch = orc_pack3_pitch(k_cols);
    for (int64_t n = 0; n < n_rows; ++n) {
        for (int64_t b = 0; b < pitch; ++b) {
            unsigned value = 0, weight = 1;
            for (int i = 0; i < 5; ++i) {
                int64_t k = 5 * b + i;
                int digit = 1;
                if (k < k_cols)
                    digit = t[n * k_cols + k] + 1;
                value += (unsigned)digit * weight;
                weight *= 3;
            }
            packed[n * pitch + b] = (uint8_t)value;
        }
    }
}

void orc_unpack3(const uint8_t *packed, int64_t n_rows, int64_t k_cols, int8_t *t)
{
    int64_t pitch = orc_pack3_pitch(k_cols);
    for (int64_t n = 0; n < n_rows; ++n) {
        for (int64_t k = 0; k < k_cols; ++k) {
            unsigned value = packed[n * pitch + k / 5];
            for (int64_t i = 0; i < k % 5; ++i)
                value /= 3;
            t[n * k_cols + k] = (int8_t)((int)(value % 3) - 1);
        }
    }
}

/* ---- activations: per-token absmax to 8 bits [CS "What is BitNet b1.58?",
 *      activation bullet; ASI, 8-bit messages; LUMEN, absmax] ------------- */

/* b-bit activations [CS, outlook: activations compressed to 4 bits or fewer]:
 * the same quantiser with Q = 2^(b-1) - 1 in place of 127. */
void orc_quantize_act_bits(const void *x, int dtype, int64_t m_rows, int64_t k_cols, int bits,
                           int8_t *q, float *scale, int32_t *rowsum)
{
    const float qmax = (float)((1 << (bits - 1)) - 1);
    for (int64_t m = 0; m < m_rows; ++m) {
        float amax = 0.0f;
        for (int64_t k = 0; k < k_cols; ++k) {
            float a = fabsf(load_elem(x, dtype, m * k_cols + k));
            if (a > amax)
                amax = a;
        }
        int32_t sum = 0;
        if (amax == 0.0f) {
            scale[m] = 1.0f;
            for (int64_t k = 0; k < k_cols; ++k)
                q[m * k_cols + k] = 0;
        } else {
            float s = qmax / amax;
            if (s > FLT_MAX) s = FLT_MAX;    /* qmax / amax overflowed */
            scale[m] = s;
            for (int64_t k = 0; k < k_cols; ++k) {
                float r = rintf(load_elem(x, dtype, m * k_cols + k) * s);
                if (r > qmax) r = qmax;
                if (r < -qmax) r = -qmax;
                q[m * k_cols + k] = (int8_t)r;
                sum += (int32_t)r;
            }
        }
        if (rowsum)
            rowsum[m] = sum;
    }
}

void orc_quantize_act(const void *x, int dtype, int64_t m_rows, int64_t k_cols,
                      int8_t *q, float *scale, int32_t *rowsum)
{
    for (int64_t m = 0; m < m_rows; ++m) {
        float amax = 0.0f;
        for (int64_t k = 0; k < k_cols; ++k) {
            float a = fabsf(load_elem(x, dtype, m * k_cols + k));
            if (a > amax)
                amax = a;
        }
        int32_t sum = 0;
        if (amax == 0.0f) {
            scale[m] = 1.0f;
            for (int64_t k = 0; k < k_cols; ++k)
                q[m * k_cols + k] = 0;
        } else {
            float s = 127.0f / amax;
            if (s > FLT_MAX) s = FLT_MAX;    /* 127 / amax overflowed */
            scale[m] = s;
            for (int64_t k = 0; k < k_cols; ++k) {
                float v = load_elem(x, dtype, m * k_cols + k) * s;
                float r = rintf(v);
                if (r > 127.0f) r = 127.0f;
                if (r < -127.0f) r = -127.0f;
                q[m * k_cols + k] = (int8_t)r;
                sum += (int32_t)r;
            }
        }
        if (rowsum)
            rowsum[m] = sum;
    }
}

/* ---- backward through BitLinear with straight-through estimators [LUMEN:
 *      training uses straight-through estimators for the gradient flow] ------
 * Both quantisers pass the gradient unchanged, so the layer acts on x as the
 * matrix gamma * t: grad_x[m][k] = gamma * sum_n grad_y[m][n] * t[n][k],
 * evaluated in double precision from the exact inputs. */
void orc_backward_input(const void *grad_y, int dtype, int64_t m_rows, int64_t n_rows,
                        const int8_t *t, int64_t k_cols, float gamma, double *grad_x)
{
    for (int64_t m = 0; m < m_rows; ++m)
        for (int64_t k = 0; k < k_cols; ++k) {
            double acc = 0.0;
            for (int64_t n = 0; n < n_rows; ++n)
                acc += (double)load_elem(grad_y, dtype, m * n_rows + n) * (double)t[n * k_cols + k];
            grad_x[m * k_cols + k] = (double)gamma * acc;
        }
}

/* ---- integer contraction and rescale [ASI, custom-software paragraph: the
 *      trits are multiplied with the 8-bit activations] ------------------- */

/* acc[m][n] = sum_k t[n][k] * q[m][k], exact. */
void orc_matmul_i32(const int8_t *q, int64_t m_rows, const int8_t *t, int64_t n_rows,
                    int64_t k_cols, int32_t *acc)
{
    for (int64_t m = 0; m < m_rows; ++m) {
        for (int64_t n = 0; n < n_rows; ++n) {
            int64_t sum = 0;
            for (int64_t k = 0; k < k_cols; ++k)
                sum += (int64_t)t[n * k_cols + k] * (int64_t)q[m * k_cols + k];
            acc[m * n_rows + n] = (int32_t)sum;
        }
    }
}

/* y[m][n] = acc[m][n] * gamma / s[m]: undoes both quantiser scalings. */
void orc_rescale(const int32_t *acc, const float *scale, float gamma, int64_t m_rows,
                 int64_t n_rows, double *y)
{
    for (int64_t m = 0; m < m_rows; ++m)
        for (int64_t n = 0; n < n_rows; ++n)
            y[m * n_rows + n] =
                (double)acc[m * n_rows + n] * (double)gamma / (double)scale[m];
}

/* The same with one weight scale per group of N / groups consecutive output
 * features: y[m][n] = acc[m][n] * beta[n / (N / groups)] / s[m]. */
void orc_rescale_groups(const int32_t *acc, const float *scale, const float *beta,
                        int64_t groups, int64_t m_rows, int64_t n_rows, double *y)
{
    const int64_t rows = n_rows / groups;
    for (int64_t m = 0; m < m_rows; ++m)
        for (int64_t n = 0; n < n_rows; ++n)
            y[m * n_rows + n] =
                (double)acc[m * n_rows + n] * (double)beta[n / rows] / (double)scale[m];
}

/* ---- 2B-class decoder block glue, used only by the layer-stack workload ----
 * [ASI, stabiliser paragraph: a sub-layer norm and squared ReLU; CS "What is
 * BitNet b1.58?", third bullet: RMSNorm, no bias].  Double precision. */

/* out = x / sqrt(mean(x^2) + eps), unit gain, one row of length K at a time. */
void orc_rmsnorm(const double *x, int64_t m_rows, int64_t k_cols, double eps, double *out)
{
    for (int64_t m = 0; m < m_rows; ++m) {
        double ss = 0.0;
        for (int64_t k = 0; k < k_cols; ++k)
            ss += x[m * k_cols + k] * x[m * k_cols + k];
        double inv = 1.0 / sqrt(ss / (double)k_cols + eps);
        for (int64_t k = 0; k < k_cols; ++k)
            out[m * k_cols + k] = x[m * k_cols + k] * inv;
    }
}

/* out = relu(gate)^2 * up, elementwise. */
void orc_relu2_mul(const double *gate, const double *up, int64_t count, double *out)
{
    for (int64_t i = 0; i < count; ++i) {
        double g = gate[i] > 0.0 ? gate[i] : 0.0;
        out[i] = g * g * up[i];
    }
}

/* x[i] = x[i] + y[i] in single precision: the residual stream of the block. */
void orc_add_f32(float *x, const float *y, int64_t count)
{
    for (int64_t i = 0; i < count; ++i)
        x[i] = x[i] + y[i];
}

/* Attention of the first token (sequence position 0): there is one key, so
 * the softmax weight is 1 and each query head returns the value vector of its
 * key-value head; with grouped-query attention head h reads key-value head
 * h / (heads / kv_heads).  v holds kv_heads * head_dim values per row, rows
 * v_stride floats apart; out is [m_rows, heads * head_dim] in double. */
void orc_gqa_expand(const float *v, int64_t m_rows, int64_t v_stride, int64_t heads,
                    int64_t kv_heads, int64_t head_dim, double *out)
{
    const int64_t group = heads / kv_heads;
    for (int64_t m = 0; m < m_rows; ++m)
        for (int64_t h = 0; h < heads; ++h)
            for (int64_t d = 0; d < head_dim; ++d)
                out[(m * heads + h) * head_dim + d] =
                    (double)v[m * v_stride + (h / group) * head_dim + d];
}
