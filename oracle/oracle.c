/*
 * oracle.c -- plain, single-threaded CPU oracle of the W4A8 decode GEMV path.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the bench's
 * CPU-baseline leg may load this library.  The GPU path shares no code,
 * header, table or helper with it; neither includes or links the other.
 *
 * Every step follows the pages' definitions literally, in their order:
 *   [Orin] "Jetson Orin AGX INT4 推理优化实践：super 分支从 9 tok/s 到 24 tok/s"
 *          sections "从 FP 线性层到 INT4 DP4A 的数学推导" (FP linear -> INT4
 *          DP4A derivation), "INT32 accumulator 是否安全" (int32 safety),
 *          "DP4A 做了什么" (what DP4A does; the packed-word layout).
 *   [Ascend] "在香橙派上跑 Gemma4：vLLM 适配昇腾 310B 的内核开发实录"
 *          sections 3.1 (Q4_0 fused dequant matmul: int4 + one fp16 scale per
 *          32 weights), 3.2 (lm_head expanded to int8 with fp16 group scales),
 *          5 (M=K verification of K draft tokens).
 *
 * Precision.  Where a floating-point value decides an integer (a weight or
 * activation code), the decision is taken in fp32, the precision of the
 * GPU path: correctly rounded fp32 divisions and round-half-to-even.  Every
 * other floating-point result (the outputs y) is computed in binary64.
 * Integer sums are exact in int64 and checked against the int32 bound.
 * Built with -ffp-contract=off and without fast-math; x86-64 SSE arithmetic
 * has no excess precision.
 *
 * Return codes: 0 ok, ORC_E_ARG (-1) bad size/argument, ORC_E_RANGE (-2)
 * input outside the format's range, ORC_E_NONFINITE (-3) NaN/Inf input,
 * ORC_E_BOUND (-4) accumulator outside the int32 bound.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ORC_OK 0
#define ORC_E_ARG (-1)
#define ORC_E_RANGE (-2)
#define ORC_E_NONFINITE (-3)
#define ORC_E_BOUND (-4)

/* ------------------------------------------------------------------------ */
/* IEEE 754 binary16 <-> binary32 (the fp16 scales of [Ascend] 3.1 and 3.2,  */
/* and the fp16 activations of the W8A16 lm_head).                          */
/* ------------------------------------------------------------------------ */

/* binary16 -> binary32, exact.  value = (-1)^s * 2^(e-15) * 1.m for normal
 * numbers and (-1)^s * 2^-14 * 0.m for subnormals. */
float orc_f16_to_f32(uint16_t h)
{
    unsigned sign = (h >> 15) & 1u;
    unsigned e = (h >> 10) & 0x1Fu;
    unsigned m = h & 0x3FFu;
    float v;
    if (e == 0)
        v = ldexpf((float)m, -24);                 /* m * 2^-24, exact */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexpf((float)(1024u + m), (int)e - 25); /* (1024+m) * 2^(e-25) */
    return sign ? -v : v;
}

/* binary32 -> binary16, round to nearest, ties to even. */
uint16_t orc_f32_to_f16(float f)
{
    uint32_t bits;
    memcpy(&bits, &f, 4);
    uint16_t sign = (uint16_t)((bits >> 16) & 0x8000u);
    float a = fabsf(f);
    if (isnan(f))
        return sign | 0x7E00u;
    /* 65520 lies half-way between 65504 (largest finite, odd significand)
     * and 2^16 (even): ties-to-even rounds it, and everything above, to Inf. */
    if (a >= 65520.0f)
        return sign | 0x7C00u;
    if (a < 0x1p-14f) {
        /* subnormal range: the quantum is 2^-24; a*2^24 is exact.  A result
         * of 1024 is the bit pattern of the smallest normal, as it should be. */
        float n = nearbyintf(a * 0x1p24f);
        return sign | (uint16_t)n;
    }
    int e;
    float m = frexpf(a, &e);                 /* a = m * 2^e, 0.5 <= m < 1   */
    float q = nearbyintf(ldexpf(m, 11));     /* 11-bit significand, RNE     */
    if (q == 2048.0f) {                      /* rounded up to the next binade */
        q = 1024.0f;
        e += 1;
    }
    int E = e + 14;                          /* biased exponent: (e-1) + 15 */
    if (E >= 31)
        return sign | 0x7C00u;
    return (uint16_t)(sign | (uint16_t)(E << 10) | (uint16_t)((int)q - 1024));
}

void orc_f32_to_f16_array(const float* x, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_f32_to_f16(x[i]);
}

void orc_f16_to_f32_array(const uint16_t* x, int64_t n, float* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_f16_to_f32(x[i]);
}

/* ------------------------------------------------------------------------ */
/* Symmetric quantisation of one value: clip(round(v / s), lo, hi) with an   */
/* fp32 division and round-half-to-even ([Orin] derivation section).         */
/* ------------------------------------------------------------------------ */
static int8_t quant_code(float v, float s, int lo, int hi)
{
    if (s == 0.0f)
        return 0; /* all-zero row/group/vector: every code is 0 */
    float r = nearbyintf(v / s);
    if (r < (float)lo)
        r = (float)lo;
    if (r > (float)hi)
        r = (float)hi;
    return (int8_t)r;
}

static int max_abs_f32(const float* v, int64_t n, float* amax)
{
    float a = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float t = fabsf(v[i]);
        if (!(t <= FLT_MAX))
            return ORC_E_NONFINITE;
        if (t > a)
            a = t;
    }
    *amax = a;
    return ORC_OK;
}

/* Per-row INT4 weights: s^W_j = max_i |W_ji| / 7 (fp32),
 * q^W_ji = clip(round(W_ji / s^W_j), -8, 7).  [Orin] derivation section. */
int orc_quantize_weights_int4_rowwise(const float* W, int64_t N, int64_t K,
                                      int8_t* q, float* s)
{
    if (N < 0 || K <= 0)
        return ORC_E_ARG;
    for (int64_t j = 0; j < N; ++j) {
        const float* row = W + j * K;
        float amax;
        int rc = max_abs_f32(row, K, &amax);
        if (rc)
            return rc;
        float sj = amax / 7.0f;
        s[j] = sj;
        for (int64_t i = 0; i < K; ++i)
            q[j * K + i] = quant_code(row[i], sj, -8, 7);
    }
    return ORC_OK;
}

/* Group-of-32 quantisation with one fp16 scale per group: the stored scale
 * is fp16(max|W_g| / d) and codes are taken against that stored value. */
static int quantize_group32(const float* W, int64_t N, int64_t K, float d, int lo,
                            int hi, int8_t* q, uint16_t* s16)
{
    if (N < 0 || K <= 0 || K % 32)
        return ORC_E_ARG;
    int64_t G = K / 32;
    for (int64_t j = 0; j < N; ++j) {
        for (int64_t g = 0; g < G; ++g) {
            const float* v = W + j * K + g * 32;
            float amax;
            int rc = max_abs_f32(v, 32, &amax);
            if (rc)
                return rc;
            uint16_t h = orc_f32_to_f16(amax / d);
            s16[j * G + g] = h;
            float sg = orc_f16_to_f32(h);
            for (int i = 0; i < 32; ++i)
                q[j * K + g * 32 + i] = quant_code(v[i], sg, lo, hi);
        }
    }
    return ORC_OK;
}

/* Q4_0-style: int4 codes in [-8, 7], one fp16 scale per 32 weights.
 * [Ascend] 3.1 gives the block (16 bytes of 4-bit data + one fp16 scale). */
int orc_quantize_weights_int4_group32(const float* W, int64_t N, int64_t K,
                                      int8_t* q, uint16_t* s16)
{
    return quantize_group32(W, N, K, 7.0f, -8, 7, q, s16);
}

/* lm_head expanded to int8: codes in [-32, 31] (the 6-bit value range) with
 * one fp16 scale per 32 weights.  [Ascend] 3.2. */
int orc_quantize_weights_int8_group32(const float* W, int64_t N, int64_t K,
                                      int8_t* q, uint16_t* s16)
{
    return quantize_group32(W, N, K, 31.0f, -32, 31, q, s16);
}

/* ------------------------------------------------------------------------ */
/* Packing: eight signed INT4 codes per uint32, w0 in the low nibble,        */
/* word = [w7 w6 w5 w4 w3 w2 w1 w0].  [Orin] section "DP4A 做了什么".          */
/* A nibble holds the code's two's-complement low four bits.                 */
/* ------------------------------------------------------------------------ */
uint32_t orc_pack_word(const int8_t q[8])
{
    uint32_t w = 0;
    for (int k = 0; k < 8; ++k)
        w |= ((uint32_t)(uint8_t)q[k] & 0xFu) << (4 * k);
    return w;
}

void orc_unpack_word(uint32_t w, int8_t q[8])
{
    for (int k = 0; k < 8; ++k) {
        int n = (int)((w >> (4 * k)) & 0xFu);
        q[k] = (int8_t)(n >= 8 ? n - 16 : n);
    }
}

int orc_pack_int4(const int8_t* q, int64_t N, int64_t K, uint32_t* w)
{
    if (N < 0 || K <= 0 || K % 8)
        return ORC_E_ARG;
    for (int64_t i = 0; i < N * K; ++i)
        if (q[i] < -8 || q[i] > 7)
            return ORC_E_RANGE;
    for (int64_t t = 0; t < N * K / 8; ++t)
        w[t] = orc_pack_word(q + 8 * t);
    return ORC_OK;
}

int orc_unpack_int4(const uint32_t* w, int64_t N, int64_t K, int8_t* q)
{
    if (N < 0 || K <= 0 || K % 8)
        return ORC_E_ARG;
    for (int64_t t = 0; t < N * K / 8; ++t)
        orc_unpack_word(w[t], q + 8 * t);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Dynamic per-token activation quantisation ([Orin] derivation section):    */
/*   s^x = max_i |x_i| / 127,  q^x_i = clip(round(x_i / s^x), -127, 127).    */
/* ------------------------------------------------------------------------ */
int orc_quantize_act_f32(const float* x, int64_t M, int64_t K, int8_t* q, float* s)
{
    if (M < 0 || K <= 0)
        return ORC_E_ARG;
    for (int64_t m = 0; m < M; ++m) {
        const float* v = x + m * K;
        float amax;
        int rc = max_abs_f32(v, K, &amax);
        if (rc)
            return rc;
        float sx = amax / 127.0f;
        s[m] = sx;
        for (int64_t i = 0; i < K; ++i)
            q[m * K + i] = quant_code(v[i], sx, -127, 127);
    }
    return ORC_OK;
}

/* fp16 activations are widened exactly to fp32 first. */
int orc_quantize_act_f16(const uint16_t* x, int64_t M, int64_t K, int8_t* q, float* s)
{
    if (M < 0 || K <= 0)
        return ORC_E_ARG;
    for (int64_t m = 0; m < M; ++m) {
        float amax = 0.0f;
        for (int64_t i = 0; i < K; ++i) {
            float t = fabsf(orc_f16_to_f32(x[m * K + i]));
            if (!(t <= FLT_MAX))
                return ORC_E_NONFINITE;
            if (t > amax)
                amax = t;
        }
        float sx = amax / 127.0f;
        s[m] = sx;
        for (int64_t i = 0; i < K; ++i)
            q[m * K + i] = quant_code(orc_f16_to_f32(x[m * K + i]), sx, -127, 127);
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* W4A8 GEMV ([Orin] derivation section):                                    */
/*   acc_j = sum_i q^W_ji q^x_i           (exact integer dot product)        */
/*   y_j   = s^W_j s^x acc_j + b_j        (binary64 here)                    */
/* The int32 check follows [Orin] "INT32 accumulator 是否安全": per term      */
/* |q^W q^x| <= 8 * 127 = 1016, so |acc| <= 1016 K must fit in int32.        */
/* ------------------------------------------------------------------------ */
static int64_t dot_row_int4(const uint32_t* wrow, const int8_t* qx, int64_t K)
{
    int64_t acc = 0;
    int8_t qw[8];
    for (int64_t t = 0; t < K / 8; ++t) {
        orc_unpack_word(wrow[t], qw);
        for (int k = 0; k < 8; ++k)
            acc += (int64_t)qw[k] * (int64_t)qx[8 * t + k];
    }
    return acc;
}

static int check_acc(int64_t acc, int64_t K)
{
    if (acc > 1016 * K || acc < -1016 * K || acc > INT32_MAX || acc < INT32_MIN)
        return ORC_E_BOUND;
    return ORC_OK;
}

int orc_gemv_w4a8(const uint32_t* w, const float* sw, const float* bias,
                  const int8_t* qx, float sx, int64_t N, int64_t K,
                  int32_t* acc_out, double* y)
{
    if (N < 0 || K <= 0 || K % 8)
        return ORC_E_ARG;
    if (1016 * K > (int64_t)INT32_MAX)
        return ORC_E_BOUND;
    for (int64_t i = 0; i < K; ++i)
        if (qx[i] < -127)
            return ORC_E_RANGE;
    for (int64_t j = 0; j < N; ++j) {
        int64_t acc = dot_row_int4(w + j * (K / 8), qx, K);
        int rc = check_acc(acc, K);
        if (rc)
            return rc;
        if (acc_out)
            acc_out[j] = (int32_t)acc;
        double v = (double)sw[j] * (double)sx * (double)acc;
        y[j] = bias ? v + (double)bias[j] : v;
    }
    return ORC_OK;
}

/* The binary32 value of y_j that the GPU path writes and that a decoder
 * chain hands on as the next linear's activation ([Orin] derivation section:
 * each linear's input comes from the previous output).  The next codes are
 * decided from it, so it is taken in the GPU path's precision: with
 * s = fl32(s^W_j * s^x) and a = fl32(acc_j) (exact while |acc| < 2^24),
 *   y_j = fl32(s * a + b_j)      (one rounding: C99 fmaf)
 * and b_j = +0 when there is no bias. */
int orc_epilogue_f32(const float* sw, const float* bias, float sx, const int32_t* acc, int64_t N, float* y)
{
    if (N < 0)
        return ORC_E_ARG;
    for (int64_t j = 0; j < N; ++j) {
        const float s = sw[j] * sx;
        y[j] = fmaf(s, (float)acc[j], bias ? bias[j] : 0.0f);
    }
    return ORC_OK;
}

/* Group-32 W4A8: acc_jg over each block of 32 weights, then
 *   y_j = s^x * sum_g s_jg * acc_jg + b_j   (binary64, ascending g). */
int orc_gemv_w4a8_group32(const uint32_t* w, const uint16_t* s16, const float* bias,
                          const int8_t* qx, float sx, int64_t N, int64_t K,
                          int32_t* accg_out, double* y)
{
    if (N < 0 || K <= 0 || K % 32)
        return ORC_E_ARG;
    if (1016 * K > (int64_t)INT32_MAX)
        return ORC_E_BOUND;
    for (int64_t i = 0; i < K; ++i)
        if (qx[i] < -127)
            return ORC_E_RANGE;
    int64_t G = K / 32;
    for (int64_t j = 0; j < N; ++j) {
        double sum = 0.0;
        for (int64_t g = 0; g < G; ++g) {
            int64_t acc = dot_row_int4(w + j * (K / 8) + g * 4, qx + g * 32, 32);
            if (accg_out)
                accg_out[j * G + g] = (int32_t)acc;
            sum += (double)orc_f16_to_f32(s16[j * G + g]) * (double)acc;
        }
        double v = (double)sx * sum;
        y[j] = bias ? v + (double)bias[j] : v;
    }
    return ORC_OK;
}

/* W8A16 lm_head: int8 codes with fp16 group-32 scales against fp16 x,
 *   y_j = sum_g s_jg * sum_{i in g} q_ji x_i   (binary64; each group's inner
 * sum is exact in binary64: fp16 values are multiples of 2^-24 below 2^16). */
int orc_gemv_w8a16_group32(const int8_t* w, const uint16_t* s16, const uint16_t* x16,
                           int64_t N, int64_t K, double* y)
{
    if (N < 0 || K <= 0 || K % 32)
        return ORC_E_ARG;
    int64_t G = K / 32;
    for (int64_t i = 0; i < K; ++i) {
        float t = orc_f16_to_f32(x16[i]);
        if (!(fabsf(t) <= FLT_MAX))
            return ORC_E_NONFINITE;
    }
    for (int64_t j = 0; j < N; ++j) {
        double sum = 0.0;
        for (int64_t g = 0; g < G; ++g) {
            double p = 0.0;
            for (int i = 0; i < 32; ++i)
                p += (double)w[j * K + g * 32 + i] * (double)orc_f16_to_f32(x16[g * 32 + i]);
            sum += (double)orc_f16_to_f32(s16[j * G + g]) * p;
        }
        y[j] = sum;
    }
    return ORC_OK;
}

/* W4A16 comparison GEMV (the float-unpack route [Orin] "为什么 INT4 float
 * 解包不快" weighs against the integer dot, and the fp16-MAC dequantisation of
 * [Ascend] 3.1): the same packed per-row INT4 weights against an fp16
 * activation, no activation quantisation.
 *   y_j = s^W_j * sum_i q^W_ji x_i + b_j,
 * every product q x exact in binary64 (|q| <= 8, x an fp16), the sum in
 * binary64 in i order. */
int orc_gemv_w4a16(const uint32_t* w, const float* sw, const float* bias, const uint16_t* x16,
                   int64_t N, int64_t K, double* y)
{
    if (N < 0 || K <= 0 || K % 8)
        return ORC_E_ARG;
    for (int64_t i = 0; i < K; ++i) {
        float t = orc_f16_to_f32(x16[i]);
        if (!(fabsf(t) <= FLT_MAX))
            return ORC_E_NONFINITE;
    }
    for (int64_t j = 0; j < N; ++j) {
        double sum = 0.0;
        int8_t q[8];
        for (int64_t t = 0; t < K / 8; ++t) {
            orc_unpack_word(w[j * (K / 8) + t], q);
            for (int k = 0; k < 8; ++k)
                sum += (double)q[k] * (double)orc_f16_to_f32(x16[8 * t + k]);
        }
        y[j] = (double)sw[j] * sum + (bias ? (double)bias[j] : 0.0);
    }
    return ORC_OK;
}

/* M=K verification ([Ascend] 5): the same weights against M quantised
 * tokens; token m uses its own scale s^x_m.
 *   acc[m][j] = sum_i q^W_ji q^x_mi,  y[m][j] = s^W_j s^x_m acc[m][j] + b_j. */
int orc_gemm_w4a8_verify(const uint32_t* w, const float* sw, const float* bias,
                         const int8_t* qx, const float* sx, int64_t M, int64_t N,
                         int64_t K, int32_t* acc_out, double* y)
{
    if (M < 0 || N < 0 || K <= 0 || K % 8)
        return ORC_E_ARG;
    if (1016 * K > (int64_t)INT32_MAX)
        return ORC_E_BOUND;
    for (int64_t i = 0; i < M * K; ++i)
        if (qx[i] < -127)
            return ORC_E_RANGE;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t j = 0; j < N; ++j) {
            int64_t acc = dot_row_int4(w + j * (K / 8), qx + m * K, K);
            int rc = check_acc(acc, K);
            if (rc)
                return rc;
            if (acc_out)
                acc_out[m * N + j] = (int32_t)acc;
            double v = (double)sw[j] * (double)sx[m] * (double)acc;
            y[m * N + j] = bias ? v + (double)bias[j] : v;
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Producers of the activation, fused with its quantisation ([Orin]          */
/* "后续还能继续优化什么", items 1 and 2: RMSNorm, quantisation, SwiGLU and  */
/* the residual add still sit behind separate kernels, and the activation    */
/* quantisation could be fused with the operator before it).  The page names */
/* these operators without defining them; the textbook forms are used:       */
/*   RMSNorm  y_i = h_i / sqrt(mean_k h_k^2 + eps) * gamma_i                 */
/*   SwiGLU   h_i = silu(g_i) * u_i,  silu(g) = g / (1 + e^-g)               */
/* followed by the per-token quantisation above.  Every value that decides   */
/* a code is an fp32 result of a fully specified sequence of IEEE           */
/* operations, so any implementation of the same sequence obtains the same  */
/* codes.                                                                    */
/* ------------------------------------------------------------------------ */

/* e^x in fp32: Cody & Waite's argument reduction x = n ln2 + r with
 * n = round(x / ln2) and ln2 split into a head with 9 significant bits
 * (n * head is exact) and a tail, then the degree-7 Taylor polynomial of
 * e^r (|r| <= ln2 / 2, truncation below 6e-9 relative) in Horner form,
 * coefficients fp32(1/k!), and e^x = p * 2^n.  Every step is one IEEE fp32
 * operation (fmaf is a single rounding).  x is clamped to [-104, 89], where
 * the result already underflows to 0 or overflows to +Inf. */
float orc_exp_f32(float x)
{
    if (x != x)
        return x;
    if (x > 89.0f)
        x = 89.0f;
    if (x < -104.0f)
        x = -104.0f;
    const float n = nearbyintf(x * 1.44269504088896341f);
    float r = fmaf(-n, 0.693359375f, x);
    r = fmaf(-n, -2.12194440054690583e-4f, r);
    float p = (float)(1.0 / 5040.0);
    p = fmaf(p, r, (float)(1.0 / 720.0));
    p = fmaf(p, r, (float)(1.0 / 120.0));
    p = fmaf(p, r, (float)(1.0 / 24.0));
    p = fmaf(p, r, (float)(1.0 / 6.0));
    p = fmaf(p, r, 0.5f);
    p = fmaf(p, r, 1.0f);
    p = fmaf(p, r, 1.0f);
    return ldexpf(p, (int)n);
}

void orc_exp_f32_array(const float* x, int64_t n, float* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_exp_f32(x[i]);
}

/* Residual add, RMSNorm and quantisation of M tokens of K values:
 *   h1 = h + delta                              (fp32; delta may be NULL)
 *   ms = sum_i h1_i^2 / K                       (binary64: each square is exact)
 *   r  = fp32(1 / sqrt(ms + eps))               (binary64, one final rounding)
 *   y_i = (h1_i * r) * gamma_i                  (two fp32 products)
 *   s^x = max|y| / 127, q_i = clip(round(y_i / s^x), -127, 127).
 * h_out (h1) and y_out are optional.  eps >= 0; a token with ms + eps = 0
 * (all zero, eps = 0) normalises to zeros. */
int orc_add_rmsnorm_quant(const float* h, const float* delta, const float* gamma, float eps,
                          int64_t M, int64_t K, float* h_out, float* y_out, int8_t* q, float* s)
{
    if (M < 0 || K <= 0 || !(eps >= 0.0f) || !(eps <= FLT_MAX))
        return ORC_E_ARG;
    for (int64_t i = 0; i < K; ++i)
        if (!(fabsf(gamma[i]) <= FLT_MAX))
            return ORC_E_NONFINITE;
    for (int64_t m = 0; m < M; ++m) {
        const float* hm = h + m * K;
        const float* dm = delta ? delta + m * K : NULL;
        /* residual add and the mean square */
        double ss = 0.0;
        for (int64_t i = 0; i < K; ++i) {
            const float a = dm ? hm[i] + dm[i] : hm[i];
            if (!(fabsf(a) <= FLT_MAX))
                return ORC_E_NONFINITE;
            ss += (double)a * (double)a;
            if (h_out)
                h_out[m * K + i] = a;
        }
        const double v = ss / (double)K + (double)eps;
        const float r = v > 0.0 ? (float)(1.0 / sqrt(v)) : 0.0f;
        if (!(r <= FLT_MAX))
            return ORC_E_RANGE;
        /* normalised values and their largest magnitude */
        float amax = 0.0f;
        for (int64_t i = 0; i < K; ++i) {
            const float a = dm ? hm[i] + dm[i] : hm[i];
            const float y = (a * r) * gamma[i];
            if (!(fabsf(y) <= FLT_MAX))
                return ORC_E_RANGE;
            if (fabsf(y) > amax)
                amax = fabsf(y);
            if (y_out)
                y_out[m * K + i] = y;
        }
        /* per-token quantisation */
        const float sx = amax / 127.0f;
        s[m] = sx;
        for (int64_t i = 0; i < K; ++i) {
            const float a = dm ? hm[i] + dm[i] : hm[i];
            q[m * K + i] = quant_code((a * r) * gamma[i], sx, -127, 127);
        }
    }
    return ORC_OK;
}

/* SwiGLU and quantisation of M tokens.  gu holds each token's fused
 * gate/up projection output, [M, 2I]: gate g = gu[m, 0:I], up u = gu[m, I:2I].
 *   e = exp_f32(-g_i); h_i = (g_i / (1 + e)) * u_i   (fp32, correctly rounded
 *   division), then the per-token quantisation.  h_out is optional. */
int orc_swiglu_quant(const float* gu, int64_t M, int64_t I, float* h_out, int8_t* q, float* s)
{
    if (M < 0 || I <= 0)
        return ORC_E_ARG;
    for (int64_t m = 0; m < M; ++m) {
        const float* g = gu + m * 2 * I;
        const float* u = g + I;
        float* hv = h_out ? h_out + m * I : NULL;
        for (int64_t i = 0; i < I; ++i) {
            if (!(fabsf(g[i]) <= FLT_MAX) || !(fabsf(u[i]) <= FLT_MAX))
                return ORC_E_NONFINITE;
            const float e = orc_exp_f32(-g[i]);
            const float t = (g[i] / (1.0f + e)) * u[i];
            if (!(fabsf(t) <= FLT_MAX))
                return ORC_E_RANGE;
        }
        float amax = 0.0f;
        for (int64_t i = 0; i < I; ++i) {
            const float t = (g[i] / (1.0f + orc_exp_f32(-g[i]))) * u[i];
            if (fabsf(t) > amax)
                amax = fabsf(t);
            if (hv)
                hv[i] = t;
        }
        const float sx = amax / 127.0f;
        s[m] = sx;
        for (int64_t i = 0; i < I; ++i) {
            const float t = (g[i] / (1.0f + orc_exp_f32(-g[i]))) * u[i];
            q[m * I + i] = quant_code(t, sx, -127, 127);
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Packed 6-bit lm_head ([Ascend] 3.2: a Q6_K weight stores 256 weights in  */
/* 210 bytes -- 4-bit low and 2-bit high fields of each 6-bit code, one     */
/* int8 scale per 16 weights and one fp16 scale per 256; the page expands   */
/* it to int8 at load time because decoding the packed fields cost too many */
/* vector instructions on its chip).  The quantiser and the array layout    */
/* below are this library's own (the page gives the sizes, not a rule):     */
/*   sub-block s (16 weights):  t_s = max|w| / 31                (fp32)     */
/*   super-block (256 weights): d = fp16(max_s t_s / 127)                   */
/*                              sc_s = clip(round(t_s / d), 0, 127) (int8)  */
/*   weight i in sub-block s:   q_i = clip(round(w_i / (d * sc_s)), -32, 31)*/
/*   value:                     w_i ~ d * sc_s * q_i                        */
/* with fp32 divisions and round-half-to-even; a zero scale gives zero      */
/* codes.  Storage per row (K % 256 == 0), as separate aligned arrays:      */
/*   ql [K/2] bytes:  u_i = q_i + 32 in [0, 63]; low nibble of u_i in byte  */
/*                    i/2, bits 0-3 for even i, 4-7 for odd i;              */
/*   qh [K/4] bytes:  per 16 weights one little-endian uint32; weight j =   */
/*                    8k + e (k in {0,1}, e in 0..7) puts bits 4-5 of u at  */
/*                    bit 2(e mod 4) + 8k + 16[e >= 4];                     */
/*   sc [K/16] int8;  d [K/256] fp16.                                       */
/* 128 + 64 + 16 + 2 = 210 bytes per 256 weights, as on the page.           */
/* ------------------------------------------------------------------------ */
int orc_quantize_weights_q6k(const float* W, int64_t N, int64_t K, int8_t* q, int8_t* sc,
                             uint16_t* d)
{
    if (N < 0 || K <= 0 || K % 256)
        return ORC_E_ARG;
    for (int64_t j = 0; j < N; ++j) {
        for (int64_t b = 0; b < K / 256; ++b) {
            const float* wb = W + j * K + 256 * b;
            float t[16], tmax = 0.0f;
            for (int s = 0; s < 16; ++s) {
                float m;
                int rc = max_abs_f32(wb + 16 * s, 16, &m);
                if (rc)
                    return rc;
                t[s] = m / 31.0f;
                if (t[s] > tmax)
                    tmax = t[s];
            }
            const uint16_t dh = orc_f32_to_f16(tmax / 127.0f);
            const float df = orc_f16_to_f32(dh);
            d[j * (K / 256) + b] = dh;
            for (int s = 0; s < 16; ++s) {
                const int8_t scs = quant_code(t[s], df, 0, 127);
                sc[j * (K / 16) + 16 * b + s] = scs;
                const float e = df * (float)scs; /* exact: 11 x 7 significant bits */
                for (int i = 0; i < 16; ++i)
                    q[j * K + 256 * b + 16 * s + i] = quant_code(wb[16 * s + i], e, -32, 31);
            }
        }
    }
    return ORC_OK;
}

static int qh_bit(int64_t i)
{
    const int j = (int)(i % 16), k = j / 8, e = j % 8;
    return 2 * (e % 4) + 8 * k + 16 * (e >= 4);
}

int orc_pack_q6k(const int8_t* q, int64_t N, int64_t K, uint8_t* ql, uint8_t* qh)
{
    if (N < 0 || K <= 0 || K % 256)
        return ORC_E_ARG;
    for (int64_t n = 0; n < N * K; ++n)
        if (q[n] < -32 || q[n] > 31)
            return ORC_E_RANGE;
    memset(ql, 0, (size_t)(N * K / 2));
    memset(qh, 0, (size_t)(N * K / 4));
    for (int64_t j = 0; j < N; ++j) {
        for (int64_t i = 0; i < K; ++i) {
            const unsigned u = (unsigned)(q[j * K + i] + 32);
            ql[j * (K / 2) + i / 2] |= (uint8_t)((u & 15u) << (4 * (i % 2)));
            const int bit = qh_bit(i);
            const int64_t word = j * (K / 16) + i / 16; /* one uint32 per 16 weights */
            qh[4 * word + bit / 8] |= (uint8_t)((u >> 4) << (bit % 8));
        }
    }
    return ORC_OK;
}

int orc_unpack_q6k(const uint8_t* ql, const uint8_t* qh, int64_t N, int64_t K, int8_t* q)
{
    if (N < 0 || K <= 0 || K % 256)
        return ORC_E_ARG;
    for (int64_t j = 0; j < N; ++j) {
        for (int64_t i = 0; i < K; ++i) {
            const unsigned lo = (ql[j * (K / 2) + i / 2] >> (4 * (i % 2))) & 15u;
            const int bit = qh_bit(i);
            const int64_t word = j * (K / 16) + i / 16;
            const unsigned hi = (qh[4 * word + bit / 8] >> (bit % 8)) & 3u;
            q[j * K + i] = (int8_t)((int)(lo | (hi << 4)) - 32);
        }
    }
    return ORC_OK;
}

/* y_j = sum_b sum_s fp32(d_b) * sc_s * sum_{i in s} q_i * fp32(x_i), every
 * product exact and the sums in binary64. */
int orc_gemv_q6k_f16(const uint8_t* ql, const uint8_t* qh, const int8_t* sc, const uint16_t* d,
                     const uint16_t* x16, int64_t N, int64_t K, double* y)
{
    if (N < 0 || K <= 0 || K % 256)
        return ORC_E_ARG;
    for (int64_t i = 0; i < K; ++i)
        if (!(fabsf(orc_f16_to_f32(x16[i])) <= FLT_MAX))
            return ORC_E_NONFINITE;
    int8_t qrow[65536];
    if (K > 65536)
        return ORC_E_ARG;
    for (int64_t j = 0; j < N; ++j) {
        int rc = orc_unpack_q6k(ql + j * (K / 2), qh + j * (K / 4), 1, K, qrow);
        if (rc)
            return rc;
        double acc = 0.0;
        for (int64_t s = 0; s < K / 16; ++s) {
            double part = 0.0;
            for (int i = 0; i < 16; ++i)
                part += (double)qrow[16 * s + i] * (double)orc_f16_to_f32(x16[16 * s + i]);
            const double e = (double)orc_f16_to_f32(d[j * (K / 256) + s / 16]) * (double)sc[j * (K / 16) + s];
            acc += e * part;
        }
        y[j] = acc;
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* INT8-X (3,5,8) lossless codec of INT8 weights ("定長無損 INT8 壓縮與       */
/* Triton 融合解碼", sections 2.1-2.5), over the row-major flattened tensor:  */
/*   level 1: |v| <= 3   -> 3-bit two's complement code, stream L1          */
/*   level 2: |v| <= 15  -> 5-bit two's complement code, stream L2          */
/*   level 3: otherwise  -> the raw byte, stream L3                          */
/*   B1: one bit per weight, 1 = not level 1;                                */
/*   B2: one bit per weight outside level 1, in order, 1 = level 3;          */
/*   b1_blk[b], b2_blk[b]: set bits of B1 and of B2 before block b (blocks   */
/*   of blk weights; one extra entry holds the totals).                      */
/* Bit streams are LSB-first: bit p is bit p % 32 of word p / 32.            */
/* ------------------------------------------------------------------------ */
static int int8x_level(int8_t v)
{
    const int a = v < 0 ? -(int)v : (int)v;
    return a <= 3 ? 1 : (a <= 15 ? 2 : 3);
}

static void put_bits(uint32_t* s, int64_t pos, uint32_t val, int width)
{
    for (int k = 0; k < width; ++k)
        if ((val >> k) & 1u)
            s[(pos + k) / 32] |= 1u << ((pos + k) % 32);
}

static uint32_t get_bits(const uint32_t* s, int64_t pos, int width)
{
    uint32_t v = 0;
    for (int k = 0; k < width; ++k)
        v |= ((s[(pos + k) / 32] >> ((pos + k) % 32)) & 1u) << k;
    return v;
}

static int32_t sign_extend(uint32_t v, int width)
{
    return (int32_t)(v << (32 - width)) >> (32 - width);
}

/* Level counts of n weights. */
void orc_int8x_counts(const int8_t* q, int64_t n, int64_t* n1, int64_t* n2, int64_t* n3)
{
    int64_t c[4] = {0, 0, 0, 0};
    for (int64_t t = 0; t < n; ++t)
        c[int8x_level(q[t])]++;
    *n1 = c[1];
    *n2 = c[2];
    *n3 = c[3];
}

/* Encode n weights.  Stream arrays must hold the word counts that the
 * level counts imply (b1: ceil(n/32), b2: ceil((n2+n3)/32), l1:
 * ceil(3 n1/32), l2: ceil(5 n2/32) words; l3: n3 bytes; b1_blk, b2_blk:
 * ceil(n/blk) + 1 entries); they are zeroed here first. */
int orc_int8x_encode(const int8_t* q, int64_t n, int64_t blk, uint32_t* b1, uint32_t* b2, uint32_t* l1,
                     uint32_t* l2, uint8_t* l3, int32_t* b1_blk, int32_t* b2_blk)
{
    if (n <= 0 || blk <= 0 || blk % 32)
        return ORC_E_ARG;
    int64_t n1, n2, n3;
    orc_int8x_counts(q, n, &n1, &n2, &n3);
    memset(b1, 0, (size_t)((n + 31) / 32) * 4);
    memset(b2, 0, (size_t)((n2 + n3 + 31) / 32) * 4);
    memset(l1, 0, (size_t)((3 * n1 + 31) / 32) * 4);
    memset(l2, 0, (size_t)((5 * n2 + 31) / 32) * 4);
    int64_t c1 = 0, c2 = 0, c3 = 0; /* elements of each level so far */
    for (int64_t t = 0; t < n; ++t) {
        if (t % blk == 0) {
            b1_blk[t / blk] = (int32_t)(c2 + c3);
            b2_blk[t / blk] = (int32_t)c3;
        }
        const int lv = int8x_level(q[t]);
        if (lv == 1) {
            put_bits(l1, 3 * c1, (uint32_t)q[t] & 7u, 3);
            ++c1;
            continue;
        }
        b1[t / 32] |= 1u << (t % 32);
        if (lv == 2) {
            put_bits(l2, 5 * c2, (uint32_t)q[t] & 31u, 5);
            ++c2;
        } else {
            b2[(c2 + c3) / 32] |= 1u << ((c2 + c3) % 32);
            l3[c3] = (uint8_t)q[t];
            ++c3;
        }
    }
    const int64_t nb = (n + blk - 1) / blk;
    b1_blk[nb] = (int32_t)(c2 + c3);
    b2_blk[nb] = (int32_t)c3;
    return ORC_OK;
}

/* Decode weights [t0, t0 + count) of an encoded tensor, using the block
 * prefix sums to start at the block of t0 (the decoder of the page's
 * section 2.4: a weight's position in its level's stream is the number of
 * weights of that level before it). */
int orc_int8x_decode(const uint32_t* b1, const uint32_t* b2, const uint32_t* l1, const uint32_t* l2,
                     const uint8_t* l3, const int32_t* b1_blk, const int32_t* b2_blk, int64_t blk,
                     int64_t t0, int64_t count, int8_t* q)
{
    if (blk <= 0 || blk % 32 || t0 < 0 || count < 0)
        return ORC_E_ARG;
    const int64_t b = t0 / blk;
    int64_t nonl1 = b1_blk[b];            /* B1 bits set before the block */
    int64_t c3 = b2_blk[b];               /* level-3 weights before the block */
    int64_t c2 = nonl1 - c3;
    int64_t c1 = b * blk - nonl1;
    for (int64_t t = b * blk; t < t0 + count; ++t) {
        int8_t v;
        if (!((b1[t / 32] >> (t % 32)) & 1u)) {
            v = (int8_t)sign_extend(get_bits(l1, 3 * c1, 3), 3);
            ++c1;
        } else if (!((b2[nonl1 / 32] >> (nonl1 % 32)) & 1u)) {
            v = (int8_t)sign_extend(get_bits(l2, 5 * c2, 5), 5);
            ++c2;
            ++nonl1;
        } else {
            v = (int8_t)l3[c3];
            ++c3;
            ++nonl1;
        }
        if (t >= t0)
            q[t - t0] = v;
    }
    return ORC_OK;
}

/* W8A8 GEMV over INT8-X weights [N, K] with one per-tensor weight scale:
 *   acc_j = sum_i q_ji qx_i (exact),  y_j = sw * sx * acc_j (binary64). */
int orc_gemv_int8x(const uint32_t* b1, const uint32_t* b2, const uint32_t* l1, const uint32_t* l2,
                   const uint8_t* l3, const int32_t* b1_blk, const int32_t* b2_blk, int64_t blk,
                   const int8_t* qx, float sx, float sw, int64_t N, int64_t K, int32_t* acc_out,
                   double* y)
{
    if (N < 0 || K <= 0 || K > 65536)
        return ORC_E_ARG;
    int8_t row[65536];
    for (int64_t j = 0; j < N; ++j) {
        int rc = orc_int8x_decode(b1, b2, l1, l2, l3, b1_blk, b2_blk, blk, j * K, K, row);
        if (rc)
            return rc;
        int64_t acc = 0;
        for (int64_t i = 0; i < K; ++i)
            acc += (int64_t)row[i] * (int64_t)qx[i];
        if (acc > INT32_MAX || acc < INT32_MIN)
            return ORC_E_BOUND;
        if (acc_out)
            acc_out[j] = (int32_t)acc;
        y[j] = (double)sw * (double)sx * (double)acc;
    }
    return ORC_OK;
}
