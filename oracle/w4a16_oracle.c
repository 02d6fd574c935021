/*
 * CPU oracle for the W4A16 quantized linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this file.  Only the test-suite, the smoke check and the CPU
 * baseline leg of the benchmark use it.  It shares no code, header, table or
 * constant with the HIP library: it is a plain, slow, obviously correct
 * restatement of what the method computes.
 *
 * What it computes, and where that is defined:
 *
 *  - Post-training quantization at load time by round-to-nearest, to INT4,
 *    with one scale for every group of 128 weights, activations left in
 *    BF16/FP16: "Kernel dispatch and Humming quantization in PhyAI", section
 *    "Humming makes the separation useful".
 *  - Quantization arithmetic in FP32 and FP32 reference arithmetic:
 *    "Piper Kernels" (piper-kernels 0.7.3), introduction.
 *  - Weight shape [out_features, in_features], input [..., in_features],
 *    output [..., out_features]: "Piper Kernels", section "ConvRot INT8".
 *  - Bias added in FP32 before the final 16-bit conversion:
 *    "Piper Kernels", section "NVFP4 construction".
 *  - A usable scale for an all-zero group is part of the algorithm:
 *    "Piper Kernels", section "Validation contract".
 *
 * Readings taken where the pages are silent (the pages fix only RTN, INT4 and
 * the group size):
 *  - symmetric codes, no zero point; scale s = max|w| / 7 over the group, an
 *    FP32 value obtained by one correctly rounded FP32 division;
 *  - the group runs along K (in_features), 128 consecutive elements of one
 *    output row;
 *  - code q = clamp(round_half_even(fl32(w / s)), -8, 7); s == 0 gives q = 0;
 *  - canonical byte layout: codes[n][j] holds q[n][2j] in the low nibble and
 *    q[n][2j+1] in the high nibble, two's complement;
 *  - dequantized weight W^[n][k] = q[n][k] * s[n][k/128] (exact in double);
 *  - y[m][n] = sum_k x[m][k] * W^[n][k] + bias[n], accumulated in double
 *    (the plain definition; it is more accurate than any FP32 order) and
 *    returned unrounded.
 *
 * Activations fused into a linear's input ("Piper Kernels", section "ConvRot
 * INT8": the SwiGLU input row is [up | gate] of twice the layer's in_features
 * and gives up * silu(gate); the GELU input is tanh-approximate GELU of the
 * row; fused activation preparation keeps FP32 arithmetic, section "ConvRot
 * INT8 ... FFN", and outputs keep the input dtype).  Readings: the activation
 * is evaluated in double here (more accurate than the FP32 it asks for) and
 * rounded once, to the nearest 16-bit value of the input dtype (ties to
 * even), which is then the layer's input, as a separately materialised
 * activation would be.
 *
 * INT8 weights (the Humming integration also supports INT8 weight schemes:
 * "Kernel dispatch and Humming quantization in PhyAI", section "Choose
 * precision by layer and hardware"): the same round-to-nearest quantizer with
 * one FP32 scale per group of 128, the scale mapping the group's largest
 * magnitude onto code 127 (reading: symmetric, s = amax / 127, codes
 * clamp(round_half_even(w / s), -128, 127)), one signed code per byte.
 *
 * Updates of a quantized weight ("Piper Kernels", sections "ConvRot INT8"
 * (add_ / addmm_ with an optional rounding_seed, requantizing the result)
 * and "Stochastic quantization"): W' = beta * dequant(W) + alpha * U, U a
 * dense update or a low-rank product mat1 @ mat2 accumulated in FP32, then
 * requantized with the same deterministic scales as round-to-nearest; with a
 * seed, each code is one of the two adjacent codes with probability
 * proportional to distance (values outside the code range and exact hits are
 * never perturbed), drawn by logical element offset from a seeded generator.
 * Readings: every step is one FP32 operation in this order --
 *   d = fl32(q * s); p = U widened to FP32, or p = fma(mat1[n][r], mat2[r][k], p)
 *   over r ascending from p = 0; w' = fma(alpha, p, fl32(beta * d)) --
 *   then the quantizer above on w'.  The generator is SplitMix64 (Steele, Lea
 *   and Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014):
 *   element e of the weight (row-major offset n * K + k) draws the (e+1)-th
 *   output of SplitMix64 seeded with the 64-bit seed; its top 24 bits give a
 *   uniform u in [0, 1) (u = bits * 2^-24), and the code rounds up exactly
 *   when u < v - floor(v), v = fl32(w' / s').  The same update applies to
 *   INT8 weights with the INT8 quantizer and code range (bits = 8), as the
 *   pages describe it for their 8-bit codes.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fopenmp -fPIC -shared
 * The quantizer relies on IEEE binary32 division and on nearbyintf under the
 * default round-to-nearest-even mode; -ffp-contract=off keeps every step a
 * separately rounded operation.
 */
#define _GNU_SOURCE
#include <fenv.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_GROUP 128

/* dtype tags used by the entry points below (their own numbering) */
#define ORACLE_F32 0
#define ORACLE_BF16 1
#define ORACLE_F16 2

/* ---- 16-bit floating-point decoding, written from the format definitions ---- */

/* bfloat16 is, by definition, the upper half of an IEEE binary32 pattern. */
double oracle_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_f16_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);              /* subnormal: f * 2^-24 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);  /* (1 + f/1024) * 2^(e-15) */
    return sign ? -v : v;
}

static double decode16(uint16_t bits, int dtype)
{
    return dtype == ORACLE_BF16 ? oracle_bf16_to_double(bits) : oracle_f16_to_double(bits);
}

/* A weight element as FP32.  16-bit inputs widen exactly to FP32. */
static float weight_as_float(const void *w, int dtype, int64_t idx)
{
    if (dtype == ORACLE_F32)
        return ((const float *)w)[idx];
    return (float)decode16(((const uint16_t *)w)[idx], dtype);
}

/* ---- round-to-nearest INT4 quantization, one FP32 scale per group of 128 ---- */

/*
 * w: [n][ldw] elements of dtype w_dtype (only the first k of each row are used)
 * q: [n][k] one signed code per byte, s: [n][k/128] FP32 scales.
 * Returns 0, or -1 when k is not a positive multiple of 128.
 */
int oracle_quantize(const void *w, int w_dtype, int64_t n, int64_t k, int64_t ldw,
                    int8_t *q, float *s)
{
    if (k <= 0 || k % ORACLE_GROUP != 0 || ldw < k || n < 0)
        return -1;
    if (fegetround() != FE_TONEAREST)
        fesetround(FE_TONEAREST);
    const int64_t groups = k / ORACLE_GROUP;
    for (int64_t row = 0; row < n; ++row) {
        for (int64_t g = 0; g < groups; ++g) {
            /* step 1: the group's largest magnitude */
            float amax = 0.0f;
            for (int64_t j = 0; j < ORACLE_GROUP; ++j) {
                float a = fabsf(weight_as_float(w, w_dtype, row * ldw + g * ORACLE_GROUP + j));
                if (a > amax)
                    amax = a;
            }
            /* step 2: the scale maps the largest magnitude onto code 7 */
            float scale = amax / 7.0f;
            s[row * groups + g] = scale;
            /* step 3: each code is the quotient rounded to the nearest integer */
            for (int64_t j = 0; j < ORACLE_GROUP; ++j) {
                int64_t kk = g * ORACLE_GROUP + j;
                int code = 0;
                if (scale != 0.0f) {
                    float ratio = weight_as_float(w, w_dtype, row * ldw + kk) / scale;
                    float r = nearbyintf(ratio);   /* ties go to the even integer */
                    if (r < -8.0f)
                        r = -8.0f;
                    if (r > 7.0f)
                        r = 7.0f;
                    code = (int)r;
                }
                q[row * k + kk] = (int8_t)code;
            }
        }
    }
    return 0;
}

/*
 * Round-to-nearest INT8 quantization with one FP32 scale per group of 128.
 * w: [n][ldw] of w_dtype; q: [n][k] one signed code per byte (the canonical
 * INT8 storage), s: [n][k/128].  Returns 0, or -1 on a bad shape.
 */
int oracle_quantize_int8(const void *w, int w_dtype, int64_t n, int64_t k, int64_t ldw,
                         int8_t *q, float *s)
{
    if (k <= 0 || k % ORACLE_GROUP != 0 || ldw < k || n < 0)
        return -1;
    if (fegetround() != FE_TONEAREST)
        fesetround(FE_TONEAREST);
    const int64_t groups = k / ORACLE_GROUP;
    for (int64_t row = 0; row < n; ++row) {
        for (int64_t g = 0; g < groups; ++g) {
            float amax = 0.0f;
            for (int64_t j = 0; j < ORACLE_GROUP; ++j) {
                float mag = fabsf(weight_as_float(w, w_dtype, row * ldw + g * ORACLE_GROUP + j));
                if (mag > amax)
                    amax = mag;
            }
            /* the scale maps the largest magnitude onto code 127 */
            float scale8 = amax / 127.0f;
            s[row * groups + g] = scale8;
            for (int64_t j = 0; j < ORACLE_GROUP; ++j) {
                int64_t kk = g * ORACLE_GROUP + j;
                int code8 = 0;
                if (scale8 != 0.0f) {
                    float r8 = nearbyintf(weight_as_float(w, w_dtype, row * ldw + kk) / scale8);
                    if (r8 < -128.0f)
                        r8 = -128.0f;
                    if (r8 > 127.0f)
                        r8 = 127.0f;
                    code8 = (int)r8;
                }
                q[row * k + kk] = (int8_t)code8;
            }
        }
    }
    return 0;
}

/* Canonical storage: two codes per byte, even k in the low nibble. */
void oracle_codes_to_nibbles(const int8_t *q, int64_t n, int64_t k, uint8_t *codes)
{
    for (int64_t row = 0; row < n; ++row)
        for (int64_t j = 0; j < k / 2; ++j) {
            unsigned lo = (unsigned)q[row * k + 2 * j] & 0xFu;
            unsigned hi = (unsigned)q[row * k + 2 * j + 1] & 0xFu;
            codes[row * (k / 2) + j] = (uint8_t)(lo | (hi << 4));
        }
}

/* Inverse of the canonical storage: sign-extend each nibble. */
void oracle_nibbles_to_codes(const uint8_t *codes, int64_t n, int64_t k, int8_t *q)
{
    for (int64_t row = 0; row < n; ++row)
        for (int64_t kk = 0; kk < k; ++kk) {
            unsigned byte = codes[row * (k / 2) + kk / 2];
            int v = (kk % 2 == 0) ? (int)(byte & 0xFu) : (int)(byte >> 4);
            q[row * k + kk] = (int8_t)(v >= 8 ? v - 16 : v);
        }
}

/* Dequantized weight W^[n][k] = q * s, exact in double. */
void oracle_dequantize(const int8_t *q, const float *s, int64_t n, int64_t k, double *w_hat)
{
    const int64_t groups = k / ORACLE_GROUP;
    for (int64_t row = 0; row < n; ++row)
        for (int64_t kk = 0; kk < k; ++kk)
            w_hat[row * k + kk] = (double)q[row * k + kk] * (double)s[row * groups + kk / ORACLE_GROUP];
}

/* ---- the quantized linear layer: y = x . W^T + bias ---- */

/* One output element, straight from the definition, k ascending. */
static double one_output(const uint16_t *x, int x_dtype, int64_t ldx, int64_t i,
                         const int8_t *q, const float *s, int64_t k, int64_t j,
                         const uint16_t *bias)
{
    const int64_t groups = k / ORACLE_GROUP;
    double acc = 0.0;
    for (int64_t kk = 0; kk < k; ++kk) {
        double xv = decode16(x[i * ldx + kk], x_dtype);
        double wv = (double)q[j * k + kk] * (double)s[j * groups + kk / ORACLE_GROUP];
        acc += xv * wv;
    }
    if (bias)
        acc += decode16(bias[j], x_dtype);
    return acc;
}

/*
 * x: [m][ldx] 16-bit activations of dtype x_dtype (BF16 or F16)
 * q, s: codes [n][k] and scales [n][k/128] as produced by oracle_quantize
 * bias: [n] of x_dtype, or NULL.  y: [m][n] doubles (not rounded to 16 bits).
 */
int oracle_linear(const uint16_t *x, int x_dtype, int64_t m, int64_t k, int64_t ldx,
                  const int8_t *q, const float *s, int64_t n, const uint16_t *bias, double *y)
{
    if (k <= 0 || k % ORACLE_GROUP != 0 || ldx < k || m < 0 || n < 0)
        return -1;
    if (x_dtype != ORACLE_BF16 && x_dtype != ORACLE_F16)
        return -1;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j)
            y[i * n + j] = one_output(x, x_dtype, ldx, i, q, s, k, j, bias);
    return 0;
}

/* The same computation for a list of (row, column) output positions. */
int oracle_linear_entries(const uint16_t *x, int x_dtype, int64_t m, int64_t k, int64_t ldx,
                          const int8_t *q, const float *s, int64_t n, const uint16_t *bias,
                          const int64_t *rows, const int64_t *cols, int64_t count, double *out)
{
    if (k <= 0 || k % ORACLE_GROUP != 0 || ldx < k || m < 0 || n < 0)
        return -1;
    if (x_dtype != ORACLE_BF16 && x_dtype != ORACLE_F16)
        return -1;
    for (int64_t e = 0; e < count; ++e)
        if (rows[e] < 0 || rows[e] >= m || cols[e] < 0 || cols[e] >= n)
            return -1;
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < count; ++e)
        out[e] = one_output(x, x_dtype, ldx, rows[e], q, s, k, cols[e], bias);
    return 0;
}

/* ---- activations fused into the input of a linear layer ---- */

#define ORACLE_ACT_SWIGLU 1
#define ORACLE_ACT_GELU_TANH 2

/*
 * Nearest 16-bit value of a double, ties to the even significand, from the
 * format definitions:
 *   BF16: 8 significant bits, normal numbers from 2^-126 (the binary32
 *         exponent range), subnormal spacing 2^-133, exponent bias 127;
 *   F16:  11 significant bits, normal numbers from 2^-14, subnormal spacing
 *         2^-24, exponent bias 15, largest finite 65504.
 * Magnitudes that round beyond the largest finite value give infinity.
 * Returns the bit pattern.
 */
uint16_t oracle_round16(double v, int dtype)
{
    const int p = dtype == ORACLE_BF16 ? 8 : 11;          /* significant bits */
    const int emin = dtype == ORACLE_BF16 ? -126 : -14;   /* smallest normal exponent */
    const int emax = dtype == ORACLE_BF16 ? 127 : 15;     /* largest exponent */
    const int bias = dtype == ORACLE_BF16 ? 127 : 15;
    const int mbits = p - 1;                               /* stored fraction bits */
    const unsigned sign = signbit(v) ? 1u : 0u;
    if (isnan(v))
        return (uint16_t)((sign << 15) | (dtype == ORACLE_BF16 ? 0x7fc0u : 0x7e00u));
    double a = fabs(v);
    const uint16_t inf = (uint16_t)((sign << 15) | (((1u << (15 - mbits)) - 1u) << mbits));
    if (isinf(a))
        return inf;
    if (a == 0.0)
        return (uint16_t)(sign << 15);
    int e2;
    frexp(a, &e2);                       /* a = f * 2^e2, f in [0.5, 1) */
    int e = e2 - 1;                      /* exponent of the leading bit */
    int q = (e < emin ? emin : e) - mbits;          /* exponent of one unit in the last place */
    double units = nearbyint(ldexp(a, -q));         /* ties to even under the default mode */
    double r = ldexp(units, q);
    if (r >= ldexp(1.0, emax + 1))
        return inf;
    if (r < ldexp(1.0, emin))            /* subnormal (or rounded to zero) */
        return (uint16_t)((sign << 15) | (unsigned)units);
    frexp(r, &e2);
    e = e2 - 1;
    unsigned frac = (unsigned)(ldexp(r, mbits - e) - ldexp(1.0, mbits));
    return (uint16_t)((sign << 15) | ((unsigned)(e + bias) << mbits) | frac);
}

/*
 * The activation's value for one element (double arithmetic):
 *   SwiGLU:    up * silu(gate), silu(g) = g / (1 + e^-g);
 *   GELU_TANH: x/2 * (1 + tanh(u)), u = sqrt(2/pi) * (x + 0.044715 x^3),
 *              x = v, evaluated as x / (1 + e^-2u): the same function
 *              ((1 + tanh u) / 2 = 1 / (1 + e^-2u)) without the cancellation
 *              of 1 + tanh(u) for large negative x.
 * For GELU_TANH the second argument is ignored.
 */
double oracle_act_value(double v, double up, int act)
{
    if (act == ORACLE_ACT_SWIGLU)
        return up * (v / (1.0 + exp(-v)));
    const double u = sqrt(2.0 / M_PI) * (v + 0.044715 * v * v * v);
    return v / (1.0 + exp(-2.0 * u));
}

/*
 * x: [m][ldx] 16-bit values of dtype x_dtype.  SwiGLU rows hold [up | gate],
 * up in columns 0..k-1 and gate in columns k..2k-1 (ldx >= 2k); GELU rows
 * hold k values.  a: [m][k] bit patterns of the activated input, each value
 * rounded once to x_dtype.  Returns 0, or -1 on a bad argument.
 */
int oracle_activate(const uint16_t *x, int x_dtype, int act, int64_t m, int64_t k, int64_t ldx,
                    uint16_t *a)
{
    if (k <= 0 || m < 0 || (x_dtype != ORACLE_BF16 && x_dtype != ORACLE_F16))
        return -1;
    if (act != ORACLE_ACT_SWIGLU && act != ORACLE_ACT_GELU_TANH)
        return -1;
    if (ldx < (act == ORACLE_ACT_SWIGLU ? 2 * k : k))
        return -1;
    if (fegetround() != FE_TONEAREST)
        fesetround(FE_TONEAREST);
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < k; ++j) {
            double v;
            if (act == ORACLE_ACT_SWIGLU) {
                double up = decode16(x[i * ldx + j], x_dtype);
                double gate = decode16(x[i * ldx + k + j], x_dtype);
                v = oracle_act_value(gate, up, act);
            } else {
                v = oracle_act_value(decode16(x[i * ldx + j], x_dtype), 0.0, act);
            }
            a[i * k + j] = oracle_round16(v, x_dtype);
        }
    return 0;
}

/* ---- updates of a quantized weight, with optional stochastic rounding ---- */

/* The (e+1)-th output of SplitMix64 seeded with `seed`. */
uint64_t oracle_splitmix64(uint64_t seed, uint64_t e)
{
    uint64_t z = seed + (e + 1) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* Uniform in [0, 1) with 24 bits, for element e. */
float oracle_uniform(uint64_t seed, uint64_t e)
{
    return (float)(oracle_splitmix64(seed, e) >> 40) * 0x1p-24f;
}

static float update_value(const void *u, int u_dtype, int64_t idx)
{
    return weight_as_float(u, u_dtype, idx);
}

/*
 * In place on canonical codes q [n][k] and scales s [n][k/128]:
 *   rank == 0: W' = beta * dequant + alpha * upd, upd [n][k] (row stride ldu)
 *   rank  > 0: W' = beta * dequant + alpha * (mat1 @ mat2), mat1 [n][rank],
 *              mat2 [rank][k], both row-major of dtype u_dtype
 * then requantized (round to nearest, or stochastic when has_seed).
 * u_dtype: F32, BF16 or F16.  Returns 0, or -1 on a bad argument.
 */
int oracle_update(int8_t *q, float *s, int64_t n, int64_t k, const void *upd, int64_t ldu,
                  const void *mat1, const void *mat2, int64_t rank, int u_dtype,
                  float alpha, float beta, int has_seed, uint64_t seed, int bits)
{
    if (k <= 0 || k % ORACLE_GROUP != 0 || n < 0 || rank < 0)
        return -1;
    if (bits != 4 && bits != 8)
        return -1;
    /* the code range of the weight's format: [-8, 7] or [-128, 127] */
    const int qmax = bits == 8 ? 127 : 7;
    const int qmin = -qmax - 1;
    if (u_dtype != ORACLE_F32 && u_dtype != ORACLE_BF16 && u_dtype != ORACLE_F16)
        return -1;
    if (rank == 0 && (!upd || ldu < k))
        return -1;
    if (rank > 0 && (!mat1 || !mat2))
        return -1;
    if (fegetround() != FE_TONEAREST)
        fesetround(FE_TONEAREST);
    const int64_t groups = k / ORACLE_GROUP;
    float w[ORACLE_GROUP];
    for (int64_t row = 0; row < n; ++row) {
        for (int64_t g = 0; g < groups; ++g) {
            /* the updated group in FP32 */
            const float sc = s[row * groups + g];
            for (int64_t j = 0; j < ORACLE_GROUP; ++j) {
                const int64_t kk = g * ORACLE_GROUP + j;
                const float d = (float)q[row * k + kk] * sc;
                float p;
                if (rank == 0) {
                    p = update_value(upd, u_dtype, row * ldu + kk);
                } else {
                    p = 0.0f;
                    for (int64_t r = 0; r < rank; ++r)
                        p = fmaf(update_value(mat1, u_dtype, row * rank + r),
                                 update_value(mat2, u_dtype, r * k + kk), p);
                }
                const float bd = beta * d;
                w[j] = fmaf(alpha, p, bd);
            }
            /* requantize: the scale of round-to-nearest, then the codes */
            float amax = 0.0f;
            for (int j = 0; j < ORACLE_GROUP; ++j)
                if (fabsf(w[j]) > amax)
                    amax = fabsf(w[j]);
            const float scale = amax / (float)qmax;
            s[row * groups + g] = scale;
            for (int64_t j = 0; j < ORACLE_GROUP; ++j) {
                const int64_t kk = g * ORACLE_GROUP + j;
                int code = 0;
                if (scale != 0.0f) {
                    const float v = w[j] / scale;
                    const float lo = floorf(v);
                    if (has_seed && lo >= (float)qmin && lo + 1.0f <= (float)qmax) {
                        /* interior: one of the two adjacent codes */
                        const float frac = v - lo;
                        const float u = oracle_uniform(seed, (uint64_t)(row * k + kk));
                        code = (int)lo + (u < frac ? 1 : 0);
                    } else {
                        float r = nearbyintf(v);
                        if (r < (float)qmin)
                            r = (float)qmin;
                        if (r > (float)qmax)
                            r = (float)qmax;
                        code = (int)r;
                    }
                }
                q[row * k + kk] = (int8_t)code;
            }
        }
    }
    return 0;
}

/* Number of OpenMP threads a parallel region uses (reported by the baseline). */
int oracle_num_threads(void)
{
    int t = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            t = omp_get_num_threads();
#endif
        }
    }
    return t;
}
