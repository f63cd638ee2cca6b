/*
 * convrot_oracle.c -- CPU oracle for the INT8 ConvRot linear layer.
 *
 * TEST INFRASTRUCTURE ONLY (see convrot_oracle.h).  Plain scalar C99, one
 * thread, no intrinsics, no blocking or fusion.  Build it with
 *   gcc -O2 -std=c99 -ffp-contract=off -fno-fast-math -fPIC -shared
 * so that every float operation below is one IEEE binary32 operation in
 * round-to-nearest-even, in the order written.
 *
 * Sources of each step:
 *  - page "int8 Compute" (InvokeAI docs), opening section: the activation is
 *    rotated and coded as int8 with one scale per token, the integer codes of
 *    activation and weight are multiplied together, and the weight is stored
 *    as int8 codes with one scale for the whole tensor.
 *  - same page, "What stays on the default path": rotation is done in
 *    groups (256 in every published build); without it one outlier channel
 *    sets the scale of a whole token.
 *  - page "Explanation of INT8 ConvRot", "What is INT8 ConvRot?": group-wise
 *    rotation applied block by block, like a convolution.
 *  - page "int8 Compute", "What stays on the default path": compute is BF16
 *    (outputs are bf16 here).
 * The matrix, rounding and scale formulas the pages leave open are the
 * readings stated in convrot_oracle.h.
 */
#include "convrot_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

static int is_pow2(int g) { return g >= 1 && (g & (g - 1)) == 0; }

float oracle_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0)
        return 0x7fc0; /* NaN (never produced on the tested path) */
    /* round to nearest, ties to even, on the 16 dropped bits */
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * Widening decodes the three classes (zero/subnormal, normal, inf/NaN)
 * exactly. */
float oracle_f16_to_f32(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int e = (h >> 10) & 0x1f;
    const int m = h & 0x3ff;
    float v;
    if (e == 0)
        v = ldexpf((float)m, -24);                 /* m * 2^-24: zero or subnormal */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexpf((float)(1024 + m), e - 25);     /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* Narrowing to binary16, round to nearest, ties to even.  Magnitudes of at
 * least 65520 (halfway between the largest finite 65504 and 2^16) become
 * infinity; below 2^-14 the spacing is the subnormal quantum 2^-24. */
uint16_t oracle_f32_to_f16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    const uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    u &= 0x7fffffffu;
    if (u > 0x7f800000u) return (uint16_t)(sign | 0x7e00u);      /* NaN */
    if (u >= 0x477ff000u) return (uint16_t)(sign | 0x7c00u);     /* >= 65520: inf */
    if (u < 0x38800000u) {                                        /* below 2^-14 */
        float a;
        memcpy(&a, &u, sizeof a);
        /* a * 2^24 is exact; nearbyintf rounds half to even */
        return (uint16_t)(sign | (uint16_t)nearbyintf(a * 16777216.0f));
    }
    /* normal: rebias the exponent, keep 10 of the 23 fraction bits, round on
     * the 13 dropped ones (a carry out of the fraction bumps the exponent) */
    uint32_t h = ((((u >> 23) & 0xffu) - 127u + 15u) << 10) | ((u >> 13) & 0x3ffu);
    const uint32_t rem = u & 0x1fffu;
    if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h += 1u;
    return (uint16_t)(sign | h);
}

static float io_to_f32(uint16_t b, int io_f16)
{
    return io_f16 ? oracle_f16_to_f32(b) : oracle_bf16_to_f32(b);
}

static uint16_t f32_to_io(float f, int io_f16)
{
    return io_f16 ? oracle_f32_to_f16(f) : oracle_f32_to_bf16(f);
}

float oracle_rot_scale(int g)
{
    return (float)(1.0 / sqrt((double)g));
}

/* O1.  Sylvester Hadamard: H[i][j] = (-1)^popcount(i & j). */
int oracle_hadamard(int g, int32_t *H)
{
    if (!is_pow2(g) || H == NULL) return -1;
    for (int i = 0; i < g; ++i) {
        for (int j = 0; j < g; ++j) {
            int bits = i & j, parity = 0;
            while (bits) { parity ^= bits & 1; bits >>= 1; }
            H[(int64_t)i * g + j] = parity ? -1 : 1;
        }
    }
    return 0;
}

/* O2 on one block of g floats: butterfly with half-span h ascending, then
 * the normalisation multiply.  H_g v equals this butterfly because the
 * Sylvester matrix factors as a product of one (a+b, a-b) stage per bit of
 * the index. */
static void rotate_block(float *v, int g, float c)
{
    for (int h = 1; h < g; h <<= 1) {
        for (int i = 0; i < g; i += 2 * h) {
            for (int j = i; j < i + h; ++j) {
                float a = v[j];
                float b = v[j + h];
                v[j] = a + b;
                v[j + h] = a - b;
            }
        }
    }
    for (int j = 0; j < g; ++j) v[j] = v[j] * c;
}

int oracle_rotate_rows(float *v, int64_t rows, int64_t K, int g)
{
    if (!is_pow2(g) || rows < 0 || K < 0 || (K % g) != 0 || (rows > 0 && K > 0 && v == NULL))
        return -1;
    float c = oracle_rot_scale(g);
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < K; b += g)
            rotate_block(v + r * K + b, g, c);
    return 0;
}

/* Symmetric int8 code of v under scale s: clamp(rne(v / s), -127, 127).
 * nearbyintf rounds half to even in the default rounding mode. */
static int8_t quant_code(float v, float s)
{
    if (s == 0.0f) return 0;
    float r = nearbyintf(v / s);
    if (r > 127.0f) r = 127.0f;
    if (r < -127.0f) r = -127.0f;
    return (int8_t)r;
}

/* O3.  Tensorwise: one absmax over the whole rotated weight. */
int oracle_quant_weight(const float *w, int64_t N, int64_t K, int g,
                        int8_t *wq, float *s_w, float *w_rot)
{
    if (!is_pow2(g) || N < 1 || K < 1 || (K % g) != 0 || w == NULL || wq == NULL || s_w == NULL)
        return -1;
    float *rot = w_rot ? w_rot : (float *)malloc((size_t)(N * K) * sizeof(float));
    if (rot == NULL) return -3;
    memcpy(rot, w, (size_t)(N * K) * sizeof(float));
    oracle_rotate_rows(rot, N, K, g);

    float amax = 0.0f;
    for (int64_t i = 0; i < N * K; ++i) {
        float a = fabsf(rot[i]);
        if (a > amax) amax = a;
    }
    float s = amax / 127.0f;
    for (int64_t i = 0; i < N * K; ++i) wq[i] = quant_code(rot[i], s);
    *s_w = s;
    if (rot != w_rot) free(rot);
    return 0;
}

/* Row-wise variant of O3: the same rotation, one absmax and one scale per
 * output channel (row n), as for a token in O4. */
int oracle_quant_weight_rows(const float *w, int64_t N, int64_t K, int g,
                             int8_t *wq, float *s_w, float *w_rot)
{
    if (!is_pow2(g) || N < 1 || K < 1 || (K % g) != 0 || w == NULL || wq == NULL || s_w == NULL)
        return -1;
    float *rot = (float *)malloc((size_t)K * sizeof(float));
    if (rot == NULL) return -3;
    for (int64_t n = 0; n < N; ++n) {
        memcpy(rot, w + n * K, (size_t)K * sizeof(float));
        oracle_rotate_rows(rot, 1, K, g);
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float a = fabsf(rot[k]);
            if (a > amax) amax = a;
        }
        float s = amax / 127.0f;
        for (int64_t k = 0; k < K; ++k) wq[n * K + k] = quant_code(rot[k], s);
        s_w[n] = s;
        if (w_rot) memcpy(w_rot + n * K, rot, (size_t)K * sizeof(float));
    }
    free(rot);
    return 0;
}

/* O4 for one token row: widen bf16 (or fp16) -> fp32, rotate, absmax,
 * scale, codes. */
static void quant_act_row(const uint16_t *xrow, int io_f16, int64_t K, int g, float *rot,
                          int8_t *qrow, float *srow)
{
    for (int64_t k = 0; k < K; ++k) rot[k] = io_to_f32(xrow[k], io_f16);
    oracle_rotate_rows(rot, 1, K, g);
    float amax = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
        float a = fabsf(rot[k]);
        if (a > amax) amax = a;
    }
    float s = amax / 127.0f;
    for (int64_t k = 0; k < K; ++k) qrow[k] = quant_code(rot[k], s);
    *srow = s;
}

int oracle_quant_act(const uint16_t *x, int64_t M, int64_t K, int g,
                     int8_t *q, float *s, float *x_rot)
{
    return oracle_quant_act_ex(x, 0, M, K, g, q, s, x_rot);
}

int oracle_quant_act_ex(const uint16_t *x, int io_f16, int64_t M, int64_t K, int g,
                        int8_t *q, float *s, float *x_rot)
{
    if (!is_pow2(g) || M < 0 || K < 1 || (K % g) != 0 || (M > 0 && (x == NULL || q == NULL || s == NULL)))
        return -1;
    float *rot = (float *)malloc((size_t)K * sizeof(float));
    if (rot == NULL) return -3;
    for (int64_t m = 0; m < M; ++m) {
        quant_act_row(x + m * K, io_f16, K, g, rot, q + m * K, s + m);
        if (x_rot) memcpy(x_rot + m * K, rot, (size_t)K * sizeof(float));
    }
    free(rot);
    return 0;
}

/* O5.  Exact integer dot products; int64 accumulation, then a range check. */
int oracle_gemm_i32(const int8_t *a, const int8_t *b, int64_t M, int64_t N,
                    int64_t K, int32_t *acc)
{
    if (M < 0 || N < 0 || K < 0 || ((M > 0 && N > 0) && (a == NULL || b == NULL || acc == NULL)))
        return -1;
    int rc = 0;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            int64_t sum = 0;
            for (int64_t k = 0; k < K; ++k)
                sum += (int64_t)a[m * K + k] * (int64_t)b[n * K + k];
            if (sum > INT32_MAX || sum < INT32_MIN) rc = -2;
            acc[m * N + n] = (int32_t)sum;
        }
    }
    return rc;
}

/* O6.  alpha = s_x[m] * s_w first, then one fused multiply-add with the
 * bias, then one rounding to bf16. */
int oracle_epilogue(const int32_t *acc, const float *s_x, float s_w,
                    const uint16_t *bias, int64_t M, int64_t N, uint16_t *y)
{
    if (M < 0 || N < 0 || ((M > 0 && N > 0) && (acc == NULL || s_x == NULL || y == NULL)))
        return -1;
    for (int64_t m = 0; m < M; ++m) {
        float alpha = s_x[m] * s_w;
        for (int64_t n = 0; n < N; ++n) {
            float bn = bias ? oracle_bf16_to_f32(bias[n]) : 0.0f;
            float v = fmaf((float)acc[m * N + n], alpha, bn);
            y[m * N + n] = oracle_f32_to_bf16(v);
        }
    }
    return 0;
}

/* O6 with the variants: s_w holds one scale (row_scale = 0) or one per
 * output channel (row_scale = 1), alpha = s_x[m] * s_w[n or 0] in fp32; the
 * bias and the output are bf16 (io_f16 = 0) or fp16 (io_f16 = 1) bits. */
int oracle_epilogue_ex(const int32_t *acc, const float *s_x, const float *s_w, int row_scale,
                       const uint16_t *bias, int io_f16, int64_t M, int64_t N, uint16_t *y)
{
    if (M < 0 || N < 0 || ((M > 0 && N > 0) && (acc == NULL || s_x == NULL || s_w == NULL || y == NULL)))
        return -1;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            float alpha = s_x[m] * s_w[row_scale ? n : 0];
            float bn = bias ? io_to_f32(bias[n], io_f16) : 0.0f;
            float v = fmaf((float)acc[m * N + n], alpha, bn);
            y[m * N + n] = f32_to_io(v, io_f16);
        }
    }
    return 0;
}

int oracle_linear_rows(const uint16_t *x, int64_t M, int64_t K,
                       const int64_t *rows, int64_t R,
                       const int8_t *wq, float s_w, int64_t N, int g,
                       const uint16_t *bias, uint16_t *y,
                       int8_t *q_rows, float *s_rows)
{
    if (!is_pow2(g) || M < 1 || K < 1 || N < 1 || R < 0 || (K % g) != 0 ||
        x == NULL || wq == NULL || y == NULL || (R > 0 && rows == NULL))
        return -1;
    for (int64_t r = 0; r < R; ++r)
        if (rows[r] < 0 || rows[r] >= M) return -1;

    float *rot = (float *)malloc((size_t)K * sizeof(float));
    int8_t *q = (int8_t *)malloc((size_t)K);
    int32_t *acc = (int32_t *)malloc((size_t)N * sizeof(int32_t));
    if (!rot || !q || !acc) { free(rot); free(q); free(acc); return -3; }

    int rc = 0;
    for (int64_t r = 0; r < R; ++r) {
        float s;
        quant_act_row(x + rows[r] * K, 0, K, g, rot, q, &s);
        if (oracle_gemm_i32(q, wq, 1, N, K, acc) != 0) rc = -2;
        oracle_epilogue(acc, &s, s_w, bias, 1, N, y + r * N);
        if (q_rows) memcpy(q_rows + r * K, q, (size_t)K);
        if (s_rows) s_rows[r] = s;
    }
    free(rot); free(q); free(acc);
    return rc;
}

int oracle_linear_rows_ex(const uint16_t *x, int io_f16, int64_t M, int64_t K,
                          const int64_t *rows, int64_t R,
                          const int8_t *wq, const float *s_w, int row_scale, int64_t N, int g,
                          const uint16_t *bias, uint16_t *y,
                          int8_t *q_rows, float *s_rows)
{
    if (!is_pow2(g) || M < 1 || K < 1 || N < 1 || R < 0 || (K % g) != 0 ||
        x == NULL || wq == NULL || s_w == NULL || y == NULL || (R > 0 && rows == NULL))
        return -1;
    for (int64_t r = 0; r < R; ++r)
        if (rows[r] < 0 || rows[r] >= M) return -1;

    float *rot = (float *)malloc((size_t)K * sizeof(float));
    int8_t *q = (int8_t *)malloc((size_t)K);
    int32_t *acc = (int32_t *)malloc((size_t)N * sizeof(int32_t));
    if (!rot || !q || !acc) { free(rot); free(q); free(acc); return -3; }

    int rc = 0;
    for (int64_t r = 0; r < R; ++r) {
        float s;
        quant_act_row(x + rows[r] * K, io_f16, K, g, rot, q, &s);
        if (oracle_gemm_i32(q, wq, 1, N, K, acc) != 0) rc = -2;
        oracle_epilogue_ex(acc, &s, s_w, row_scale, bias, io_f16, 1, N, y + r * N);
        if (q_rows) memcpy(q_rows + r * K, q, (size_t)K);
        if (s_rows) s_rows[r] = s;
    }
    free(rot); free(q); free(acc);
    return rc;
}

/* ---------------------------------------------------------------- default path
 *
 * The guarded layer is checked against the default path, which keeps
 * unpacking the weight (page "int8 Compute", InvokeAI docs, "When something
 * goes wrong" and "What stays on the default path").  Unpacking a rotated
 * int8 weight: dequantize each row (s_w * q in fp32) and rotate it back by R.
 * R = blockdiag(H_g / sqrt(g)) is symmetric and orthogonal, so R^-1 = R and
 * the same O2 butterfly undoes the rotation; the result is rounded to the
 * compute format.  The layer is then the plain product of the (unrotated)
 * activation with the unpacked weight, plus the bias.
 */
int oracle_unpack_weight(const int8_t *wq, const float *s_w, int row_scale, int64_t N,
                         int64_t K, int g, int io_f16, uint16_t *wu)
{
    if (!is_pow2(g) || N < 1 || K < 1 || (K % g) != 0 || wq == NULL || s_w == NULL ||
        wu == NULL)
        return -1;
    float *row = (float *)malloc((size_t)K * sizeof(float));
    if (!row) return -3;
    float c = oracle_rot_scale(g);
    for (int64_t n = 0; n < N; ++n) {
        float s = s_w[row_scale ? n : 0];
        for (int64_t k = 0; k < K; ++k) row[k] = s * (float)wq[n * K + k];
        for (int64_t b = 0; b < K; b += g) rotate_block(row + b, g, c);
        for (int64_t k = 0; k < K; ++k) wu[n * K + k] = f32_to_io(row[k], io_f16);
    }
    free(row);
    return 0;
}

/* y[r][n] = rnd(sum_k x[rows[r]][k] * wu[n][k] + bias[n]).  Each product of two
 * bf16 (8-bit significand) or fp16 (11-bit) values is exact in fp64; the sum
 * runs in fp64 in ascending k and is then rounded to fp32 and to the io
 * format.  exact (nullable, fp64 [R, N]) receives the fp64 sum with the bias;
 * mag (nullable, fp64 [R, N]) receives sum_k |x * wu| + |bias|, the scale of
 * the rounding error of any fp32 evaluation of the same sum. */
int oracle_default_rows(const uint16_t *x, int io_f16, int64_t M, int64_t K,
                        const int64_t *rows, int64_t R, const uint16_t *wu, int64_t N,
                        const uint16_t *bias, uint16_t *y, double *exact, double *mag)
{
    if (M < 1 || K < 1 || N < 1 || R < 0 || x == NULL || wu == NULL || y == NULL ||
        (R > 0 && rows == NULL))
        return -1;
    for (int64_t r = 0; r < R; ++r)
        if (rows[r] < 0 || rows[r] >= M) return -1;
    double *xr = (double *)malloc((size_t)(R > 0 ? R : 1) * (size_t)K * sizeof(double));
    double *wr = (double *)malloc((size_t)K * sizeof(double));
    if (!xr || !wr) { free(xr); free(wr); return -3; }
    for (int64_t r = 0; r < R; ++r)
        for (int64_t k = 0; k < K; ++k) xr[r * K + k] = io_to_f32(x[rows[r] * K + k], io_f16);
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) wr[k] = io_to_f32(wu[n * K + k], io_f16);
        double b = bias ? (double)io_to_f32(bias[n], io_f16) : 0.0;
        for (int64_t r = 0; r < R; ++r) {
            double sum = 0.0, abs_sum = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double t = xr[r * K + k] * wr[k];
                sum += t;
                abs_sum += fabs(t);
            }
            sum += b;
            abs_sum += fabs(b);
            y[r * N + n] = f32_to_io((float)sum, io_f16);
            if (exact) exact[r * N + n] = sum;
            if (mag) mag[r * N + n] = abs_sum;
        }
    }
    free(xr); free(wr);
    return 0;
}
