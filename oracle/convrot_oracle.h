/*
 * convrot_oracle.h -- CPU oracle for the INT8 ConvRot linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This is a plain, slow, single-threaded C99
 * restatement of what the layer computes.  Only the test-suite, the smoke
 * check and the CPU-baseline leg of the benchmark may load it.  It shares no
 * code, header, table or constant with the HIP library.
 *
 * Method (page "int8 Compute", InvokeAI docs, opening section): a ConvRot
 * layer rotates its activation, codes it as int8 with one scale per token,
 * and multiplies those codes with the weight's int8 codes, which carry one
 * scale for the whole tensor.  The rotation works in groups (same page, "What stays on the default
 * path": published builds use groups of 256) and is the same orthogonal block
 * rotation on both operands, so x.W^T = (xR).(WR)^T (page "Explanation of INT8
 * ConvRot", section "What is INT8 ConvRot?": rotation applied group by group,
 * block after block, like a convolution).
 *
 * Readings where the pages are silent (each one is listed with its reason in
 * the design notes of the repository):
 *   R  = blockdiag(H_g / sqrt(g)), H_g the Sylvester Hadamard matrix,
 *        H[i][j] = (-1)^popcount(i & j).
 *   rotation in fp32: radix-2 butterfly with ascending half-span h = 1,2,..,g/2,
 *        pair (a,b) -> (a+b, a-b), then one multiply by c_g, the float nearest
 *        to 1/sqrt(g).
 *   scales: s = absmax / 127 (fp32, IEEE division); codes q = clamp(rne(v/s),
 *        -127, 127); an all-zero row/tensor gives s = 0 and codes 0.
 *   epilogue: y = bf16_rne(fmaf((float)acc, s_x[m]*s_w, bias[n])).
 *   variants: fp16 in place of bf16 for x, bias and y (IEEE binary16, RNE,
 *        overflow to infinity); one weight scale per output channel, computed
 *        like a token's (alpha = s_x[m] * s_w[n]).
 *   default path: the weight unpacked (dequantized in fp32, rotated back by
 *        R = R^-1, rounded to bf16/fp16), times the unrotated activation.
 *
 * All arrays are row-major and contiguous.  bf16 values travel as their raw
 * uint16 bit patterns.  Functions return 0 on success and a negative value on
 * a bad argument (nothing is written in that case).
 */
#ifndef CONVROT_ORACLE_H
#define CONVROT_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* float <-> bf16 bit conversions (widening is exact; narrowing is RNE). */
float    oracle_bf16_to_f32(uint16_t b);
uint16_t oracle_f32_to_bf16(float f);

/* float <-> IEEE binary16 bit conversions (widening exact; narrowing RNE,
 * overflow to infinity, gradual underflow). */
float    oracle_f16_to_f32(uint16_t h);
uint16_t oracle_f32_to_f16(float f);

/* c_g: the float nearest to 1/sqrt(g). */
float oracle_rot_scale(int g);

/* O1: the g x g Sylvester Hadamard matrix as +-1 integers.  g a power of 2. */
int oracle_hadamard(int g, int32_t *H);

/* O2: rotate every length-g block of each row of v (rows x K, fp32) in place.
 * g is a power of two (g = 1 is the identity rotation) and divides K. */
int oracle_rotate_rows(float *v, int64_t rows, int64_t K, int g);

/* O3: tensorwise weight quantization.  w: fp32 [N, K] (not modified).
 * wq: int8 [N, K]; *s_w: the single scale.  w_rot (nullable): fp32 [N, K]
 * receives the rotated weight. */
int oracle_quant_weight(const float *w, int64_t N, int64_t K, int g,
                        int8_t *wq, float *s_w, float *w_rot);

/* Row-wise variant of O3 (page "Explanation of INT8 ConvRot", format table:
 * row-wise scaling): s_w: fp32 [N], one scale per output channel. */
int oracle_quant_weight_rows(const float *w, int64_t N, int64_t K, int g,
                             int8_t *wq, float *s_w, float *w_rot);

/* O4: per-token activation quantization.  x: bf16 bits [M, K].
 * q: int8 [M, K]; s: fp32 [M].  x_rot (nullable): fp32 [M, K]. */
int oracle_quant_act(const uint16_t *x, int64_t M, int64_t K, int g,
                     int8_t *q, float *s, float *x_rot);

/* O4 with fp16 input bits when io_f16 != 0 (page "int8 Compute", "What
 * stays on the default path": compute is offered in BF16 or FP16). */
int oracle_quant_act_ex(const uint16_t *x, int io_f16, int64_t M, int64_t K, int g,
                        int8_t *q, float *s, float *x_rot);

/* O5: acc[m][n] = sum_k a[m][k] * b[n][k], accumulated in int64.
 * Returns -2 if a result does not fit int32. */
int oracle_gemm_i32(const int8_t *a, const int8_t *b, int64_t M, int64_t N,
                    int64_t K, int32_t *acc);

/* O6: y[m][n] = bf16_rne(fmaf((float)acc[m][n], s_x[m]*s_w, bias[n])).
 * bias: bf16 bits [N] or NULL (then +0.0f). */
int oracle_epilogue(const int32_t *acc, const float *s_x, float s_w,
                    const uint16_t *bias, int64_t M, int64_t N, uint16_t *y);

/* O6 variants: y[m][n] = rnd(fmaf((float)acc, s_x[m] * s_w[row_scale ? n : 0],
 * bias[n])), rnd = bf16 (io_f16 = 0) or fp16 (io_f16 = 1) RNE; bias in the
 * same format, or NULL. */
int oracle_epilogue_ex(const int32_t *acc, const float *s_x, const float *s_w, int row_scale,
                       const uint16_t *bias, int io_f16, int64_t M, int64_t N, uint16_t *y);

/* O4 -> O5 -> O6 for the rows of x listed in rows[0..R) (R rows, each index
 * in [0, M)).  Output y: bf16 bits [R, N]; q_rows: int8 [R, K] and s_rows:
 * fp32 [R] (both nullable) receive the rows' codes and scales.  wq/s_w come
 * from oracle_quant_weight.  This is the whole layer, evaluated on a subset
 * of tokens, which is exact because every token is quantized on its own. */
int oracle_linear_rows(const uint16_t *x, int64_t M, int64_t K,
                       const int64_t *rows, int64_t R,
                       const int8_t *wq, float s_w, int64_t N, int g,
                       const uint16_t *bias, uint16_t *y,
                       int8_t *q_rows, float *s_rows);

/* oracle_linear_rows with the variants: x, bias and y in bf16 or fp16 bits
 * (io_f16), s_w with one or N entries (row_scale). */
int oracle_linear_rows_ex(const uint16_t *x, int io_f16, int64_t M, int64_t K,
                          const int64_t *rows, int64_t R,
                          const int8_t *wq, const float *s_w, int row_scale, int64_t N, int g,
                          const uint16_t *bias, uint16_t *y,
                          int8_t *q_rows, float *s_rows);

/* Default path (page "int8 Compute", InvokeAI docs, "When something goes
 * wrong": the first result of the int8 layer is checked against it; "What
 * stays on the default path": such layers keep unpacking their weights).
 * Unpack: wu[n] = rnd(O2(s_w[row_scale ? n : 0] * wq[n])), the dequantized
 * row rotated back (R^-1 = R), rnd = bf16 or fp16 RNE.  wu: io bits [N, K]. */
int oracle_unpack_weight(const int8_t *wq, const float *s_w, int row_scale, int64_t N,
                         int64_t K, int g, int io_f16, uint16_t *wu);

/* Default-path layer on the rows listed: y[r][n] = rnd(sum_k x[rows[r]][k] *
 * wu[n][k] + bias[n]), the sum in fp64 (exact products), then fp32, then io.
 * exact / mag (nullable, fp64 [R, N]): the fp64 sum with the bias, and
 * sum_k |x * wu| + |bias|. */
int oracle_default_rows(const uint16_t *x, int io_f16, int64_t M, int64_t K,
                        const int64_t *rows, int64_t R, const uint16_t *wu, int64_t N,
                        const uint16_t *bias, uint16_t *y, double *exact, double *mag);

#ifdef __cplusplus
}
#endif

#endif /* CONVROT_ORACLE_H */
