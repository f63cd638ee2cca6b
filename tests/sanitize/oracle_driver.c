/* oracle_driver.c -- runs every function of the CPU oracle on small inputs,
 * edge cases included (zero rows, a zero weight, one-column layers, the
 * identity group g = 1, fp16 specials, an accumulator overflow and refused
 * arguments), for a build under AddressSanitizer and
 * UndefinedBehaviorSanitizer.  It checks status codes only; the values are
 * pinned by the Python tests.  Exit status 0 and the line
 * "oracle_driver: N calls passed" mean every status matched. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/convrot_oracle.h"

static int checks = 0, failed = 0;

static void expect(int got, int want, const char *what)
{
    ++checks;
    if (got != want) {
        ++failed;
        printf("FAIL %s: %d, expected %d\n", what, got, want);
    }
}

static uint64_t rng_state = 0x1234567ULL;
static double uni(void)
{
    rng_state = rng_state * 6364136223846793005ULL + 1442695040888963407ULL;
    return (double)(rng_state >> 11) * (1.0 / 9007199254740992.0);
}

int main(void)
{
    enum { M = 5, K = 512, N = 7 };
    float *w = malloc(sizeof(float) * N * K), *wrot = malloc(sizeof(float) * N * K);
    float *xf = malloc(sizeof(float) * M * K), *xrot = malloc(sizeof(float) * M * K);
    uint16_t *xb = malloc(2 * M * K), *xh = malloc(2 * M * K), *bias = malloc(2 * N);
    int8_t *wq = malloc(N * K), *q = malloc(M * K), *qr = malloc(M * K);
    float s_w, s_wr[N], s_x[M], s_r[M];
    int32_t *acc = malloc(sizeof(int32_t) * M * N);
    uint16_t *y = malloc(2 * M * N), *wu = malloc(2 * N * K);
    double *exact = malloc(sizeof(double) * M * N), *mag = malloc(sizeof(double) * M * N);
    int32_t *H = malloc(sizeof(int32_t) * 256 * 256);
    int64_t rows[3] = {0, 2, M - 1};

    for (int i = 0; i < N * K; ++i) w[i] = (float)((uni() - 0.5) * 0.08);
    for (int i = 0; i < M * K; ++i) xf[i] = (float)((uni() - 0.5) * 6.0);
    memset(xf, 0, sizeof(float) * K);                       /* a zero token */
    for (int i = 0; i < M * K; ++i) { xb[i] = oracle_f32_to_bf16(xf[i]); xh[i] = oracle_f32_to_f16(xf[i]); }
    for (int i = 0; i < N; ++i) bias[i] = oracle_f32_to_bf16((float)(uni() - 0.5) * 0.02f);

    /* conversions and constants, specials included */
    const float specials[] = {0.0f, -0.0f, 1.0f, 65504.0f, 65520.0f, 1e-8f, 5.96e-8f, INFINITY, -INFINITY, NAN};
    for (unsigned i = 0; i < sizeof specials / sizeof specials[0]; ++i) {
        (void)oracle_bf16_to_f32(oracle_f32_to_bf16(specials[i]));
        (void)oracle_f16_to_f32(oracle_f32_to_f16(specials[i]));
    }
    for (uint32_t b = 0; b < 65536; b += 7) { (void)oracle_bf16_to_f32((uint16_t)b); (void)oracle_f16_to_f32((uint16_t)b); }
    (void)oracle_rot_scale(128); (void)oracle_rot_scale(256); (void)oracle_rot_scale(1);
    expect(oracle_hadamard(256, H), 0, "hadamard 256");
    expect(oracle_hadamard(1, H), 0, "hadamard 1");
    expect(oracle_hadamard(12, H), -1, "hadamard 12");

    /* O2 */
    memcpy(xrot, xf, sizeof(float) * M * K);
    expect(oracle_rotate_rows(xrot, M, K, 128), 0, "rotate g128");
    expect(oracle_rotate_rows(xrot, M, K, 256), 0, "rotate g256");
    expect(oracle_rotate_rows(xrot, M, K, 1), 0, "rotate g1");
    expect(oracle_rotate_rows(xrot, M, K, 384), -1, "rotate g384");

    /* O3, O4 */
    expect(oracle_quant_weight(w, N, K, 128, wq, &s_w, wrot), 0, "quant_weight");
    expect(oracle_quant_weight(w, N, K, 256, wq, &s_w, NULL), 0, "quant_weight no rot");
    expect(oracle_quant_weight_rows(w, N, K, 128, wq, s_wr, wrot), 0, "quant_weight_rows");
    expect(oracle_quant_act(xb, M, K, 128, q, s_x, xrot), 0, "quant_act");
    expect(oracle_quant_act(xb, M, K, 1, q, s_x, NULL), 0, "quant_act g1");
    expect(oracle_quant_act_ex(xh, 1, M, K, 256, q, s_x, NULL), 0, "quant_act fp16");
    expect(oracle_quant_act(xb, M, 500, 128, q, s_x, NULL), -1, "quant_act K % g");
    {
        float zero[2 * 128] = {0};
        int8_t zq[2 * 128];
        float zs;
        expect(oracle_quant_weight(zero, 2, 128, 128, zq, &zs, NULL), 0, "quant_weight zero");
    }

    /* O5, O6 */
    expect(oracle_quant_weight(w, N, K, 128, wq, &s_w, NULL), 0, "quant_weight again");
    expect(oracle_quant_act(xb, M, K, 128, q, s_x, NULL), 0, "quant_act again");
    expect(oracle_gemm_i32(q, wq, M, N, K, acc), 0, "gemm");
    expect(oracle_epilogue(acc, s_x, s_w, bias, M, N, y), 0, "epilogue");
    expect(oracle_epilogue(acc, s_x, s_w, NULL, M, N, y), 0, "epilogue no bias");
    expect(oracle_epilogue_ex(acc, s_x, s_wr, 1, bias, 1, M, N, y), 0, "epilogue row fp16");
    expect(oracle_epilogue_ex(acc, s_x, &s_w, 0, NULL, 0, M, N, y), 0, "epilogue_ex tensor bf16");
    {
        /* 127 * 127 * K past 2^31: reported, not wrapped */
        const int64_t KB = 140000;
        int8_t *big = malloc(KB);
        int32_t one;
        memset(big, 127, KB);
        expect(oracle_gemm_i32(big, big, 1, 1, KB, &one), -2, "gemm overflow");
        free(big);
    }

    /* whole layer on rows */
    expect(oracle_linear_rows(xb, M, K, rows, 3, wq, s_w, N, 128, bias, y, qr, s_r), 0, "linear_rows");
    expect(oracle_linear_rows(xb, M, K, rows, 0, wq, s_w, N, 128, NULL, y, NULL, NULL), 0, "linear_rows R 0");
    expect(oracle_linear_rows_ex(xh, 1, M, K, rows, 3, wq, s_wr, 1, N, 128, bias, y, qr, s_r), 0,
           "linear_rows_ex");
    {
        int64_t bad[1] = {M};
        expect(oracle_linear_rows(xb, M, K, bad, 1, wq, s_w, N, 128, bias, y, NULL, NULL), -1,
               "linear_rows row out of range");
    }

    /* default path */
    expect(oracle_unpack_weight(wq, &s_w, 0, N, K, 128, 0, wu), 0, "unpack bf16");
    expect(oracle_unpack_weight(wq, s_wr, 1, N, K, 256, 1, wu), 0, "unpack fp16 rows");
    expect(oracle_default_rows(xb, 0, M, K, rows, 3, wu, N, bias, y, exact, mag), 0, "default_rows");
    expect(oracle_default_rows(xh, 1, M, K, rows, 3, wu, N, NULL, y, NULL, NULL), 0, "default_rows fp16");

    free(w); free(wrot); free(xf); free(xrot); free(xb); free(xh); free(bias); free(wq); free(q); free(qr);
    free(acc); free(y); free(wu); free(exact); free(mag); free(H);
    if (failed) {
        printf("oracle_driver: %d of %d calls failed\n", failed, checks);
        return 1;
    }
    printf("oracle_driver: %d calls passed\n", checks);
    return 0;
}
