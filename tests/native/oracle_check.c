/* The C oracle (oracle/kda_oracle.c) under AddressSanitizer and UndefinedBehaviorSanitizer, linked
 * into this driver. Built and run by tests/test_host_sanitizers.py (host only). Covers its argument
 * checks, the row-selection and checkpoint outputs, a ragged column block (dv not a multiple of 16),
 * T = 0, and two closed forms of the recurrence that the pages fix: with alpha = 1 and beta = 0 the
 * state never changes (S_T = S0, o_t = S0^T q_t); with beta = 1, alpha = 1 and a unit key the state
 * after the write recalls the written value (S_t^T k_t = v_t). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int kda_oracle_fwd(int64_t BH, int64_t T, int64_t dk, int64_t dv, const float* q, const float* k, const float* v,
                   const float* log_alpha, const float* beta, const float* S0, const int64_t* rows, int64_t nrows,
                   double* o, double* S_T, int64_t ckpt_every, double* ckpt, int nthreads);

#define CHECK(c) do { if (!(c)) { fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #c); return 1; } } while (0)

static float frand(unsigned* s) { *s = *s * 1103515245u + 12345u; return (float)((*s >> 8) & 0xffff) / 65536.0f - 0.5f; }

int main(void) {
    const int64_t BH = 3, T = 37, dk = 8, dv = 20;   /* dv: one full and one ragged 16-column block */
    float *q = malloc(sizeof(float) * BH * T * dk), *k = malloc(sizeof(float) * BH * T * dk);
    float *la = malloc(sizeof(float) * BH * T * dk), *v = malloc(sizeof(float) * BH * T * dv);
    float *beta = malloc(sizeof(float) * BH * T), *S0 = malloc(sizeof(float) * BH * dk * dv);
    double *o = malloc(sizeof(double) * BH * T * dv), *ST = malloc(sizeof(double) * BH * dk * dv);
    double *ck = malloc(sizeof(double) * BH * (T / 8) * dk * dv), *osel = malloc(sizeof(double) * BH * 3 * dv);
    unsigned s = 7;
    for (int64_t i = 0; i < BH * T * dk; ++i) { q[i] = frand(&s); k[i] = frand(&s); la[i] = 0.f; }
    for (int64_t i = 0; i < BH * T * dv; ++i) v[i] = frand(&s);
    for (int64_t i = 0; i < BH * dk * dv; ++i) S0[i] = frand(&s);
    for (int64_t i = 0; i < BH * T; ++i) beta[i] = 0.f;
    /* argument checks */
    CHECK(kda_oracle_fwd(-1, T, dk, dv, q, k, v, la, beta, S0, NULL, 0, o, ST, 0, NULL, 2) == -1);
    CHECK(kda_oracle_fwd(BH, T, 0, dv, q, k, v, la, beta, S0, NULL, 0, o, ST, 0, NULL, 2) == -1);
    int64_t bad_rows[2] = {5, 5};
    CHECK(kda_oracle_fwd(BH, T, dk, dv, q, k, v, la, beta, S0, bad_rows, 2, osel, ST, 0, NULL, 2) == -1);
    /* alpha = 1, beta = 0: S_T = S0 exactly, o_t = S0^T q_t */
    CHECK(kda_oracle_fwd(BH, T, dk, dv, q, k, v, la, beta, S0, NULL, 0, o, ST, 8, ck, 2) == 0);
    for (int64_t i = 0; i < BH * dk * dv; ++i) CHECK(ST[i] == (double)S0[i]);
    for (int64_t b = 0; b < BH; ++b)   /* every checkpoint of lane b is its S0 */
        for (int64_t j = 0; j < T / 8; ++j)
            for (int64_t i = 0; i < dk * dv; ++i) CHECK(ck[(b * (T / 8) + j) * dk * dv + i] == (double)S0[b * dk * dv + i]);
    for (int64_t b = 0; b < BH; ++b)
        for (int64_t t = 0; t < T; ++t)
            for (int64_t j = 0; j < dv; ++j) {
                double r = 0.0;
                for (int64_t c = 0; c < dk; ++c) r += (double)q[(b * T + t) * dk + c] * (double)S0[(b * dk + c) * dv + j];
                CHECK(fabs(o[(b * T + t) * dv + j] - r) <= 1e-12);
            }
    /* selected rows equal the same rows of the full output */
    int64_t rows[3] = {0, 17, 36};
    CHECK(kda_oracle_fwd(BH, T, dk, dv, q, k, v, la, beta, S0, rows, 3, osel, ST, 0, NULL, 2) == 0);
    for (int64_t b = 0; b < BH; ++b)
        for (int64_t r = 0; r < 3; ++r)
            for (int64_t j = 0; j < dv; ++j) CHECK(osel[(b * 3 + r) * dv + j] == o[(b * T + rows[r]) * dv + j]);
    /* beta = 1, alpha = 1, unit keys e_c: o_t = S_t^T k_t with q_t = k_t recalls v_t */
    for (int64_t b = 0; b < BH; ++b)
        for (int64_t t = 0; t < T; ++t) {
            for (int64_t c = 0; c < dk; ++c) k[(b * T + t) * dk + c] = q[(b * T + t) * dk + c] = (c == (t * 3 + b) % dk) ? 1.f : 0.f;
            beta[b * T + t] = 1.f;
        }
    CHECK(kda_oracle_fwd(BH, T, dk, dv, q, k, v, la, beta, S0, NULL, 0, o, ST, 0, NULL, 3) == 0);
    for (int64_t i = 0; i < BH * T * dv; ++i) CHECK(fabs(o[i] - (double)v[i]) <= 1e-12);
    /* T = 0: S_T = S0, nothing else read */
    CHECK(kda_oracle_fwd(BH, 0, dk, dv, NULL, NULL, NULL, NULL, NULL, S0, NULL, 0, NULL, ST, 0, NULL, 1) == 0);
    for (int64_t i = 0; i < BH * dk * dv; ++i) CHECK(ST[i] == (double)S0[i]);
    free(q); free(k); free(la); free(v); free(beta); free(S0); free(o); free(ST); free(ck); free(osel);
    printf("oracle check: ok\n");
    return 0;
}
