/*
 * Oracle for the Kimi Delta Attention (KDA) recurrence: plain fp64 C, token by token.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path links, loads or calls this file;
 * only the test suite, the smoke check and the benchmark's CPU-baseline leg do.
 *
 * Source of the arithmetic: the Kimi K3 reading notes (liuzhao09.github.io/papers/kimi-k3.html),
 * section 2.2 "Hybrid KDA-MLA and Block AttnRes", the state recurrence equation. Per head the
 * state S is d_k x d_v (rows = key channels). For token t:
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,   o_t = S_t^T q_t,
 * with alpha_t = exp(log_alpha_t) per key channel. Expanding the product gives the three steps
 * used below, in this order:
 *     decay:   S <- Diag(alpha_t) S                      (each key channel row scaled)
 *     write:   S <- S + beta_t k_t (v_t - S^T k_t)^T     (prediction read from the decayed state)
 *     read:    o_t = S^T q_t                              (after the write: token t sees itself)
 *
 * Inputs are fp32 arrays (a bf16 or fp32 value widens to fp32 exactly); every operation runs in
 * fp64. Layouts: q,k,log_alpha [BH][T][dk]; v [BH][T][dv]; beta [BH][T]; S0 [BH][dk][dv]
 * (NULL = zero state); o [BH][nrows][dv]; S_T [BH][dk][dv]; checkpoints [BH][T/E][dk][dv].
 * Columns of the value dimension evolve independently (column j of S and o only ever meets
 * column j of v), so the work is split over (lane, column block) with identical arithmetic.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define COLS_PER_TASK 16

static int run_task(int64_t T, int64_t dk, int64_t dv, int64_t j0, int64_t j1,
                    const float* q, const float* k, const float* v, const float* la,
                    const float* beta, const float* S0, const int64_t* rows, int64_t nrows,
                    double* o, double* ST, int64_t ckpt_every, double* ckpt)
{
    const int64_t w = j1 - j0;
    double* S = (double*)malloc(sizeof(double) * (size_t)(dk * w));
    double* r = (double*)malloc(sizeof(double) * (size_t)w);
    double* a = (double*)malloc(sizeof(double) * (size_t)dk);
    if (!S || !r || !a) { free(S); free(r); free(a); return -1; }
    for (int64_t c = 0; c < dk; ++c)
        for (int64_t j = 0; j < w; ++j)
            S[c * w + j] = S0 ? (double)S0[c * dv + j0 + j] : 0.0;
    int64_t next = 0; /* index into rows[] of the next token whose output is stored */
    for (int64_t t = 0; t < T; ++t) {
        const float* kt = k + t * dk;
        const float* qt = q + t * dk;
        const float* vt = v + t * dv;
        const double b = (double)beta[t];
        for (int64_t c = 0; c < dk; ++c) a[c] = exp((double)la[t * dk + c]);
        /* decay */
        for (int64_t c = 0; c < dk; ++c)
            for (int64_t j = 0; j < w; ++j) S[c * w + j] *= a[c];
        /* predict from the decayed state: r = S^T k */
        for (int64_t j = 0; j < w; ++j) r[j] = 0.0;
        for (int64_t c = 0; c < dk; ++c) {
            const double kc = (double)kt[c];
            for (int64_t j = 0; j < w; ++j) r[j] += kc * S[c * w + j];
        }
        /* write the correction along k */
        for (int64_t c = 0; c < dk; ++c) {
            const double bk = b * (double)kt[c];
            for (int64_t j = 0; j < w; ++j) S[c * w + j] += bk * ((double)vt[j0 + j] - r[j]);
        }
        /* read */
        int store = 0;
        int64_t orow = t;
        if (!rows) store = 1;
        else if (next < nrows && rows[next] == t) { store = 1; orow = next; ++next; }
        if (store && o) {
            for (int64_t j = 0; j < w; ++j) r[j] = 0.0;
            for (int64_t c = 0; c < dk; ++c) {
                const double qc = (double)qt[c];
                for (int64_t j = 0; j < w; ++j) r[j] += qc * S[c * w + j];
            }
            for (int64_t j = 0; j < w; ++j) o[orow * dv + j0 + j] = r[j];
        }
        /* checkpoint: the state after tokens 0..t when t + 1 is a multiple of ckpt_every */
        if (ckpt && ckpt_every > 0 && (t + 1) % ckpt_every == 0) {
            double* dst = ckpt + ((t + 1) / ckpt_every - 1) * dk * dv;
            for (int64_t c = 0; c < dk; ++c)
                for (int64_t j = 0; j < w; ++j) dst[c * dv + j0 + j] = S[c * w + j];
        }
    }
    if (ST)
        for (int64_t c = 0; c < dk; ++c)
            for (int64_t j = 0; j < w; ++j) ST[c * dv + j0 + j] = S[c * w + j];
    free(S); free(r); free(a);
    return 0;
}

/* Returns 0 on success, -1 on bad arguments or allocation failure. `rows` (sorted, strictly
 * increasing, each in [0,T)) selects which tokens' outputs are stored; NULL stores all T.
 * With ckpt_every = E > 0 and ckpt != NULL, ckpt [BH][T/E][dk][dv] receives the state after the
 * first j*E tokens, j = 1 .. T/E (the prefix-cache checkpoints of section 2.5 / Figure 12). */
int kda_oracle_fwd(int64_t BH, int64_t T, int64_t dk, int64_t dv,
                   const float* q, const float* k, const float* v, const float* log_alpha,
                   const float* beta, const float* S0, const int64_t* rows, int64_t nrows,
                   double* o, double* S_T, int64_t ckpt_every, double* ckpt, int nthreads)
{
    if (BH < 0 || T < 0 || dk <= 0 || dv <= 0 || ckpt_every < 0) return -1;
    if (T > 0 && (!q || !k || !v || !log_alpha || !beta)) return -1;
    if (rows) {
        for (int64_t i = 0; i < nrows; ++i)
            if (rows[i] < 0 || rows[i] >= T || (i > 0 && rows[i] <= rows[i - 1])) return -1;
    }
    const int64_t nblk = (dv + COLS_PER_TASK - 1) / COLS_PER_TASK;
    const int64_t ntask = BH * nblk;
    const int64_t orows = rows ? nrows : T;
    const int64_t nck = ckpt_every > 0 ? T / ckpt_every : 0;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1) reduction(| : failed)
    for (int64_t task = 0; task < ntask; ++task) {
        const int64_t lane = task / nblk, blk = task % nblk;
        const int64_t j0 = blk * COLS_PER_TASK;
        const int64_t j1 = (j0 + COLS_PER_TASK < dv) ? j0 + COLS_PER_TASK : dv;
        const int64_t xo = lane * T * dk, vo = lane * T * dv;
        failed |= run_task(T, dk, dv, j0, j1, q + xo, k + xo, v + vo, log_alpha + xo, beta + lane * T,
                           S0 ? S0 + lane * dk * dv : NULL, rows, nrows,
                           o ? o + lane * orows * dv : NULL, S_T ? S_T + lane * dk * dv : NULL,
                           ckpt_every, ckpt ? ckpt + lane * nck * dk * dv : NULL) != 0;
    }
    return failed ? -1 : 0;
}
