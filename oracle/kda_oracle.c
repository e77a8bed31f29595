/*
 * kda_oracle.c -- plain fp64 CPU oracle of the KDA / gated delta rule.
 *
 * TEST INFRASTRUCTURE ONLY (see kda_oracle.h for what is computed and which
 * passages of the pages it follows).  Plain loops, no BLAS, no intrinsics.
 * Work is split over (b, h, column block) units that are exactly independent,
 * so the result is bitwise the same for any thread count.
 */
#include "kda_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

#define COL_BLOCK 32

typedef struct {
    int64_t B, H, L, dk, dv;
    int qkv_dtype, gate_dtype, alpha_mode;
    const void *q, *k, *v, *log_alpha, *beta;
    const double* S0;
    int64_t col0, ncols;
    int delta;
    double *o, *S_final;
    int64_t n_units, n_cblk;
    int64_t next; /* next unit to take, guarded by mu */
    pthread_mutex_t mu;
} job_t;

/* exact widening of one stored element (fp64 inputs are values already
 * preprocessed on the host in fp64) */
static double load(const void* base, int64_t idx, int dtype) {
    if (dtype == ORACLE_F64) return ((const double*)base)[idx];
    if (dtype == ORACLE_BF16) {
        uint16_t bits = ((const uint16_t*)base)[idx];
        uint32_t w = (uint32_t)bits << 16;
        float f;
        memcpy(&f, &w, sizeof f);
        return (double)f;
    }
    return (double)((const float*)base)[idx];
}

/* One (b, h, column block): the token recurrence over all L tokens. */
static void run_unit(const job_t* j, int64_t unit) {
    const int64_t bh = unit / j->n_cblk;
    const int64_t cb = unit % j->n_cblk;
    const int64_t c_lo = cb * COL_BLOCK;                   /* within the requested range */
    const int64_t c_hi = c_lo + COL_BLOCK < j->ncols ? c_lo + COL_BLOCK : j->ncols;
    const int64_t nc = c_hi - c_lo;
    const int64_t dk = j->dk, dv = j->dv, L = j->L;

    double* S = (double*)malloc(sizeof(double) * (size_t)(dk * nc));
    double* a = (double*)malloc(sizeof(double) * (size_t)dk);
    double* kt = (double*)malloc(sizeof(double) * (size_t)dk);
    double* qt = (double*)malloc(sizeof(double) * (size_t)dk);
    double* u = (double*)malloc(sizeof(double) * (size_t)nc);

    /* S <- S0 (columns col0 + c_lo .. col0 + c_hi) */
    for (int64_t i = 0; i < dk; ++i)
        for (int64_t c = 0; c < nc; ++c)
            S[i * nc + c] = j->S0 ? j->S0[(bh * dk + i) * dv + j->col0 + c_lo + c] : 0.0;

    for (int64_t t = 0; t < L; ++t) {
        const int64_t row = bh * L + t; /* token index into [B*H, L] */
        for (int64_t i = 0; i < dk; ++i) {
            kt[i] = load(j->k, row * dk + i, j->qkv_dtype);
            qt[i] = load(j->q, row * dk + i, j->qkv_dtype);
            if (j->alpha_mode == ORACLE_ALPHA_CHANNEL)
                a[i] = exp(load(j->log_alpha, row * dk + i, j->gate_dtype));
            else if (j->alpha_mode == ORACLE_ALPHA_HEAD)
                a[i] = exp(load(j->log_alpha, row, j->gate_dtype));
            else
                a[i] = 1.0;
        }
        const double bt = load(j->beta, row, j->gate_dtype);

        /* S~ = diag(a) S */
        for (int64_t i = 0; i < dk; ++i)
            for (int64_t c = 0; c < nc; ++c) S[i * nc + c] *= a[i];

        /* u = beta (v - k S~)   (delta rule)   or   u = beta v   (additive) */
        for (int64_t c = 0; c < nc; ++c) {
            double ks = 0.0;
            if (j->delta)
                for (int64_t i = 0; i < dk; ++i) ks += kt[i] * S[i * nc + c];
            const double vt = load(j->v, row * dv + j->col0 + c_lo + c, j->qkv_dtype);
            u[c] = bt * (vt - ks);
        }

        /* S = S~ + k^T u */
        for (int64_t i = 0; i < dk; ++i)
            for (int64_t c = 0; c < nc; ++c) S[i * nc + c] += kt[i] * u[c];

        /* o_t = q S */
        if (j->o) {
            for (int64_t c = 0; c < nc; ++c) {
                double acc = 0.0;
                for (int64_t i = 0; i < dk; ++i) acc += qt[i] * S[i * nc + c];
                j->o[row * j->ncols + c_lo + c] = acc;
            }
        }
    }

    if (j->S_final)
        for (int64_t i = 0; i < dk; ++i)
            for (int64_t c = 0; c < nc; ++c)
                j->S_final[(bh * dk + i) * j->ncols + c_lo + c] = S[i * nc + c];

    free(S);
    free(a);
    free(kt);
    free(qt);
    free(u);
}

static void* worker(void* arg) {
    job_t* j = (job_t*)arg;
    for (;;) {
        pthread_mutex_lock(&j->mu);
        const int64_t unit = j->next++;
        pthread_mutex_unlock(&j->mu);
        if (unit >= j->n_units) break;
        run_unit(j, unit);
    }
    return NULL;
}

int kda_oracle_forward(int64_t B, int64_t H, int64_t L, int64_t dk, int64_t dv,
                       int qkv_dtype, int gate_dtype, int alpha_mode,
                       const void* q, const void* k, const void* v,
                       const void* log_alpha, const void* beta,
                       const double* S0, int64_t col0, int64_t ncols, int delta,
                       double* o, double* S_final, int nthreads) {
    if (B < 0 || H < 0 || L < 0 || dk <= 0 || dv <= 0) return -1;
    if (col0 < 0 || ncols < 0 || col0 + ncols > dv) return -1;
    if (qkv_dtype < ORACLE_F32 || qkv_dtype > ORACLE_F64) return -1;
    if (gate_dtype < ORACLE_F32 || gate_dtype > ORACLE_F64) return -1;
    if (alpha_mode < ORACLE_ALPHA_NONE || alpha_mode > ORACLE_ALPHA_CHANNEL) return -1;
    if (L > 0 && (!q || !k || !v || !beta)) return -1;
    if (L > 0 && alpha_mode != ORACLE_ALPHA_NONE && !log_alpha) return -1;
    if (B * H == 0 || ncols == 0) return 0;

    job_t j;
    memset(&j, 0, sizeof j);
    j.B = B; j.H = H; j.L = L; j.dk = dk; j.dv = dv;
    j.qkv_dtype = qkv_dtype; j.gate_dtype = gate_dtype; j.alpha_mode = alpha_mode;
    j.q = q; j.k = k; j.v = v; j.log_alpha = log_alpha; j.beta = beta;
    j.S0 = S0; j.col0 = col0; j.ncols = ncols; j.delta = delta;
    j.o = o; j.S_final = S_final;
    j.n_cblk = (ncols + COL_BLOCK - 1) / COL_BLOCK;
    j.n_units = B * H * j.n_cblk;
    j.next = 0;
    pthread_mutex_init(&j.mu, NULL);

    int nt = nthreads > 0 ? nthreads : 1;
    if (nt > j.n_units) nt = (int)j.n_units;
    if (nt <= 1) {
        worker(&j);
    } else {
        pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nt);
        int started = 0;
        for (int i = 0; i < nt; ++i)
            if (pthread_create(&th[i], NULL, worker, &j) == 0) ++started;
        if (started == 0) worker(&j);
        for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
        free(th);
    }
    pthread_mutex_destroy(&j.mu);
    return 0;
}
