/*
 * Sanitizer driver for the C oracle (test infrastructure).  Built with
 * -fsanitize=address,undefined and run by tests/test_sanitizers.py: it calls
 * kda_oracle_forward on small problems of every decay mode, dtype and column
 * range, checks that the thread count and column slicing change nothing
 * (bitwise), that rejected arguments return -1, and exits 0.  Inputs come
 * from a fixed linear congruential sequence; no arithmetic of the method is
 * here.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kda_oracle.h"

static uint64_t g_state = 88172645463325252ull;
static double next_uniform(void) { /* in [-1, 1) */
    g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(g_state >> 11) / (double)(1ull << 52) - 1.0;
}

static uint16_t bf16_bits(float x) { /* round to nearest even */
    uint32_t u;
    memcpy(&u, &x, 4);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* n values in dtype (ORACLE_F32 or ORACLE_BF16); scale and offset applied */
static void* fill(size_t n, int dtype, double scale, double offset) {
    if (n == 0) n = 1;
    if (dtype == ORACLE_BF16) {
        uint16_t* p = (uint16_t*)malloc(n * 2);
        for (size_t i = 0; i < n; ++i) p[i] = bf16_bits((float)(offset + scale * next_uniform()));
        return p;
    }
    float* p = (float*)malloc(n * 4);
    for (size_t i = 0; i < n; ++i) p[i] = (float)(offset + scale * next_uniform());
    return p;
}

static int fails = 0;
#define CHECK(c)                                                              \
    do {                                                                      \
        if (!(c)) {                                                           \
            fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__);    \
            ++fails;                                                          \
        }                                                                     \
    } while (0)

static void run_case(int64_t B, int64_t H, int64_t L, int64_t dk, int64_t dv, int qd, int gd,
                     int mode, int with_s0) {
    const int64_t bh = B * H;
    void* q = fill((size_t)(bh * L * dk), qd, 0.3, 0.0);
    void* k = fill((size_t)(bh * L * dk), qd, 0.3, 0.0);
    void* v = fill((size_t)(bh * L * dv), qd, 1.0, 0.0);
    void* la = fill((size_t)(bh * L * (mode == ORACLE_ALPHA_CHANNEL ? dk : 1)), gd, 0.05, -0.06);
    void* beta = fill((size_t)(bh * L), gd, 0.4, 0.5);
    double* S0 = NULL;
    if (with_s0) {
        S0 = (double*)malloc((size_t)(bh * dk * dv) * 8);
        for (int64_t i = 0; i < bh * dk * dv; ++i) S0[i] = 0.02 * next_uniform();
    }
    const size_t no = (size_t)(bh * L * dv), ns = (size_t)(bh * dk * dv);
    double* o1 = (double*)malloc((no ? no : 1) * 8);
    double* s1 = (double*)malloc(ns * 8);
    double* o4 = (double*)malloc((no ? no : 1) * 8);
    double* s4 = (double*)malloc(ns * 8);
    CHECK(kda_oracle_forward(B, H, L, dk, dv, qd, gd, mode, q, k, v, la, beta, S0, 0, dv, 1, o1,
                             s1, 1) == 0);
    CHECK(kda_oracle_forward(B, H, L, dk, dv, qd, gd, mode, q, k, v, la, beta, S0, 0, dv, 1, o4,
                             s4, 4) == 0);
    CHECK(memcmp(o1, o4, no * 8) == 0);
    CHECK(memcmp(s1, s4, ns * 8) == 0);
    for (size_t i = 0; i < no; ++i) CHECK(isfinite(o1[i]));
    /* a column range alone equals those columns of the whole */
    const int64_t c0 = dv / 4, nc = dv / 2;
    double* oc = (double*)malloc(((size_t)(bh * L * nc) ? (size_t)(bh * L * nc) : 1) * 8);
    double* sc = (double*)malloc((size_t)(bh * dk * nc) * 8);
    CHECK(kda_oracle_forward(B, H, L, dk, dv, qd, gd, mode, q, k, v, la, beta, S0, c0, nc, 1, oc,
                             sc, 3) == 0);
    for (int64_t r = 0; r < bh * L; ++r)
        for (int64_t c = 0; c < nc; ++c) CHECK(oc[r * nc + c] == o1[r * dv + c0 + c]);
    for (int64_t r = 0; r < bh * dk; ++r)
        for (int64_t c = 0; c < nc; ++c) CHECK(sc[r * nc + c] == s1[r * dv + c0 + c]);
    /* the additive (no delta) mode and an o-less call run too */
    CHECK(kda_oracle_forward(B, H, L, dk, dv, qd, gd, mode, q, k, v, la, beta, S0, 0, dv, 0, NULL,
                             s4, 2) == 0);
    free(q), free(k), free(v), free(la), free(beta), free(S0);
    free(o1), free(s1), free(o4), free(s4), free(oc), free(sc);
}

int main(void) {
    const int modes[] = {ORACLE_ALPHA_NONE, ORACLE_ALPHA_HEAD, ORACLE_ALPHA_CHANNEL};
    const int dts[] = {ORACLE_F32, ORACLE_BF16};
    for (int m = 0; m < 3; ++m)
        for (int a = 0; a < 2; ++a)
            for (int b = 0; b < 2; ++b) {
                run_case(2, 2, 37, 16, 64, dts[a], dts[b], modes[m], (a + b) & 1);
                run_case(1, 3, 1, 32, 16, dts[a], dts[b], modes[m], 1);
            }
    run_case(1, 1, 0, 8, 8, ORACLE_F32, ORACLE_F32, ORACLE_ALPHA_CHANNEL, 1); /* L = 0 */
    /* rejected arguments */
    float x[64] = {0};
    double y[64];
    CHECK(kda_oracle_forward(1, 1, 1, 8, 8, 7, 0, 0, x, x, x, x, x, NULL, 0, 8, 1, y, y, 1) == -1);
    CHECK(kda_oracle_forward(1, 1, 1, 8, 8, 0, 0, 9, x, x, x, x, x, NULL, 0, 8, 1, y, y, 1) == -1);
    CHECK(kda_oracle_forward(1, 1, 1, 8, 8, 0, 0, 0, x, x, x, x, x, NULL, 4, 8, 1, y, y, 1) == -1);
    CHECK(kda_oracle_forward(-1, 1, 1, 8, 8, 0, 0, 0, x, x, x, x, x, NULL, 0, 8, 1, y, y, 1) == -1);
    if (fails) {
        fprintf(stderr, "%d checks failed\n", fails);
        return 1;
    }
    printf("oracle sanitizer driver: ok\n");
    return 0;
}
