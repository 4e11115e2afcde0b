/*
 * Runs the float64 oracle (oracle/gdn_oracle.c) on small seeded inputs,
 * built with AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_oracle_sanitized.py: every entry point, both gate kinds, one
 * and several slots, shared q/k heads in both orders, a final state,
 * rollback with valid and invalid indices, and the chunked form with a
 * ragged last chunk.  Exit status 0 when every call returns as documented
 * and the chunked form agrees with the token loop.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_gdn_forward(int B, int T, int H, int Hqk, int tiled, int dk, int dv, int K, int kda,
                       const double* q, const double* k, const double* v, const double* g,
                       const double* beta, double* state, double* final_state, double* o);
int oracle_gdn_rollback(int B, int H, int K, int dk, int dv, const int32_t* accepted, double* state);
int oracle_gdn_chunked(int B, int T, int H, int dk, int dv, int C, int kda, const double* q,
                       const double* k, const double* v, const double* g, const double* beta,
                       double* state, double* o);

static uint64_t rng = 88172645463325252ull;
static double uni(void) { /* xorshift64, uniform in [0, 1) */
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (double)(rng >> 11) * (1.0 / 9007199254740992.0);
}
static double* filled(size_t n, double lo, double hi) {
    double* p = (double*)malloc(sizeof(double) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i) p[i] = lo + (hi - lo) * uni();
    return p;
}

static int run(int B, int T, int H, int Hqk, int tiled, int dk, int dv, int K, int kda) {
    const size_t nq = (size_t)B * T * Hqk * dk, nv = (size_t)B * T * H * dv;
    const size_t ng = (size_t)B * T * H * (kda ? dk : 1), nb = (size_t)B * T * H;
    const size_t tile = (size_t)dk * dv, ns = (size_t)B * H * K * tile;
    double *q = filled(nq, -0.3, 0.3), *k = filled(nq, -0.3, 0.3), *v = filled(nv, -1, 1);
    double *g = filled(ng, -2, 0), *beta = filled(nb, 0, 1), *st = filled(ns, -0.1, 0.1);
    double *fin = filled((size_t)B * H * tile, 0, 0), *o = filled(nv, 0, 0);
    int err = 0;
    if (oracle_gdn_forward(B, T, H, Hqk, tiled, dk, dv, K, kda, q, k, v, g, beta, st, fin, o) != 0) err = 1;
    int32_t* acc = (int32_t*)malloc(sizeof(int32_t) * (B ? B : 1));
    for (int b = 0; b < B; ++b) acc[b] = (b % 3 == 2) ? K + b : b % K; /* some out of range */
    int invalid = 0;
    for (int b = 0; b < B; ++b) invalid += (acc[b] < 0 || acc[b] >= K);
    if (oracle_gdn_rollback(B, H, K, dk, dv, acc, st) != invalid) err = 1;
    if (Hqk == H && K == 1) {
        /* the chunked form against the token loop, from the same start state */
        double *s1 = filled((size_t)B * H * tile, -0.1, 0.1), *s2 = (double*)malloc(sizeof(double) * B * H * tile);
        for (size_t i = 0; i < (size_t)B * H * tile; ++i) s2[i] = s1[i];
        double* o2 = filled(nv, 0, 0);
        if (oracle_gdn_forward(B, T, H, H, 0, dk, dv, 1, kda, q, k, v, g, beta, s1, NULL, o) != 0) err = 1;
        if (oracle_gdn_chunked(B, T, H, dk, dv, 8, kda, q, k, v, g, beta, s2, o2) != 0) err = 1;
        double d = 0, m = 0;
        for (size_t i = 0; i < nv; ++i) { d = fmax(d, fabs(o[i] - o2[i])); m = fmax(m, fabs(o[i])); }
        for (size_t i = 0; i < (size_t)B * H * tile; ++i) d = fmax(d, fabs(s1[i] - s2[i]));
        if (!(d <= 1e-9 * (m > 1 ? m : 1))) { fprintf(stderr, "chunked vs token loop: %g\n", d); err = 1; }
        free(s1); free(s2); free(o2);
    }
    /* bad arguments are refused */
    if (oracle_gdn_forward(B, T, H, 0, 0, dk, dv, K, kda, q, k, v, g, beta, st, NULL, o) != -1) err = 1;
    if (oracle_gdn_chunked(B, T, H, dk, dv, 0, kda, q, k, v, g, beta, st, o) != -1) err = 1;
    free(q); free(k); free(v); free(g); free(beta); free(st); free(fin); free(o); free(acc);
    return err;
}

int main(void) {
    int err = 0;
    /* B, T, H, Hqk, tiled, dk, dv, K, kda */
    err |= run(2, 5, 2, 2, 0, 8, 8, 1, 0);
    err |= run(3, 19, 2, 2, 0, 8, 4, 1, 1);   /* ragged chunked tail (C = 8), KDA, dk != dv */
    err |= run(3, 6, 4, 2, 0, 4, 8, 4, 0);    /* shared q/k heads, grouped; snapshots */
    err |= run(2, 3, 4, 1, 1, 8, 8, 5, 1);    /* tiled, more slots than tokens */
    err |= run(1, 0, 2, 2, 0, 8, 8, 3, 0);    /* no token */
    err |= run(0, 4, 2, 2, 0, 8, 8, 1, 0);    /* no sequence */
    printf(err ? "FAIL\n" : "ok\n");
    return err;
}
