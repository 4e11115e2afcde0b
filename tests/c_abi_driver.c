/*
 * c_abi_driver.c -- the library used from plain C, the way a C or C++
 * engine would link it: gcc, the HIP runtime API and include/gdn.h, with no
 * hipcc, no C++ and no Python.  Test infrastructure: it links the float64
 * oracle (oracle/gdn_oracle.c) to check what the library computes.
 *
 * Cases (on one HIP stream the program creates, inputs copied from host
 * memory):
 *   1. a verification of 4 draft tokens with K = 4 state slots and a final
 *      state, 4 value heads sharing 2 q/k heads, d = 128, GDA gates, bf16
 *      q/k/v (gdn_forward_qk_broadcast) -- the partial-rollback slot
 *      semantics of the koboldcpp commit log (tag v1.113.1, bullet "metal:
 *      add GDN partial rollback") and the shared q/k heads of the llama.cpp
 *      commit log (tag b9752, bullet "models : avoid Q and K repeats when
 *      using fused GDA");
 *   2. the rollback to the accepted draft lengths (gdn_rollback_select, the
 *      koboldcpp bullet "llama: allow partial seq_rm for GDN models for
 *      speculative decoding"): slot 0 must equal slot accepted[b] bit for bit;
 *   3. the next draft of 100 tokens through the chunked path with the
 *      rollback fused in (gdn_prefill_chunked_ex_after_rollback), KDA gates
 *      (one per key row), float32 q/k/v, d = 64 (llama.cpp bullets "metal :
 *      add Metal backend for GGML_OP_GATED_DELTA_NET" and "llama : enable
 *      chunked fused GDN path");
 *   4. the error path: a NULL input returns GDN_ERR_NULL and launches nothing.
 * Bars: max|gpu - ref| / max|ref| per output tensor, 2e-4 for the token
 * kernel (float32 arithmetic) and 1e-2 for the chunked path (bf16 MFMA).
 * Exit status 0 when every check passes.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "gdn.h"

/* the oracle (oracle/gdn_oracle.c) */
int oracle_gdn_forward(int B, int T, int H, int Hqk, int tiled, int dk, int dv, int K, int kda,
                       const double* q, const double* k, const double* v, const double* g,
                       const double* beta, double* state, double* final_state, double* o);
int oracle_gdn_rollback(int B, int H, int K, int dk, int dv, const int32_t* accepted, double* state);

static int failures = 0;

#define HIP_OK(x)                                                                       \
    do {                                                                                \
        hipError_t e_ = (x);                                                            \
        if (e_ != hipSuccess) {                                                         \
            fprintf(stderr, "%s:%d: %s: %s\n", __FILE__, __LINE__, #x, hipGetErrorString(e_)); \
            exit(2);                                                                    \
        }                                                                               \
    } while (0)

/* splitmix64, then Box-Muller: seeded standard normals */
static uint64_t rng_state;
static double uniform01(void) {
    uint64_t z = (rng_state += 0x9e3779b97f4a7c15ULL);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
    z ^= z >> 31;
    return ((double)(z >> 11) + 0.5) / 9007199254740992.0;
}
static double normal(void) {
    const double u = uniform01(), v = uniform01();
    return sqrt(-2.0 * log(u)) * cos(6.283185307179586 * v);
}

/* float -> bf16 bits, round to nearest even (finite inputs) */
static uint16_t to_bf16(float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
static double from_bf16(uint16_t b) {
    const uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* n rows of length d, each of unit length times `scale`, in float32 */
static void unit_rows(float* x, size_t n, int d, double scale) {
    for (size_t r = 0; r < n; ++r) {
        double ss = 0.0;
        for (int i = 0; i < d; ++i) {
            const double z = normal();
            x[r * d + i] = (float)z;
            ss += z * z;
        }
        const double f = scale / sqrt(ss);
        for (int i = 0; i < d; ++i) x[r * d + i] = (float)(x[r * d + i] * f);
    }
}

static void* dev_copy(const void* host, size_t bytes, hipStream_t s) {
    void* p = NULL;
    HIP_OK(hipMalloc(&p, bytes ? bytes : 16));
    if (bytes) HIP_OK(hipMemcpyAsync(p, host, bytes, hipMemcpyHostToDevice, s));
    return p;
}

static double* f64_of(const float* x, size_t n) {
    double* d = (double*)malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i) d[i] = x[i];
    return d;
}

static void check(const char* what, const float* got, const double* ref, size_t n, double bar) {
    double diff = 0.0, mag = 0.0;
    int finite = 1;
    for (size_t i = 0; i < n; ++i) {
        const double d = fabs((double)got[i] - ref[i]);
        if (!isfinite(d)) finite = 0;
        else if (d > diff) diff = d;
        if (fabs(ref[i]) > mag) mag = fabs(ref[i]);
    }
    const double rel = finite ? diff / mag : NAN;
    const int ok = finite && rel <= bar;
    printf("%-44s max|diff|/max|ref| = %.3e (bar %.0e) %s\n", what, rel, bar, ok ? "ok" : "FAIL");
    if (!ok) ++failures;
}

int main(void) {
    hipStream_t s;
    HIP_OK(hipStreamCreate(&s));
    rng_state = 20261203u;

    /* ---- 1. verification, K = 4, shared q/k heads, bf16 q/k/v ---- */
    const int B = 3, T = 4, H = 4, Hq = 2, d = 128, K = 4;
    const size_t tile = (size_t)d * d;
    const size_t nqk = (size_t)B * T * Hq * d, nv = (size_t)B * T * H * d, nt = (size_t)B * T * H;
    const size_t nst = (size_t)B * H * K * tile, nfin = (size_t)B * H * tile;
    float* q = malloc(nqk * 4);
    float* k = malloc(nqk * 4);
    float* v = malloc(nv * 4);
    float* g = malloc(nt * 4);
    float* beta = malloc(nt * 4);
    float* st = calloc(nst, 4);
    unit_rows(q, (size_t)B * T * Hq, d, 1.0 / sqrt((double)d));
    unit_rows(k, (size_t)B * T * Hq, d, 1.0);
    for (size_t i = 0; i < nv; ++i) v[i] = (float)normal();
    for (size_t i = 0; i < nt; ++i) {
        g[i] = (float)-log1p(exp(normal())); /* log-gates <= 0 */
        beta[i] = (float)(1.0 / (1.0 + exp(-normal())));
    }
    for (int bh = 0; bh < B * H; ++bh)
        for (size_t e = 0; e < tile; ++e) st[(size_t)bh * K * tile + e] = (float)(0.1 * normal());
    uint16_t* qb = malloc(nqk * 2);
    uint16_t* kb = malloc(nqk * 2);
    uint16_t* vb = malloc(nv * 2);
    double *qd = malloc(nqk * 8), *kd = malloc(nqk * 8), *vd = malloc(nv * 8);
    for (size_t i = 0; i < nqk; ++i) {
        qb[i] = to_bf16(q[i]);
        kb[i] = to_bf16(k[i]);
        qd[i] = from_bf16(qb[i]);
        kd[i] = from_bf16(kb[i]);
    }
    for (size_t i = 0; i < nv; ++i) {
        vb[i] = to_bf16(v[i]);
        vd[i] = from_bf16(vb[i]);
    }
    void* dq = dev_copy(qb, nqk * 2, s);
    void* dk = dev_copy(kb, nqk * 2, s);
    void* dv = dev_copy(vb, nv * 2, s);
    float* dg = dev_copy(g, nt * 4, s);
    float* dbeta = dev_copy(beta, nt * 4, s);
    float* dst = dev_copy(st, nst * 4, s);
    float *dfin = NULL, *dout = NULL;
    HIP_OK(hipMalloc((void**)&dfin, nfin * 4));
    HIP_OK(hipMalloc((void**)&dout, nv * 4));
    int rc = gdn_forward_qk_broadcast(B, T, H, Hq, GDN_HEADS_GROUPED, d, d, GDN_BF16, GDN_GATE_HEAD, K, dq, dk, dv,
                                      dg, dbeta, dst, dfin, dout, (void*)s);
    if (rc != GDN_OK) {
        fprintf(stderr, "gdn_forward_qk_broadcast: %s\n", gdn_status_str(rc));
        return 1;
    }
    float* o = malloc(nv * 4);
    float* fin = malloc(nfin * 4);
    float* st_out = malloc(nst * 4);
    HIP_OK(hipMemcpyAsync(o, dout, nv * 4, hipMemcpyDeviceToHost, s));
    HIP_OK(hipMemcpyAsync(fin, dfin, nfin * 4, hipMemcpyDeviceToHost, s));
    HIP_OK(hipMemcpyAsync(st_out, dst, nst * 4, hipMemcpyDeviceToHost, s));
    HIP_OK(hipStreamSynchronize(s));

    double* gd = f64_of(g, nt);
    double* bd = f64_of(beta, nt);
    double* rst = f64_of(st, nst);
    double* rfin = malloc(nfin * 8);
    double* ro = malloc(nv * 8);
    if (oracle_gdn_forward(B, T, H, Hq, 0, d, d, K, 0, qd, kd, vd, gd, bd, rst, rfin, ro) != 0) return 1;
    check("verify: o", o, ro, nv, 2e-4);
    check("verify: final state", fin, rfin, nfin, 2e-4);
    for (int slot = 1; slot < K; ++slot) {
        /* gather slot `slot` of every head */
        float* gs = malloc((size_t)B * H * tile * 4);
        double* rs = malloc((size_t)B * H * tile * 8);
        for (int bh = 0; bh < B * H; ++bh) {
            memcpy(gs + (size_t)bh * tile, st_out + ((size_t)bh * K + slot) * tile, tile * 4);
            memcpy(rs + (size_t)bh * tile, rst + ((size_t)bh * K + slot) * tile, tile * 8);
        }
        char name[64];
        snprintf(name, sizeof name, "verify: snapshot slot %d", slot);
        check(name, gs, rs, (size_t)B * H * tile, 2e-4);
        free(gs);
        free(rs);
    }

    /* ---- 2. rollback to the accepted draft lengths, bit for bit ---- */
    const int32_t acc[3] = {0, 3, 2};
    int32_t* dacc = dev_copy(acc, sizeof acc, s);
    int32_t zero = 0, flag = -1;
    int32_t* dflag = dev_copy(&zero, 4, s);
    rc = gdn_rollback_select(B, H, K, d, d, dacc, dst, dflag, (void*)s);
    if (rc != GDN_OK) {
        fprintf(stderr, "gdn_rollback_select: %s\n", gdn_status_str(rc));
        return 1;
    }
    float* rolled = malloc(nst * 4);
    HIP_OK(hipMemcpyAsync(rolled, dst, nst * 4, hipMemcpyDeviceToHost, s));
    HIP_OK(hipMemcpyAsync(&flag, dflag, 4, hipMemcpyDeviceToHost, s));
    HIP_OK(hipStreamSynchronize(s));
    int exact = flag == 0;
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h) {
            const size_t base = ((size_t)b * H + h) * K * tile;
            /* slot 0 now holds slot acc[b] of the verification, every slot else unchanged */
            exact &= memcmp(rolled + base, st_out + base + (size_t)acc[b] * tile, tile * 4) == 0;
            exact &= memcmp(rolled + base + tile, st_out + base + tile, (K - 1) * tile * 4) == 0;
        }
    printf("%-44s %s\n", "rollback: slot 0 = slot accepted[b], exact", exact ? "ok" : "FAIL");
    if (!exact) ++failures;

    /* ---- 3. the next draft through the chunked path, rollback fused ---- */
    {
        const int T2 = 100, H2 = 2, d2 = 64, K2 = 4;
        const size_t tile2 = (size_t)d2 * d2;
        const size_t n_qkv = (size_t)B * T2 * H2 * d2, n_g = n_qkv, n_t = (size_t)B * T2 * H2;
        const size_t n_st = (size_t)B * H2 * K2 * tile2;
        float* q2 = malloc(n_qkv * 4);
        float* k2 = malloc(n_qkv * 4);
        float* v2 = malloc(n_qkv * 4);
        float* g2 = malloc(n_g * 4);
        float* b2 = malloc(n_t * 4);
        float* s2 = malloc(n_st * 4);
        unit_rows(q2, (size_t)B * T2 * H2, d2, 1.0 / sqrt((double)d2));
        unit_rows(k2, (size_t)B * T2 * H2, d2, 1.0);
        for (size_t i = 0; i < n_qkv; ++i) v2[i] = (float)normal();
        for (size_t i = 0; i < n_g; ++i) g2[i] = (float)-log1p(exp(normal()));
        for (size_t i = 0; i < n_t; ++i) b2[i] = (float)(1.0 / (1.0 + exp(-normal())));
        for (size_t i = 0; i < n_st; ++i) s2[i] = (float)(0.1 * normal()); /* a previous draft in every slot */
        const int32_t acc2[3] = {2, 0, 7}; /* 7 >= K: flagged, that sequence starts from slot 0 */
        void* dq2 = dev_copy(q2, n_qkv * 4, s);
        void* dk2 = dev_copy(k2, n_qkv * 4, s);
        void* dv2 = dev_copy(v2, n_qkv * 4, s);
        float* dg2 = dev_copy(g2, n_g * 4, s);
        float* db2 = dev_copy(b2, n_t * 4, s);
        float* ds2 = dev_copy(s2, n_st * 4, s);
        int32_t* dacc2 = dev_copy(acc2, sizeof acc2, s);
        HIP_OK(hipMemcpyAsync(dflag, &zero, 4, hipMemcpyHostToDevice, s));
        float* do2 = NULL;
        HIP_OK(hipMalloc((void**)&do2, n_qkv * 4));
        const size_t ws_bytes = gdn_prefill_workspace_size_ex(B, T2, H2, d2, d2, 64, GDN_F32, GDN_GATE_KEY);
        void* ws = NULL;
        HIP_OK(hipMalloc(&ws, ws_bytes));
        rc = gdn_prefill_chunked_ex_after_rollback(B, T2, H2, H2, GDN_HEADS_GROUPED, d2, d2, 64, GDN_F32, GDN_GATE_KEY,
                                                   K2, dacc2, dq2, dk2, dv2, dg2, db2, ds2, NULL, do2, ws, ws_bytes,
                                                   dflag, (void*)s);
        if (rc != GDN_OK) {
            fprintf(stderr, "gdn_prefill_chunked_ex_after_rollback: %s\n", gdn_status_str(rc));
            return 1;
        }
        float* o2 = malloc(n_qkv * 4);
        float* s2_out = malloc(n_st * 4);
        HIP_OK(hipMemcpyAsync(o2, do2, n_qkv * 4, hipMemcpyDeviceToHost, s));
        HIP_OK(hipMemcpyAsync(s2_out, ds2, n_st * 4, hipMemcpyDeviceToHost, s));
        HIP_OK(hipMemcpyAsync(&flag, dflag, 4, hipMemcpyDeviceToHost, s));
        HIP_OK(hipStreamSynchronize(s));

        /* the oracle: rollback, then the token loop on the float32 inputs */
        double* r2 = f64_of(s2, n_st);
        const int bad = oracle_gdn_rollback(B, H2, K2, d2, d2, acc2, r2);
        double *q2d = f64_of(q2, n_qkv), *k2d = f64_of(k2, n_qkv), *v2d = f64_of(v2, n_qkv);
        double *g2d = f64_of(g2, n_g), *b2d = f64_of(b2, n_t);
        double* ro2 = malloc(n_qkv * 8);
        if (oracle_gdn_forward(B, T2, H2, H2, 0, d2, d2, K2, 1, q2d, k2d, v2d, g2d, b2d, r2, NULL, ro2) != 0) return 1;
        check("prefill after rollback (KDA, f32 in): o", o2, ro2, n_qkv, 1e-2);
        for (int slot = 0; slot < K2; ++slot) {
            float* gs = malloc((size_t)B * H2 * tile2 * 4);
            double* rs = malloc((size_t)B * H2 * tile2 * 8);
            for (int bh = 0; bh < B * H2; ++bh) {
                memcpy(gs + (size_t)bh * tile2, s2_out + ((size_t)bh * K2 + slot) * tile2, tile2 * 4);
                memcpy(rs + (size_t)bh * tile2, r2 + ((size_t)bh * K2 + slot) * tile2, tile2 * 8);
            }
            char name[64];
            snprintf(name, sizeof name, "prefill after rollback: slot %d", slot);
            /* slot 0 is the rolled-back input itself: exact */
            check(name, gs, rs, (size_t)B * H2 * tile2, slot == 0 ? 0.0 : 1e-2);
            free(gs);
            free(rs);
        }
        const int flag_ok = bad == 1 && flag == 1;
        printf("%-44s %s\n", "prefill after rollback: invalid index flagged", flag_ok ? "ok" : "FAIL");
        if (!flag_ok) ++failures;
        free(q2); free(k2); free(v2); free(g2); free(b2); free(s2); free(o2); free(s2_out);
        free(r2); free(q2d); free(k2d); free(v2d); free(g2d); free(b2d); free(ro2);
        HIP_OK(hipFree(dq2)); HIP_OK(hipFree(dk2)); HIP_OK(hipFree(dv2)); HIP_OK(hipFree(dg2));
        HIP_OK(hipFree(db2)); HIP_OK(hipFree(ds2)); HIP_OK(hipFree(dacc2)); HIP_OK(hipFree(do2));
        HIP_OK(hipFree(ws));
    }

    /* ---- 4. the error path: nothing is launched ---- */
    rc = gdn_forward(B, T, H, d, d, GDN_BF16, GDN_GATE_HEAD, NULL, dk, dv, dg, dbeta, dst, dout, (void*)s);
    const int err_ok = rc == GDN_ERR_NULL && hipStreamQuery(s) == hipSuccess;
    printf("%-44s %s (%s)\n", "gdn_forward with q = NULL", err_ok ? "ok" : "FAIL", gdn_status_str(rc));
    if (!err_ok) ++failures;

    HIP_OK(hipFree(dq)); HIP_OK(hipFree(dk)); HIP_OK(hipFree(dv)); HIP_OK(hipFree(dg));
    HIP_OK(hipFree(dbeta)); HIP_OK(hipFree(dst)); HIP_OK(hipFree(dfin)); HIP_OK(hipFree(dout));
    HIP_OK(hipFree(dacc)); HIP_OK(hipFree(dflag));
    HIP_OK(hipStreamDestroy(s));
    free(q); free(k); free(v); free(g); free(beta); free(st); free(qb); free(kb); free(vb);
    free(qd); free(kd); free(vd); free(o); free(fin); free(st_out); free(gd); free(bd); free(rst);
    free(rfin); free(ro); free(rolled);
    printf("%s\n", failures ? "FAILED" : "all checks passed");
    return failures ? 1 : 0;
}
