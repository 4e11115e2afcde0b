/*
 * gdn_oracle.c -- float64 CPU oracle for the gated delta net (GDN) recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain reference that the
 * GPU library is checked against.  Only the test suite, the smoke check and
 * the benchmark's CPU-baseline leg may load it; the product path never does.
 * It shares no code, header or constant with the HIP library.
 *
 * Sources (commit-log pages; cited by page and commit bullet):
 *  [P1] koboldcpp commit log, tag v1.113.1 -- bullets "llama: allow partial
 *       seq_rm for GDN models for speculative decoding" (roll back up to
 *       draft_max by keeping the GDN intermediates) and "metal: add GDN
 *       partial rollback" (K snapshot slots, input read from slot 0 of a 3-D
 *       state tensor, intermediate states written to slots inside the token
 *       loop, K=1 keeps the single-slot behaviour).
 *  [P2] llama.cpp commit log, tag b9752 (src/models/qwen35.cpp) -- bullet
 *       "metal : add Metal backend for GGML_OP_GATED_DELTA_NET" (GDA: one
 *       scalar gate per head; KDA: one gate per key row; head sizes 64 and
 *       128) and bullet "llama : enable chunked fused GDN path".
 *
 * The pages name the operation but do not write it out.  The readings used
 * here (the gated delta rule in its usual form):
 *   per (sequence b, head h), state S is d_k x d_v, row i = key index,
 *   column j = value index;  for each token t in order:
 *     decay   GDA: S <- exp(g_t) S        KDA: S[i,:] <- exp(g_t[i]) S[i,:]
 *     delta   u = S^T k_t,  w = beta_t (v_t - u),  S <- S + k_t w^T
 *     readout o_t = S^T q_t   (the state after this token's update)
 *   No scale is applied to q inside the operation.
 *
 * Every function is a direct loop over the definition, in float64, with no
 * blocking, fusion or reordering.  OpenMP parallelises the independent
 * (sequence, head) pairs only; each pair runs the same sequential loop, so
 * results do not depend on the thread count.
 *
 * Layouts (row-major, last axis contiguous):
 *   q, k [B,T,H,dk]   v, o [B,T,H,dv]   g [B,T,H] (GDA) or [B,T,H,dk] (KDA)
 *   (oracle_gdn_forward also takes q, k with Hqk heads shared by the H value
 *   heads, see there)
 *   beta [B,T,H]      state [B,H,K,dk,dv]   final_state [B,H,dk,dv]
 *
 * Parity pins: every function here is pinned by the CPU tests against closed
 * forms, special cases and brute-force matrix algebra (see tests/).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* One token of the recurrence on one head's state S (dk x dv, row-major),
 * in the order decay, delta update, readout.  u and w are scratch of length
 * dv.  `gate` points at one log-gate (GDA) or dk log-gates (KDA). */
static void token_step(int dk, int dv, int kda, double* S, const double* q, const double* k,
                       const double* v, const double* gate, double beta, double* o,
                       double* u, double* w) {
    /* decay */
    for (int i = 0; i < dk; ++i) {
        double a = exp(kda ? gate[i] : gate[0]);
        for (int j = 0; j < dv; ++j) S[i * dv + j] *= a;
    }
    /* u = S^T k */
    for (int j = 0; j < dv; ++j) u[j] = 0.0;
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) u[j] += S[i * dv + j] * k[i];
    /* w = beta (v - u);  S <- S + k w^T */
    for (int j = 0; j < dv; ++j) w[j] = beta * (v[j] - u[j]);
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) S[i * dv + j] += k[i] * w[j];
    /* o = S^T q */
    for (int j = 0; j < dv; ++j) o[j] = 0.0;
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) o[j] += S[i * dv + j] * q[i];
}

/*
 * Sequential recurrence over T tokens with K state slots [P1 "metal: add GDN
 * partial rollback"].  Slot 0 of `state` is the input.  Writes:
 *   o[b,t,h,:]                      for every token;
 *   K == 1: state[b,h,0] <- S_T      (single-slot, in place);
 *   K  > 1: state[b,h,t] <- S_t for 1 <= t <= min(T, K-1), where S_t is the
 *           state after the first t tokens; slot 0 and slots above T are
 *           not written;
 *   final_state[b,h] <- S_T          when final_state is not NULL.
 * q and k have Hqk heads ([B,T,Hqk,dk]) read by the H value heads without
 * repeating them [P2 "models : avoid Q and K repeats when using fused GDA";
 * "reorder v heads for linear attention to avoid expensive interleaved
 * repeat"]: value head h reads q/k head h / (H / Hqk) when tiled == 0 (the
 * interleaved repeat: consecutive value heads share a q/k head) and
 * h % Hqk when tiled == 1.  Hqk == H is the plain case.
 * Returns 0, or -1 on a bad argument.
 */
int oracle_gdn_forward(int B, int T, int H, int Hqk, int tiled, int dk, int dv, int K, int kda,
                       const double* q, const double* k, const double* v, const double* g,
                       const double* beta, double* state, double* final_state, double* o) {
    if (B < 0 || T < 0 || H < 0 || dk < 1 || dv < 1 || K < 1) return -1;
    if (Hqk < 1 || H % Hqk != 0) return -1;
    const size_t tile = (size_t)dk * dv;
    int bad = 0;
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < H; ++h) {
            double* S = (double*)malloc(sizeof(double) * (tile + 2 * (size_t)dv));
            if (!S) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            double* u = S + tile;
            double* w = u + dv;
            double* slots = state + ((size_t)b * H + h) * K * tile;
            memcpy(S, slots, sizeof(double) * tile);
            const int hq = tiled ? h % Hqk : h / (H / Hqk);  /* the q/k head of value head h */
            for (int t = 0; t < T; ++t) {
                size_t bth = ((size_t)b * T + t) * H + h;
                size_t btq = ((size_t)b * T + t) * Hqk + hq;
                const double* gate = kda ? g + bth * dk : g + bth;
                token_step(dk, dv, kda, S, q + btq * dk, k + btq * dk, v + bth * dv, gate,
                           beta[bth], o + bth * dv, u, w);
                if (K > 1 && t + 1 <= K - 1) memcpy(slots + (size_t)(t + 1) * tile, S, sizeof(double) * tile);
            }
            if (K == 1) memcpy(slots, S, sizeof(double) * tile);
            if (final_state) memcpy(final_state + ((size_t)b * H + h) * tile, S, sizeof(double) * tile);
            free(S);
        }
    }
    return bad ? -1 : 0;
}

/*
 * Rollback after verification [P1 "llama: allow partial seq_rm for GDN
 * models for speculative decoding", "llama-memory: enable checkpointing with
 * partial rollback"]: for each sequence b with a = accepted[b],
 *   1 <= a <= K-1 : slot 0 of every head <- slot a (exact copy);
 *   a == 0        : nothing changes;
 *   otherwise     : the sequence is left untouched and counted as invalid.
 * Returns the number of invalid entries.
 */
int oracle_gdn_rollback(int B, int H, int K, int dk, int dv, const int32_t* accepted,
                        double* state) {
    const size_t tile = (size_t)dk * dv;
    int invalid = 0;
    for (int b = 0; b < B; ++b) {
        int a = accepted[b];
        if (a < 0 || a >= K) {
            ++invalid;
            continue;
        }
        if (a == 0) continue;
        for (int h = 0; h < H; ++h) {
            double* slots = state + ((size_t)b * H + h) * K * tile;
            memcpy(slots, slots + (size_t)a * tile, sizeof(double) * tile);
        }
    }
    return invalid;
}

/* Solve (I + A) X = R for X in place of R, A strictly lower triangular (n x n,
 * row-major), R n x m: forward substitution row by row. */
static void unit_lower_solve(int n, int m, const double* A, double* R) {
    for (int r = 0; r < n; ++r)
        for (int s = 0; s < r; ++s) {
            double a = A[r * n + s];
            for (int j = 0; j < m; ++j) R[r * m + j] -= a * R[s * m + j];
        }
}

/*
 * Chunked form of the recurrence [P2 "llama : enable chunked fused GDN
 * path"] -- the pages name the chunked path but not its algebra; this is the
 * standard WY / UT form obtained by unrolling the recurrence inside a chunk.
 * For a chunk of C tokens with start state S and in-chunk cumulative
 * log-gates G_r = g_0 + ... + g_r (GDA: one number per token; KDA: one per
 * key row i, G_r[i], [P2 "metal : add Metal backend for
 * GGML_OP_GATED_DELTA_NET"] for the two gate kinds):
 *   GDA
 *   A[r][s] = beta_r exp(G_r - G_s) (k_r . k_s)          for s < r, else 0
 *   W  = (I + A)^-1 diag(beta) (V - diag(exp G) K S)     (C x dv)
 *   O  = diag(exp G) Q S + (M o Q K^T) W,   M[r][s] = exp(G_r - G_s), s <= r
 *   S <- exp(G_{C-1}) S + (diag(exp(G_{C-1} - G)) K)^T W
 *   KDA (the decay of row i between tokens s and r is exp(G_r[i] - G_s[i]))
 *   A[r][s] = beta_r sum_i k_r[i] k_s[i] exp(G_r[i] - G_s[i])   for s < r
 *   W  = (I + A)^-1 diag(beta) (V - Kg S),   Kg[r][i] = k_r[i] exp(G_r[i])
 *   O  = Qg S + QKm W,   Qg[r][i] = q_r[i] exp(G_r[i]),
 *        QKm[r][s] = sum_i q_r[i] k_s[i] exp(G_r[i] - G_s[i])   for s <= r
 *   S[i,:] <- exp(G_{C-1}[i]) S[i,:] + sum_s exp(G_{C-1}[i] - G_s[i]) k_s[i] W[s,:]
 * Both follow from S_r = Gam_r S + sum_{s<=r} Gam_r Gam_s^-1 k_s w_s^T with
 * Gam_r = diag(exp G_r) and w_s the token deltas (the rows of W).
 * T need not be a multiple of C: the final chunk is simply shorter, which
 * equals padding it with k = q = v = 0, beta = 0, g = 0.
 * state [B,H,dk,dv] is read and overwritten with S_T; o [B,T,H,dv];
 * g [B,T,H] (kda = 0) or [B,T,H,dk] (kda = 1).
 * Returns 0, or -1 on a bad argument.
 */
int oracle_gdn_chunked(int B, int T, int H, int dk, int dv, int C, int kda, const double* q,
                       const double* k, const double* v, const double* g, const double* beta,
                       double* state, double* o) {
    if (B < 0 || T < 0 || H < 0 || dk < 1 || dv < 1 || C < 1) return -1;
    const size_t tile = (size_t)dk * dv;
    const int gw = kda ? dk : 1; /* gates per token */
    int bad = 0;
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < H; ++h) {
            size_t need = tile /* S */ + (size_t)C * dk * 2 /* Kc, Qc */ + (size_t)C * dv /* W */ +
                          (size_t)C * C * 2 /* A, QKm */ + (size_t)C * gw /* G */ +
                          (size_t)C * dv /* tmp */;
            double* buf = (double*)malloc(sizeof(double) * need);
            if (!buf) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            double* S = buf;
            double* Kc = S + tile;
            double* Qc = Kc + (size_t)C * dk;
            double* W = Qc + (size_t)C * dk;
            double* A = W + (size_t)C * dv;
            double* QK = A + (size_t)C * C;
            double* G = QK + (size_t)C * C; /* G[r * gw + i] */
            double* tmp = G + (size_t)C * gw;
            double* S0 = state + ((size_t)b * H + h) * tile;
            memcpy(S, S0, sizeof(double) * tile);
            for (int t0 = 0; t0 < T; t0 += C) {
                int n = T - t0 < C ? T - t0 : C;
                double bet[n > 0 ? n : 1];
                /* gather the chunk and its cumulative log-gates */
                for (int r = 0; r < n; ++r) {
                    size_t bth = ((size_t)b * T + t0 + r) * H + h;
                    for (int i = 0; i < gw; ++i)
                        G[(size_t)r * gw + i] = (r > 0 ? G[(size_t)(r - 1) * gw + i] : 0.0) + g[bth * gw + i];
                    bet[r] = beta[bth];
                    memcpy(Kc + (size_t)r * dk, k + bth * dk, sizeof(double) * dk);
                    memcpy(Qc + (size_t)r * dk, q + bth * dk, sizeof(double) * dk);
                }
                /* A and the decay-masked Q K^T */
                for (int r = 0; r < n; ++r)
                    for (int s = 0; s < n; ++s) {
                        double kk = 0.0, qk = 0.0;
                        if (!kda) {
                            for (int i = 0; i < dk; ++i) {
                                kk += Kc[(size_t)r * dk + i] * Kc[(size_t)s * dk + i];
                                qk += Qc[(size_t)r * dk + i] * Kc[(size_t)s * dk + i];
                            }
                            double m = exp(G[r] - G[s]);
                            kk *= m;
                            qk *= m;
                        } else if (s <= r) {
                            for (int i = 0; i < dk; ++i) {
                                double m = exp(G[(size_t)r * dk + i] - G[(size_t)s * dk + i]);
                                kk += Kc[(size_t)r * dk + i] * Kc[(size_t)s * dk + i] * m;
                                qk += Qc[(size_t)r * dk + i] * Kc[(size_t)s * dk + i] * m;
                            }
                        }
                        A[r * n + s] = s < r ? bet[r] * kk : 0.0;
                        QK[r * n + s] = s <= r ? qk : 0.0;
                    }
                /* right-hand side diag(beta) (V - (decayed K) S), then solve */
                for (int r = 0; r < n; ++r) {
                    size_t bth = ((size_t)b * T + t0 + r) * H + h;
                    for (int j = 0; j < dv; ++j) {
                        double ks = 0.0;
                        if (!kda) {
                            for (int i = 0; i < dk; ++i) ks += Kc[(size_t)r * dk + i] * S[(size_t)i * dv + j];
                            ks *= exp(G[r]);
                        } else {
                            for (int i = 0; i < dk; ++i)
                                ks += Kc[(size_t)r * dk + i] * exp(G[(size_t)r * dk + i]) * S[(size_t)i * dv + j];
                        }
                        W[(size_t)r * dv + j] = bet[r] * (v[bth * dv + j] - ks);
                    }
                }
                unit_lower_solve(n, dv, A, W);
                /* outputs */
                for (int r = 0; r < n; ++r) {
                    size_t bth = ((size_t)b * T + t0 + r) * H + h;
                    for (int j = 0; j < dv; ++j) {
                        double qs = 0.0;
                        if (!kda) {
                            for (int i = 0; i < dk; ++i) qs += Qc[(size_t)r * dk + i] * S[(size_t)i * dv + j];
                            qs *= exp(G[r]);
                        } else {
                            for (int i = 0; i < dk; ++i)
                                qs += Qc[(size_t)r * dk + i] * exp(G[(size_t)r * dk + i]) * S[(size_t)i * dv + j];
                        }
                        double intra = 0.0;
                        for (int s = 0; s <= r; ++s) intra += QK[r * n + s] * W[(size_t)s * dv + j];
                        tmp[j] = qs + intra;
                    }
                    memcpy(o + bth * dv, tmp, sizeof(double) * dv);
                }
                /* carry the state to the end of the chunk */
                for (int i = 0; i < dk; ++i) {
                    const int gi = kda ? i : 0;
                    const double gl = G[(size_t)(n - 1) * gw + gi];
                    const double el = exp(gl);
                    for (int j = 0; j < dv; ++j) {
                        double add = 0.0;
                        for (int s = 0; s < n; ++s)
                            add += exp(gl - G[(size_t)s * gw + gi]) * Kc[(size_t)s * dk + i] * W[(size_t)s * dv + j];
                        S[(size_t)i * dv + j] = el * S[(size_t)i * dv + j] + add;
                    }
                }
            }
            memcpy(S0, S, sizeof(double) * tile);
            free(buf);
        }
    }
    return bad ? -1 : 0;
}
