// gdn_prefill.hip -- chunked prefill of the GDA recurrence on bf16 MFMA (gfx950).
//
// The pages enable a chunked fused GDN path for prompt processing (llama.cpp
// commit log, tag b9752, bullet "llama : enable chunked fused GDN path") but
// do not give its algebra.  This is the WY / UT form obtained by unrolling the
// recurrence inside a chunk of C = 64 tokens.  With chunk start state S,
// in-chunk cumulative log-gates G_r = g_0 + ... + g_r, and
//   A[r][s] = beta_r exp(G_r - G_s) (k_r . k_s)   (s < r),   T = (I + A)^-1,
//   T1 = T diag(beta),   QKm[r][s] = exp(G_r - G_s) (q_r . k_s)   (s <= r):
//     W      = T1 (V - diag(exp G) K S)                (the delta-rule writes)
//     O      = diag(exp G) Q S + QKm W
//     S_next = exp(G_last) S + K^T (diag(exp(G_last - G)) W)
// (equal to the token loop up to rounding; a short final chunk acts as if
// padded with k = q = v = 0, beta = 0, g = 0).
//
// Two kernels:
//  prep  (one wavefront per chunk and head, all chunks in parallel): G,
//        K K^T and Q K^T on MFMA, the gate masks, the unit lower triangular
//        inverse T by forward substitution in fp32, and T1 and QKm written to
//        the workspace as bf16 hi + lo pairs (x = hi + lo to ~2^-17).
//  chain (one workgroup of 4 wavefronts per head and 16 state columns,
//        serial over chunks): the fp32 state block lives in MFMA accumulators
//        (wavefront w owns d_k/4 rows); per chunk it forms X = K S and Q S
//        (S rounded to bf16 as the B operand), R = V - exp(G) X, W = T1 R,
//        O, and the state update, exchanging R, W and S through LDS.
//        Products whose rounding would reach the carried state or the
//        output visibly use hi/lo operand pairs (T1 R, QKm W, K^T W').
// Matrix layouts of v_mfma_f32_16x16x32_bf16 as used here: A (16 x 32):
// lane l holds row l%16, k = 8*(l/16) + 0..7; B (32 x 16): lane l holds
// column l%16, the same k; D (16 x 16 fp32): lane l holds column l%16, rows
// 4*(l/16) + 0..3.

#include "device_common.hpp"
#include "gdn_internal.hpp"

namespace gdn {

namespace {

constexpr int kC = 64;  // chunk length

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Workspace block of one (sequence, head, chunk).
constexpr size_t kWsT1Hi = 0;
constexpr size_t kWsT1Lo = kC * kC * 2;
constexpr size_t kWsQkHi = 2 * kC * kC * 2;
constexpr size_t kWsQkLo = 3 * kC * kC * 2;
constexpr size_t kWsG = 4 * kC * kC * 2;
constexpr size_t kWsBlock = kWsG + kC * 4;  // 33024 bytes, a multiple of 256

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ bf16x8 ld16_bf16(const void* p) {
    return as_bf16x8(*reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ bf16x8 zero_bf16x8() { return as_bf16x8(u32x4{0u, 0u, 0u, 0u}); }

// float32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne(float x) {
    uint32_t u = __float_as_uint(x);
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// x = hi + lo with hi, lo bf16 (both round to nearest).
__device__ __forceinline__ void split_bf16(float x, uint32_t& hi, uint32_t& lo) {
    hi = bf16_rne(x);
    lo = bf16_rne(x - __uint_as_float(hi << 16));
}

__device__ __forceinline__ u32x2 pack4(const uint32_t (&h)[4]) {
    return u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
}

}  // namespace

size_t prefill_workspace_bytes(int B, int T, int H, int d) {
    (void)d;
    const size_t nc = (static_cast<size_t>(T) + kC - 1) / kC;
    return static_cast<size_t>(B) * H * nc * kWsBlock;
}

// ---------------------------------------------------------------------------
// prep: one wavefront per (sequence, head, chunk)
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(64)
prefill_prep_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                    const float* __restrict__ g, const float* __restrict__ beta,
                    char* __restrict__ ws, int T, int H, int NC) {
    constexpr int KS = D / 32;  // MFMA k-steps over d_k
    __shared__ __attribute__((aligned(16))) float sA[kC][kC];
    __shared__ float sG[kC];
    __shared__ float sBeta[kC];

    const int lane = threadIdx.x;
    const int blk = blockIdx.x;  // (b * H + h) * NC + n
    const int n = blk % NC;
    const int bh = blk / NC;
    const int b = bh / H;
    const int h = bh - b * H;
    const int t0 = n * kC;
    const int nvalid = min(kC, T - t0);
    const int lr = lane & 15;  // MFMA row / column inside a tile
    const int grp = lane >> 4;

    // gates: inclusive prefix sum of the log-gates over the chunk
    float gv = 0.f, bv = 0.f;
    if (lane < nvalid) {
        const size_t bth = (static_cast<size_t>(b) * T + t0 + lane) * H + h;
        gv = g[bth];
        bv = beta[bth];
    }
    float G = gv;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        float y = __shfl_up(G, off, 64);
        if (lane >= off) G += y;
    }
    sG[lane] = G;
    sBeta[lane] = bv;
    char* wsb = ws + static_cast<size_t>(blk) * kWsBlock;
    reinterpret_cast<float*>(wsb + kWsG)[lane] = G;

    // fragments of the chunk's k rows (zero beyond the sequence end)
    auto row_ptr = [&](const uint16_t* base, int r) {
        return base + ((static_cast<size_t>(b) * T + t0 + r) * H + h) * D;
    };
    bf16x8 kf[4][KS];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int r = 16 * t + lr;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            kf[t][ks] = r < nvalid ? ld16_bf16(row_ptr(k, r) + 32 * ks + 8 * grp) : zero_bf16x8();
    }
    __syncthreads();

    // A = strict lower part of diag(beta) (exp(G_r - G_s)) o (K K^T)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int nt = 0; nt <= mt; ++nt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) acc = mfma(kf[mt][ks], kf[nt][ks], acc);
            const int col = 16 * nt + lr;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int row = 16 * mt + 4 * grp + rr;
                float a = 0.f;
                if (col < row) a = sBeta[row] * expf(sG[row] - sG[col]) * acc[rr];
                sA[row][col] = a;
            }
        }
    }

    // QKm = lower part (diagonal included) of exp(G_r - G_s) o (Q K^T), as hi/lo
    {
        bf16x8 qf[4][KS];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int r = 16 * t + lr;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                qf[t][ks] = r < nvalid ? ld16_bf16(row_ptr(q, r) + 32 * ks + 8 * grp) : zero_bf16x8();
        }
        uint16_t* qkh = reinterpret_cast<uint16_t*>(wsb + kWsQkHi);
        uint16_t* qkl = reinterpret_cast<uint16_t*>(wsb + kWsQkLo);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const int col = 16 * nt + lr;
                if (nt > mt) {
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        const int row = 16 * mt + 4 * grp + rr;
                        qkh[row * kC + col] = 0;
                        qkl[row * kC + col] = 0;
                    }
                    continue;
                }
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) acc = mfma(qf[mt][ks], kf[nt][ks], acc);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int row = 16 * mt + 4 * grp + rr;
                    float x = 0.f;
                    if (col <= row) x = expf(sG[row] - sG[col]) * acc[rr];
                    uint32_t hi, lo;
                    split_bf16(x, hi, lo);
                    qkh[row * kC + col] = static_cast<uint16_t>(hi);
                    qkl[row * kC + col] = static_cast<uint16_t>(lo);
                }
            }
        }
    }
    __syncthreads();

    // T = (I + A)^-1 by forward substitution, one column per lane, in fp32
    float x[kC];
#pragma unroll
    for (int r = 0; r < kC; ++r) {
        float acc = (r == lane) ? 1.f : 0.f;
#pragma unroll
        for (int s = 0; s < r; ++s) acc = fmaf(-sA[r][s], x[s], acc);
        x[r] = acc;
    }
    // T1 = T diag(beta): scale this lane's column, store as hi/lo bf16
    uint16_t* t1h = reinterpret_cast<uint16_t*>(wsb + kWsT1Hi);
    uint16_t* t1l = reinterpret_cast<uint16_t*>(wsb + kWsT1Lo);
    const float bcol = sBeta[lane];
#pragma unroll
    for (int r = 0; r < kC; ++r) {
        uint32_t hi, lo;
        split_bf16(x[r] * bcol, hi, lo);
        t1h[r * kC + lane] = static_cast<uint16_t>(hi);
        t1l[r * kC + lane] = static_cast<uint16_t>(lo);
    }
}

// ---------------------------------------------------------------------------
// chain: one workgroup (4 wavefronts) per (sequence, head, 16-column block)
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256)
prefill_chain_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                     const uint16_t* __restrict__ v, float* __restrict__ state,
                     float* __restrict__ o, const char* __restrict__ ws, int T, int H, int NC) {
    constexpr int NCB = D / 16;     // column blocks per head
    constexpr int KS = D / 32;      // k-steps over d_k
    constexpr int SROWS = D / 4;    // state rows per wavefront
    constexpr int SMT = SROWS / 16; // state tiles per wavefront
    constexpr int KLD = D + 8;      // padded LDS row of the K chunk (bf16)
    constexpr int CLD = kC + 8;     // padded LDS row of the [col][chunk row] buffers
    constexpr int SLD = D + 8;      // padded LDS row of S^T
    constexpr int KPT = kC * D / 8 / 256;  // 16-byte K pieces per thread

    __shared__ __attribute__((aligned(16))) uint16_t sK[2][kC][KLD];
    __shared__ __attribute__((aligned(16))) uint16_t sS[16][SLD];
    __shared__ __attribute__((aligned(16))) uint16_t sR[2][16][CLD];
    __shared__ __attribute__((aligned(16))) uint16_t sW[2][16][CLD];
    __shared__ __attribute__((aligned(16))) uint16_t sWp[2][16][CLD];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int lr = lane & 15;
    const int grp = lane >> 4;
    const int cb = blockIdx.x % NCB;
    const int bh = blockIdx.x / NCB;
    const int b = bh / H;
    const int h = bh - b * H;
    const int col = cb * 16 + lr;

    auto tok = [&](int t) { return (static_cast<size_t>(b) * T + t) * H + h; };

    // ---- initial state block (fp32, accumulator layout) --------------------
    float* st = state + static_cast<size_t>(bh) * D * D;
    f32x4 S[SMT];
#pragma unroll
    for (int mt = 0; mt < SMT; ++mt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
            S[mt][rr] = st[static_cast<size_t>(wave * SROWS + 16 * mt + 4 * grp + rr) * D + col];

    auto write_state_lds = [&]() {
#pragma unroll
        for (int mt = 0; mt < SMT; ++mt) {
            uint32_t hb[4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) hb[rr] = bf16_rne(S[mt][rr]);
            *reinterpret_cast<u32x2*>(&sS[lr][wave * SROWS + 16 * mt + 4 * grp]) = pack4(hb);
        }
    };

    // ---- per-chunk operands held in registers ------------------------------
    struct Ops {
        u32x4 kpiece[KPT];     // K chunk pieces, staged to LDS
        bf16x8 qf[KS];         // Q rows 16*wave.. (A operand)
        bf16x8 t1h[2], t1l[2]; // T1 rows 16*wave.. hi/lo
        bf16x8 qkh[2], qkl[2]; // QKm rows 16*wave.. hi/lo
        float vv[4];           // V at rows 16*wave + 4*grp + rr, column col
        float G[4];            // G at the same rows
        float Glast;
    };

    auto load_ops = [&](int n, Ops& p) {
        const int t0 = n * kC;
        const int nvalid = min(kC, T - t0);
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int piece = tid + 256 * i;
            const int r = piece / (D / 8);
            const int c8 = piece % (D / 8);
            p.kpiece[i] = r < nvalid ? *reinterpret_cast<const u32x4*>(k + tok(t0 + r) * D + 8 * c8)
                                     : u32x4{0u, 0u, 0u, 0u};
        }
        const int ra = 16 * wave + lr;  // A-operand row of this lane
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            p.qf[ks] = ra < nvalid ? ld16_bf16(q + tok(t0 + ra) * D + 32 * ks + 8 * grp) : zero_bf16x8();
        const char* wsb = ws + (static_cast<size_t>(bh) * NC + n) * kWsBlock;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const size_t off = (static_cast<size_t>(ra) * kC + 32 * ks + 8 * grp) * 2;
            p.t1h[ks] = ld16_bf16(wsb + kWsT1Hi + off);
            p.t1l[ks] = ld16_bf16(wsb + kWsT1Lo + off);
            p.qkh[ks] = ld16_bf16(wsb + kWsQkHi + off);
            p.qkl[ks] = ld16_bf16(wsb + kWsQkLo + off);
        }
        const float* Gp = reinterpret_cast<const float*>(wsb + kWsG);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int r = 16 * wave + 4 * grp + rr;
            p.vv[rr] = r < nvalid ? bf16_to_f32(v[tok(t0 + r) * D + col]) : 0.f;
            p.G[rr] = Gp[r];
        }
        p.Glast = Gp[kC - 1];
    };

    auto stage_k = [&](const Ops& p, int buf) {
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int piece = tid + 256 * i;
            const int r = piece / (D / 8);
            const int c8 = piece % (D / 8);
            *reinterpret_cast<u32x4*>(&sK[buf][r][8 * c8]) = p.kpiece[i];
        }
    };

    Ops cur, nxt;
    load_ops(0, cur);
    stage_k(cur, 0);
    write_state_lds();

    for (int n = 0; n < NC; ++n) {
        const int buf = n & 1;
        const int t0 = n * kC;
        const int nvalid = min(kC, T - t0);
        __syncthreads();  // sK[buf] and sS hold chunk n's K and the chunk start state
        if (n + 1 < NC) load_ops(n + 1, nxt);

        // X = K S and P = Q S for rows 16*wave.. of the chunk
        f32x4 X = {0.f, 0.f, 0.f, 0.f};
        f32x4 P = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 bS = ld16_bf16(&sS[lr][32 * ks + 8 * grp]);
            const bf16x8 aK = ld16_bf16(&sK[buf][16 * wave + lr][32 * ks + 8 * grp]);
            X = mfma(aK, bS, X);
            P = mfma(cur.qf[ks], bS, P);
        }

        // R = V - exp(G) X  ->  LDS as hi/lo, transposed [col][row]
        float eg[4];
        {
            uint32_t rh[4], rl[4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                eg[rr] = expf(cur.G[rr]);
                split_bf16(cur.vv[rr] - eg[rr] * X[rr], rh[rr], rl[rr]);
            }
            *reinterpret_cast<u32x2*>(&sR[0][lr][16 * wave + 4 * grp]) = pack4(rh);
            *reinterpret_cast<u32x2*>(&sR[1][lr][16 * wave + 4 * grp]) = pack4(rl);
        }
        __syncthreads();

        // W = T1 R (three hi/lo products)
        f32x4 W = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const bf16x8 bh_ = ld16_bf16(&sR[0][lr][32 * ks + 8 * grp]);
            const bf16x8 bl_ = ld16_bf16(&sR[1][lr][32 * ks + 8 * grp]);
            W = mfma(cur.t1h[ks], bh_, W);
            W = mfma(cur.t1h[ks], bl_, W);
            W = mfma(cur.t1l[ks], bh_, W);
        }
        {
            uint32_t wh[4], wl[4], ph[4], pl[4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                split_bf16(W[rr], wh[rr], wl[rr]);
                split_bf16(expf(cur.Glast - cur.G[rr]) * W[rr], ph[rr], pl[rr]);
            }
            *reinterpret_cast<u32x2*>(&sW[0][lr][16 * wave + 4 * grp]) = pack4(wh);
            *reinterpret_cast<u32x2*>(&sW[1][lr][16 * wave + 4 * grp]) = pack4(wl);
            *reinterpret_cast<u32x2*>(&sWp[0][lr][16 * wave + 4 * grp]) = pack4(ph);
            *reinterpret_cast<u32x2*>(&sWp[1][lr][16 * wave + 4 * grp]) = pack4(pl);
        }
        __syncthreads();

        // O = exp(G) P + QKm W
        {
            f32x4 O;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) O[rr] = eg[rr] * P[rr];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bf16x8 bh_ = ld16_bf16(&sW[0][lr][32 * ks + 8 * grp]);
                const bf16x8 bl_ = ld16_bf16(&sW[1][lr][32 * ks + 8 * grp]);
                O = mfma(cur.qkh[ks], bh_, O);
                O = mfma(cur.qkh[ks], bl_, O);
                O = mfma(cur.qkl[ks], bh_, O);
            }
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int r = 16 * wave + 4 * grp + rr;
                if (r < nvalid) o[tok(t0 + r) * D + col] = O[rr];
            }
        }

        // S <- exp(G_last) S + K^T W'   (K^T gathered from the staged chunk)
        {
            const float el = expf(cur.Glast);
#pragma unroll
            for (int mt = 0; mt < SMT; ++mt) {
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) S[mt][rr] *= el;
                const int dk_row = wave * SROWS + 16 * mt + lr;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    uint32_t e[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) e[j] = sK[buf][32 * ks + 8 * grp + j][dk_row];
                    const bf16x8 aKt = as_bf16x8(u32x4{e[0] | (e[1] << 16), e[2] | (e[3] << 16),
                                                       e[4] | (e[5] << 16), e[6] | (e[7] << 16)});
                    const bf16x8 bh_ = ld16_bf16(&sWp[0][lr][32 * ks + 8 * grp]);
                    const bf16x8 bl_ = ld16_bf16(&sWp[1][lr][32 * ks + 8 * grp]);
                    S[mt] = mfma(aKt, bh_, S[mt]);
                    S[mt] = mfma(aKt, bl_, S[mt]);
                }
            }
        }

        // chunk n + 1: state and K into LDS (no wavefront reads sS or
        // sK[buf ^ 1] past the barriers above)
        write_state_lds();
        if (n + 1 < NC) {
            stage_k(nxt, buf ^ 1);
            cur = nxt;
        }
    }

#pragma unroll
    for (int mt = 0; mt < SMT; ++mt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
            st[static_cast<size_t>(wave * SROWS + 16 * mt + 4 * grp + rr) * D + col] = S[mt][rr];
}

template <int D>
static hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t stream) {
    const int NC = (a.T + kC - 1) / kC;
    const unsigned bh = static_cast<unsigned>(a.B) * static_cast<unsigned>(a.H);
    char* ws = static_cast<char*>(a.workspace);
    hipLaunchKernelGGL(prefill_prep_kernel<D>, dim3(bh * NC), dim3(64), 0, stream,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k), a.g,
                       a.beta, ws, a.T, a.H, NC);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(prefill_chain_kernel<D>, dim3(bh * (D / 16)), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                       static_cast<const uint16_t*>(a.v), a.state, a.o, ws, a.T, a.H, NC);
    return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
    return a.d == 128 ? launch_prefill_t<128>(a, stream) : launch_prefill_t<64>(a, stream);
}

}  // namespace gdn
