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

// Workspace: one block per (sequence, head, chunk): T1 and QKm as bf16 hi/lo
// (row-major 64 x 64) and the gate factors exp(G_r), exp(G_last - G_r) and
// exp(G_last) in fp32.
constexpr int kWsT1Hi = 0;
constexpr int kWsT1Lo = kC * kC * 2;
constexpr int kWsQkHi = 2 * kC * kC * 2;
constexpr int kWsQkLo = 3 * kC * kC * 2;
constexpr int kWsEG = 4 * kC * kC * 2;     // exp(G_r)
constexpr int kWsER = kWsEG + kC * 4;      // exp(G_last - G_r)
constexpr int kWsEL = kWsER + kC * 4;      // exp(G_last)
constexpr int kWsBlock = kWsEL + 256;      // 33536 bytes, a multiple of 256

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

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t cvt2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// Four floats -> packed bf16 (4 values in 2 words).
__device__ __forceinline__ u32x2 to_bf16x4(float a, float b, float c, float d) {
    return u32x2{cvt2(a, b), cvt2(c, d)};
}

// Four floats x = hi + lo, hi and lo packed bf16 (both round to nearest).
__device__ __forceinline__ void split4(float a, float b, float c, float d, u32x2& hi, u32x2& lo) {
    hi = to_bf16x4(a, b, c, d);
    lo = to_bf16x4(a - __uint_as_float(hi[0] << 16), b - __uint_as_float(hi[0] & 0xffff0000u),
                    c - __uint_as_float(hi[1] << 16), d - __uint_as_float(hi[1] & 0xffff0000u));
}

}  // namespace

size_t prefill_workspace_bytes(int B, int T, int H, int d) {
    (void)d;
    size_t nc = (static_cast<size_t>(T) + kC - 1) / kC;
    nc += nc & 1;  // an even chunk count (see launch_prefill_t)
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
    {
        const float Glast = __shfl(G, 63, 64);
        reinterpret_cast<float*>(wsb + kWsEG)[lane] = expf(G);
        reinterpret_cast<float*>(wsb + kWsER)[lane] = expf(Glast - G);
        if (lane == 0) reinterpret_cast<float*>(wsb + kWsEL)[0] = expf(Glast);
    }

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

    // QKm = lower part (diagonal included) of exp(G_r - G_s) o (Q K^T), as
    // hi/lo.  Each 16 x 16 tile is formed transposed (K Q^T), so a lane holds
    // 4 consecutive columns s of one row r and stores them with one 8-byte
    // write per array.
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
        for (int rt = 0; rt < 4; ++rt) {  // tile of rows r (the query index)
            const int r = 16 * rt + lr;
#pragma unroll
            for (int st = 0; st < 4; ++st) {  // tile of columns s (the key index)
                const int s0 = 16 * st + 4 * grp;
                u32x2 hi = {0u, 0u}, lo = {0u, 0u};
                if (st <= rt) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) acc = mfma(kf[st][ks], qf[rt][ks], acc);
                    // acc[j] = q_r . k_(s0 + j)
                    float x[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        x[j] = (s0 + j <= r) ? expf(sG[r] - sG[s0 + j]) * acc[j] : 0.f;
                    split4(x[0], x[1], x[2], x[3], hi, lo);
                }
                *reinterpret_cast<u32x2*>(qkh + r * kC + s0) = hi;
                *reinterpret_cast<u32x2*>(qkl + r * kC + s0) = lo;
            }
        }
    }
    __syncthreads();

    // T = (I + A)^-1 by forward substitution, one column per lane, in fp32,
    // in blocks of 16 rows: first the contributions of all earlier blocks
    // (16 independent sums), then the sequential triangle of the block.
    float x[kC];
#pragma unroll
    for (int I = 0; I < kC / 16; ++I) {
        float y[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) y[i] = (16 * I + i == lane) ? 1.f : 0.f;
#pragma unroll
        for (int s4 = 0; s4 < 16 * I; s4 += 4) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const f32x4 av = *reinterpret_cast<const f32x4*>(&sA[16 * I + i][s4]);
                y[i] = fmaf(-av.x, x[s4], y[i]);
                y[i] = fmaf(-av.y, x[s4 + 1], y[i]);
                y[i] = fmaf(-av.z, x[s4 + 2], y[i]);
                y[i] = fmaf(-av.w, x[s4 + 3], y[i]);
            }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float acc = y[i];
#pragma unroll
            for (int s = 16 * I; s < 16 * I + i; ++s) acc = fmaf(-sA[16 * I + i][s], x[s], acc);
            x[16 * I + i] = acc;
        }
    }

    // T1 = T diag(beta): this lane's column, split hi/lo, transposed through
    // LDS (the A matrix is no longer read) so the stores are 16 bytes wide.
    __syncthreads();  // every read of A is done before its storage is reused
    uint16_t (*sT)[kC][kC] = reinterpret_cast<uint16_t (*)[kC][kC]>(&sA[0][0]);
    const float bcol = sBeta[lane];
#pragma unroll
    for (int r = 0; r < kC; ++r) {
        uint32_t hi, lo;
        split_bf16(x[r] * bcol, hi, lo);
        sT[0][r][lane] = static_cast<uint16_t>(hi);
        sT[1][r][lane] = static_cast<uint16_t>(lo);
    }
    __syncthreads();
    uint16_t* t1h = reinterpret_cast<uint16_t*>(wsb + kWsT1Hi);
    uint16_t* t1l = reinterpret_cast<uint16_t*>(wsb + kWsT1Lo);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int piece = lane + 64 * i;  // 64 rows x 8 pieces of 16 bytes
        const int r = piece >> 3, c = 8 * (piece & 7);
        *reinterpret_cast<u32x4*>(t1h + r * kC + c) = *reinterpret_cast<const u32x4*>(&sT[0][r][c]);
        *reinterpret_cast<u32x4*>(t1l + r * kC + c) = *reinterpret_cast<const u32x4*>(&sT[1][r][c]);
    }
}

// ---------------------------------------------------------------------------
// chain: one workgroup (4 wavefronts) per (sequence, head, 16-column block)
// ---------------------------------------------------------------------------

// Raw buffer resource over [base, base + bytes): loads past the end return
// zeros and stores past the end are dropped (the hardware range check), which
// handles the rows after the end of a sequence without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes > 0 ? bytes : 0,
                                             0x00020000);
}

__device__ __forceinline__ bf16x8 buf_ld16(__amdgpu_buffer_rsrc_t r, int off) {
    return as_bf16x8(__builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0)));
}

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
    __shared__ __attribute__((aligned(16))) uint16_t sV[2][16][CLD];  // V block, [col][row]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int lr = lane & 15;
    const int grp = lane >> 4;
    // Workgroups are dispatched to the 8 XCDs in turn (workgroup i on XCD
    // i % 8), and each XCD has its own L2.  All column blocks of a head read
    // the same per-chunk operands, so they are placed on one XCD: with the
    // head count a multiple of 8, workgroup i runs head (i % 8) + 8 * (j / NCB)
    // and column block j % NCB, where j = i / 8.
    int cb, bh;
    if (((gridDim.x / NCB) & 7) == 0) {
        const int j = blockIdx.x >> 3;
        bh = (blockIdx.x & 7) + 8 * (j / NCB);
        cb = j % NCB;
    } else {
        cb = blockIdx.x % NCB;
        bh = blockIdx.x / NCB;
    }
    const int b = bh / H;
    const int h = bh - b * H;
    const int col = cb * 16 + lr;

    // per (sequence, head) views; a token row is H*D elements apart
    const size_t head0 = (static_cast<size_t>(b) * T * H + h) * D;  // element of (b, t=0, h, 0)
    const int row_b16 = H * D * 2;                                  // bytes per token, bf16
    const int seq_b16 = (T - 1) * row_b16 + D * 2;  // bytes of the last valid row's end

    // per-lane byte offsets inside a chunk (constant over the chunks)
    int koff[KPT];
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const int piece = tid + 256 * i;
        koff[i] = (piece / (D / 8)) * row_b16 + (piece % (D / 8)) * 16;
    }
    const int ra = 16 * wave + lr;  // A-operand row of this lane
    const int qoff = ra * row_b16 + 16 * grp;
    const int woff = (ra * kC + 8 * grp) * 2;
    // V block of the chunk (64 rows x 16 columns): one 8-byte piece per thread
    const int vrow = tid >> 2, vq = tid & 3;
    const int voff = vrow * row_b16 + (cb * 16 + 4 * vq) * 2;
    const int goff = (16 * wave + 4 * grp) * 4;  // this lane's rows in the gate-factor arrays
    float* const obase = o + head0 + static_cast<size_t>(16 * wave + 4 * grp) * H * D + col;

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
        for (int mt = 0; mt < SMT; ++mt)
            *reinterpret_cast<u32x2*>(&sS[lr][wave * SROWS + 16 * mt + 4 * grp]) =
                to_bf16x4(S[mt][0], S[mt][1], S[mt][2], S[mt][3]);
    };

    // ---- per-chunk operands held in registers ------------------------------
    struct Ops {
        u32x4 kpiece[KPT];     // K chunk pieces, staged to LDS
        bf16x8 qf[KS];         // Q rows 16*wave.. (A operand)
        bf16x8 t1h[2], t1l[2]; // T1 rows 16*wave.. hi/lo
        bf16x8 qkh[2], qkl[2]; // QKm rows 16*wave.. hi/lo
        u32x2 vpiece;          // 4 bf16 of V, staged to LDS
        f32x4 eg;              // exp(G) at rows 16*wave + 4*grp + 0..3
        f32x4 er;              // exp(G_last - G) at the same rows
        float el;              // exp(G_last)
    };

    // Loads of chunk n's operands: buffer loads with constant per-lane
    // offsets from per-chunk (scalar) resources; rows past the sequence end
    // come back as zeros.
    auto load_ops = [&](int n, Ops& p) {
        const int cbyte = n * kC;  // first token of the chunk
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + head0 + static_cast<size_t>(cbyte) * H * D,
                                                     seq_b16 - cbyte * row_b16);
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + head0 + static_cast<size_t>(cbyte) * H * D,
                                                     seq_b16 - cbyte * row_b16);
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + head0 + static_cast<size_t>(cbyte) * H * D,
                                                     seq_b16 - cbyte * row_b16);
        const __amdgpu_buffer_rsrc_t rw =
            make_rsrc(ws + (static_cast<size_t>(bh) * NC + n) * kWsBlock, kWsBlock);
#pragma unroll
        for (int i = 0; i < KPT; ++i)
            p.kpiece[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, koff[i], 0, 0));
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) p.qf[ks] = buf_ld16(rq, qoff + 64 * ks);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            p.t1h[ks] = buf_ld16(rw, kWsT1Hi + woff + 64 * ks);
            p.t1l[ks] = buf_ld16(rw, kWsT1Lo + woff + 64 * ks);
            p.qkh[ks] = buf_ld16(rw, kWsQkHi + woff + 64 * ks);
            p.qkl[ks] = buf_ld16(rw, kWsQkLo + woff + 64 * ks);
        }
        p.vpiece = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rv, voff, 0, 0));
        p.eg = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, kWsEG + goff, 0, 0));
        p.er = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, kWsER + goff, 0, 0));
        // uniform address: a scalar load
        p.el = *reinterpret_cast<const float*>(ws + (static_cast<size_t>(bh) * NC + n) * kWsBlock + kWsEL);
    };

    auto stage_k = [&](const Ops& p, int buf) {
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int piece = tid + 256 * i;
            const int r = piece / (D / 8);
            const int c8 = piece % (D / 8);
            *reinterpret_cast<u32x4*>(&sK[buf][r][8 * c8]) = p.kpiece[i];
        }
        sV[buf][4 * vq + 0][vrow] = static_cast<uint16_t>(p.vpiece[0]);
        sV[buf][4 * vq + 1][vrow] = static_cast<uint16_t>(p.vpiece[0] >> 16);
        sV[buf][4 * vq + 2][vrow] = static_cast<uint16_t>(p.vpiece[1]);
        sV[buf][4 * vq + 3][vrow] = static_cast<uint16_t>(p.vpiece[1] >> 16);
    };

    // K^T fragment (rows dk0..dk0+15 of d_k, chunk rows 32*ks + 8*grp + 0..7)
    // from the row-major K chunk with two transposing LDS reads: source lane
    // s of each 16-lane group points at K[r0 + s/4][dk0 + 4*(s%4)], and lane
    // i receives K[r0 + j][dk0 + i] for j = 0..3.
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    auto kt_frag = [&](int buf, int dk0, int ks) {
        const int r0 = 32 * ks + 8 * grp + (lr >> 2);
        const int c0 = dk0 + 4 * (lr & 3);
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4i16*)(&sK[buf][r0][c0]));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4i16*)(&sK[buf][r0 + 4][c0]));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
        const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
        return as_bf16x8(u32x4{l2[0], l2[1], h2[0], h2[1]});
    };

    // One chunk: the state chain (X, R, W, S) first, then the outputs.
    auto step = [&](int n, const Ops& cur, Ops& nxt) {
        const int buf = n & 1;
        __syncthreads();  // sK[buf] and sS hold chunk n's K and the chunk start state

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
        // prefetch the next chunk (the last chunk reloads itself) behind the
        // products on the critical path
        load_ops(min(n + 1, NC - 1), nxt);

        // R = V - exp(G) X  ->  LDS as hi/lo, transposed [col][row]
        {
            const u32x2 vv = *reinterpret_cast<const u32x2*>(&sV[buf][lr][16 * wave + 4 * grp]);
            u32x2 rh, rl;
            split4(__uint_as_float(vv[0] << 16) - cur.eg[0] * X[0],
                   __uint_as_float(vv[0] & 0xffff0000u) - cur.eg[1] * X[1],
                   __uint_as_float(vv[1] << 16) - cur.eg[2] * X[2],
                   __uint_as_float(vv[1] & 0xffff0000u) - cur.eg[3] * X[3], rh, rl);
            *reinterpret_cast<u32x2*>(&sR[0][lr][16 * wave + 4 * grp]) = rh;
            *reinterpret_cast<u32x2*>(&sR[1][lr][16 * wave + 4 * grp]) = rl;
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
            u32x2 wh, wl, ph, pl;
            split4(W[0], W[1], W[2], W[3], wh, wl);
            split4(cur.er[0] * W[0], cur.er[1] * W[1], cur.er[2] * W[2], cur.er[3] * W[3], ph, pl);
            *reinterpret_cast<u32x2*>(&sW[0][lr][16 * wave + 4 * grp]) = wh;
            *reinterpret_cast<u32x2*>(&sW[1][lr][16 * wave + 4 * grp]) = wl;
            *reinterpret_cast<u32x2*>(&sWp[0][lr][16 * wave + 4 * grp]) = ph;
            *reinterpret_cast<u32x2*>(&sWp[1][lr][16 * wave + 4 * grp]) = pl;
        }
        __syncthreads();

        // S <- exp(G_last) S + K^T W'
#pragma unroll
        for (int mt = 0; mt < SMT; ++mt) {
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) S[mt][rr] *= cur.el;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bf16x8 aKt = kt_frag(buf, wave * SROWS + 16 * mt, ks);
                const bf16x8 bh_ = ld16_bf16(&sWp[0][lr][32 * ks + 8 * grp]);
                const bf16x8 bl_ = ld16_bf16(&sWp[1][lr][32 * ks + 8 * grp]);
                S[mt] = mfma(aKt, bh_, S[mt]);
                S[mt] = mfma(aKt, bl_, S[mt]);
            }
        }
        // no wavefront reads sS past the barriers above
        write_state_lds();

        // O = exp(G) P + QKm W
        {
            f32x4 O;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) O[rr] = cur.eg[rr] * P[rr];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bf16x8 bh_ = ld16_bf16(&sW[0][lr][32 * ks + 8 * grp]);
                const bf16x8 bl_ = ld16_bf16(&sW[1][lr][32 * ks + 8 * grp]);
                O = mfma(cur.qkh[ks], bh_, O);
                O = mfma(cur.qkh[ks], bl_, O);
                O = mfma(cur.qkl[ks], bh_, O);
            }
            // plain global stores (the raw buffer store builtin miscompiles
            // element extraction from accumulator registers here)
            const int t0 = n * kC;
            float* orow = obase + static_cast<size_t>(t0) * H * D;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                if (t0 + 16 * wave + 4 * grp + rr < T) orow[rr * static_cast<size_t>(H) * D] = O[rr];
        }
        stage_k(nxt, buf ^ 1);  // sK[buf ^ 1] was last read in the previous chunk
    };

    // Two operand buffers used in turn (no register copies between chunks).
    Ops opa, opb;
    load_ops(0, opa);
    stage_k(opa, 0);
    write_state_lds();
    for (int n = 0; n < NC; n += 2) {  // NC is even
        step(n, opa, opb);
        step(n + 1, opb, opa);
    }

#pragma unroll
    for (int mt = 0; mt < SMT; ++mt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
            st[static_cast<size_t>(wave * SROWS + 16 * mt + 4 * grp + rr) * D + col] = S[mt][rr];
}

template <int D>
static hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t stream) {
    // An odd chunk count gets one more chunk past the sequence end: all its
    // rows read zeros and beta = g = 0 there, so it leaves the state exactly
    // unchanged (exp(0) S + K^T 0) and writes no output.  The chain then
    // walks chunks in pairs with two operand buffers.
    int NC = (a.T + kC - 1) / kC;
    NC += NC & 1;
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
