// gdn_prefill.hip -- chunked prefill of the GDN recurrence on bf16 MFMA (gfx950).
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
// padded with k = q = v = 0, beta = 0, g = 0).  With one log-gate per key row
// (KDA, same page, bullet "metal : add Metal backend for
// GGML_OP_GATED_DELTA_NET") the decays move inside the sums over keys: A and
// QKm take exp(G_r[i] - G_s[i]) per key i, K and Q are used as K o exp(G) and
// Q o exp(G), and the state carry is diag(exp G_last) S + (K o exp(G_last -
// G))^T W.  The key and value head sizes DK and DV (64 or 128 each) are
// separate template parameters: the state is DK x DV.
//
// Two kernels (plus, for packed sequences of different lengths, a
// one-wavefront table of sanitised offsets):
//  prep  (one wavefront per chunk and head, all chunks in parallel): G,
//        K K^T and Q K^T on MFMA, the gate masks, the unit lower triangular
//        inverse T in fp32 by 16 x 16 blocks (forward substitution on the
//        diagonal, block substitution on fp32 MFMA below).  It writes T1 and QKm to
//        the workspace as ready-made MFMA A operands (bf16 hi + lo pairs,
//        x = hi + lo to ~2^-17), in the order the chain kernel reads them,
//        plus the gate factors; for KDA also the decayed K and Q images and
//        the state update's operand fragments, and for float32 q/k/v the
//        bf16 images of K, Q and V.
//  chain (one workgroup per head and 16 state columns, serial over chunks):
//        four state wavefronts hold the DK x 16 fp32 state block in MFMA
//        accumulators and per chunk form X = K S, R = V - exp(G) X, W = T1 R
//        and S <- exp(G_last) S + K^T (exp(G_last - G) W), exchanging R, W
//        and the bf16 state through LDS (three barriers per chunk), and
//        write the K-slot snapshots that fall in the chunk; four output
//        wavefronts form O = exp(G) Q S + QKm W alongside; four loader
//        wavefronts fill a four-slot LDS ring with direct-to-LDS loads three
//        chunks ahead, and a storer wavefront writes O.
//        Products whose rounding would reach the carried state or the output
//        visibly use hi/lo operand pairs (T1 R, QKm W, K^T W').
//
// Matrix layouts of v_mfma_f32_16x16x32_bf16: A (16 x 32): lane l holds row
// l%16, k = 8*(l/16) + 0..7; B (32 x 16): lane l holds column l%16, the same
// k; D (16 x 16 fp32): lane l holds column l%16, rows 4*(l/16) + 0..3.  The
// order of k inside one instruction is free as long as A and B agree, so two
// D tiles stacked along k form a B operand as they are when A is read in the
// "split" k order {4*(l/16) + 0..3, 16 + 4*(l/16) + 0..3}.  Every product
// whose B operand is an earlier result uses that order.

#include "device_common.hpp"
#include <type_traits>

#include "gdn_internal.hpp"
#include "gdn_prefill_args.hpp"

namespace gdn {

namespace {

constexpr int kC = 64;  // chunk length

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef short v4i16 __attribute__((ext_vector_type(4)));

// Workspace: one block per (sequence, head, chunk), written by the prep
// kernel in the order the chain kernel reads it, so that each chain load
// instruction reads 1 KiB of contiguous memory:
//   T1F  T1 as A operands, [row tile 4][k-step 2][hi, lo][lane 64][8 bf16] (split k order)
//   QKF  the decay-masked Q K^T as A operands, same shape and order as T1F
//   E    fp32 [64] exp(G_r), [64] exp(G_last - G_r), [1] exp(G_last) at float 128;
//        1 KiB in all
template <int DK>
struct Ws {
    static constexpr int KS = DK / 32;  // MFMA k-steps over d_k
    static constexpr int kT1F = 0;
    static constexpr int kQKF = kT1F + 4 * 2 * 2 * 64 * 16;
    static constexpr int kE = kQKF + 4 * 2 * 2 * 64 * 16;
    static constexpr int kBlock = kE + 1024;
    static_assert(kBlock % 256 == 0, "workspace blocks stay 256-byte aligned");
};
// KDA (one log-gate per key row): the same T1F, QKF and gate block, then
// the decayed operands the chain reads in place of K and Q (rows past the end
// of the sequence are zero):
//   KG   K o exp(G), row-major [64][DK] bf16 (row r, key i: k_r[i] exp(G_r[i]))
//   QG   Q o exp(G), the same layout
//   KDF  (K o exp(G_last - G))^T as the state update's A operands: for state
//        wavefront w, state tile mt and k-step ks (chunk rows 32 ks.., split
//        order), 64 lanes x 16 bytes at ((w * DK/64 + mt) * 2 + ks) * 1 KiB
// and E holds fp32 exp(G_last[i]) for the DK key rows.
template <int DK>
struct WsKda : Ws<DK> {
    static constexpr int kKG = Ws<DK>::kBlock;
    static constexpr int kQG = kKG + kC * DK * 2;
    static constexpr int kKDF = kQG + kC * DK * 2;
    static constexpr int kBlock = kKDF + kC * DK * 2;
    static_assert(kBlock % 256 == 0, "workspace blocks stay 256-byte aligned");
};
// Workspace block of one (sequence, head, chunk) for each gate kind and input
// type.  With float32 q/k/v the prep also rounds the chunk's K, Q and V rows
// to bf16 images (zero past the sequence end), row-major [64][DK] for K and Q
// and by column block [DV/16][64][16] for V, which the chain reads in place
// of the inputs; KDA's decayed KG and QG already are such images, so KDA adds
// only V.
template <int DK, int DV, bool KDA, bool F32>
struct WsL : std::conditional_t<KDA, WsKda<DK>, Ws<DK>> {
    using Base = std::conditional_t<KDA, WsKda<DK>, Ws<DK>>;
    static constexpr int kImg = kC * DK * 2;   // a K or Q image
    static constexpr int kImgV = kC * DV * 2;  // the V image
    static constexpr int kKI = KDA ? WsKda<DK>::kKG : Base::kBlock;        // K image the chain reads
    static constexpr int kQI = KDA ? WsKda<DK>::kQG : Base::kBlock + kImg; // Q image the chain reads
    static constexpr int kVI = Base::kBlock + (KDA ? 0 : 2 * kImg);         // V image (F32), by column block
    static constexpr int kBlock = F32 ? kVI + kImgV : Base::kBlock;
    static_assert(kBlock % 256 == 0, "workspace blocks stay 256-byte aligned");
};
// float offsets inside E
constexpr int kEg = 0, kEr = 64, kEl = 128, kEs = 192;
constexpr int kEv = 0;  // KDA: exp(G_last[i]), i < DK

// Byte offset of A operand (row tile t, k-step ks, hi/lo hl) of lane `lane` in T1F / QKF.
__host__ __device__ constexpr int frag_off(int t, int ks, int hl, int lane) {
    return (((t * 2 + ks) * 2 + hl) * 64 + lane) * 16;
}

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

// Two 4-value halves (k = 4g + 0..3 and 16 + 4g + 0..3) -> one split-order operand.
__device__ __forceinline__ bf16x8 join(const u32x2& lo, const u32x2& hi) {
    return as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
}

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

__device__ __forceinline__ void split4(const f32x4& x, u32x2& hi, u32x2& lo) {
    split4(x[0], x[1], x[2], x[3], hi, lo);
}

// Raw buffer resource over [base, base + bytes): loads past the end return
// zeros (the hardware range check), which handles the rows after the end of a
// sequence without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes > 0 ? bytes : 0,
                                             0x00020000);
}

__device__ __forceinline__ u32x4 buf_ld16(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Wait until at most N of this wavefront's global and direct-to-LDS loads
// are outstanding (s_waitcnt vmcnt(N) in the gfx9 encoding, expcnt and
// lgkmcnt unconstrained; the compiler sees the wait and counts from it).
template <int N>
__device__ __forceinline__ void vm_wait_keep() {
    static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0f70);
}
__device__ __forceinline__ void vm_wait_all() { vm_wait_keep<0>(); }

// Transposing LDS read (ds_read_tr16_b64): within each 16-lane group, lane
// i receives element i%4 of the 8-byte words that lanes 4j + i/4 point at,
// j = 0..3.
__device__ __forceinline__ u32x2 ld_tr(const uint16_t* p) {
    return __builtin_bit_cast(
        u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(p)));
}

}  // namespace

// Where the sequences lie.  Tokens are rows of [total tokens, heads, d]
// arrays; sequence i covers tokens [start_i, start_i + len_i) and owns the
// workspace chunks [c0_i, c0_i + nc_i) of every head (block (h, c) at
// ws + (h * CT + c) * kBlock, CT chunks per head).  Either N sequences of T
// tokens each (tab == nullptr), or a table of sanitised starts and chunk
// offsets built by prefill_table_kernel from the caller's cu_seqlens.
struct SeqGeom {
    const int32_t* tab;  // [0, N]: first token of each sequence; [N+1, 2N+1]: first chunk
    int N, T, NC;        // N sequences; T tokens and NC chunks each when tab == nullptr
    int CT;              // chunk blocks per head in the workspace
    __device__ __forceinline__ void seq(int i, int& start, int& len, int& c0, int& nc) const {
        if (tab != nullptr) {
            start = tab[i];
            len = tab[i + 1] - start;
            c0 = tab[N + 1 + i];
            nc = tab[N + 2 + i] - c0;
        } else {
            start = i * T;
            len = T;
            c0 = i * NC;
            nc = NC;
        }
    }
    // The sequence owning chunk c, or -1 for a chunk past the last sequence's.
    __device__ __forceinline__ int owner(int c) const {
        if (tab == nullptr) return c / NC;
        const int32_t* coff = tab + N + 1;
        if (c >= coff[N]) return -1;
        int lo = 0, hi = N - 1;  // the last i with coff[i] <= c
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (coff[mid] <= c) lo = mid; else hi = mid - 1;
        }
        return lo;
    }
};

// Bytes of the varlen table at the start of the workspace (256-byte aligned).
static size_t table_bytes(int N) { return ((static_cast<size_t>(2 * (N + 1)) * 4 + 255) / 256) * 256; }

template <bool KDA, bool F32>
static size_t block_bytes_t(int dk, int dv) {
    if (dk == 128) return dv == 128 ? WsL<128, 128, KDA, F32>::kBlock : WsL<128, 64, KDA, F32>::kBlock;
    return dv == 128 ? WsL<64, 128, KDA, F32>::kBlock : WsL<64, 64, KDA, F32>::kBlock;
}
static size_t block_bytes(int dk, int dv, bool kda, bool f32) {
    if (kda) return f32 ? block_bytes_t<true, true>(dk, dv) : block_bytes_t<true, false>(dk, dv);
    return f32 ? block_bytes_t<false, true>(dk, dv) : block_bytes_t<false, false>(dk, dv);
}

size_t prefill_workspace_bytes(int B, int T, int H, int dk, int dv, bool kda, bool f32) {
    const size_t nc = (static_cast<size_t>(T) + kC - 1) / kC;
    return static_cast<size_t>(B) * H * nc * block_bytes(dk, dv, kda, f32);
}

// Variable lengths: at most total / C + N chunks over all sequences (each
// sequence adds at most one partial chunk), plus the table.
size_t prefill_varlen_workspace_bytes(int N, int total, int H, int dk, int dv, bool kda, bool f32) {
    const size_t ct = (static_cast<size_t>(total) + kC - 1) / kC + N;
    return table_bytes(N) + static_cast<size_t>(H) * ct * block_bytes(dk, dv, kda, f32);
}

// ---------------------------------------------------------------------------
// table: sanitised sequence starts and chunk offsets from cu_seqlens.  Each
// offset is clamped to [0, total] and made non-decreasing (a running maximum),
// so the sequences never overlap or leave [0, total) whatever the caller
// passes; the chunk offsets are the running sum of ceil(len / C).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(64)
prefill_table_kernel(const int32_t* __restrict__ cu, int N, int total, int32_t* __restrict__ tab) {
    const int lane = threadIdx.x;
    int run_max = 0, run_sum = 0;  // carried across blocks of 64 offsets
    for (int base = 0; base <= N; base += 64) {
        const int i = base + lane;
        int x = 0;
        if (i <= N) x = min(max(cu[i], 0), total);
        // inclusive running maximum of the clamped offsets
        int m = max(x, run_max);
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(m, off, 64);
            if (lane >= off) m = max(m, y);
        }
        // chunks of sequence i - 1, which ends at m_i and starts at m_(i-1)
        int prev = __shfl_up(m, 1, 64);
        if (lane == 0) prev = run_max;
        int c = (i >= 1 && i <= N) ? (m - prev + kC - 1) / kC : 0;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(c, off, 64);
            if (lane >= off) c += y;
        }
        if (i <= N) {
            tab[i] = m;
            tab[N + 1 + i] = run_sum + c;
        }
        run_max = __shfl(m, 63, 64);
        run_sum += __shfl(c, 63, 64);
    }
}

// ---------------------------------------------------------------------------
// prep: one wavefront per (sequence, head, chunk)
// ---------------------------------------------------------------------------
// Row pitch of the fp32 A matrix in LDS: 4 floats of padding move each row
// by 4 banks, so that 16 rows read at one column offset meet distinct banks.
constexpr int kAP = kC + 4;

__device__ __forceinline__ f32x4 mfma_f32(f32x4 acc, const f32x4& a, const f32x4& b) {
    // k = 4 (l / 16) + s at step s: lane l gives a[s] = X[l % 16][k] and
    // b[s] = Y[k][l % 16], so 4 steps sum X Y over k = 0..15 with the
    // operands in the layout of an MFMA result
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], acc, 0, 0, 0);
    return acc;
}

// T1 = (I + A)^-1 diag(beta) for one chunk, from A (strict lower part, fp32,
// pitch kAP, in sA) and beta (sBeta), written to the workspace block as T1F.
// With I + A in 16 x 16 blocks and D_b the inverse of diagonal block b, the
// inverse T has T_bb = D_b and, below the diagonal (block substitution),
//   T_ij = -D_i (A_ij D_j + sum_{j<k<i} A_ik T_kj).
// The D_b come from forward substitution in fp32 (16 lanes per block, one
// column each) and the blocks below the diagonal from fp32 MFMA 16x16x4
// products.  A 16 x 16 MFMA result holds rows 4 (l / 16) + 0..3 of column
// l % 16 in lane l.  Blocks of T that later products take as right factor
// are formed that way (T_ij = D_i P, with P = -(A_ij D_j + ...)); every
// block below the diagonal is also formed transposed (P^T D_i^T), which puts
// row l % 16, columns 4 (l / 16) + 0..3 in lane l: the split-order A operand
// layout of T1F.  The upper blocks of sA (never written with A) keep the D_b.
// Called by the whole (one-wavefront) block after a barrier that publishes A.
template <class L>
__device__ __forceinline__ void solve_store_t1(float (*sA)[kAP], const float* sBeta, char* wsb,
                                               int lane) {
    const int lr = lane & 15;
    const int grp = lane >> 4;
    // D_b is kept in upper block (0, b + 1) of sA for b < 3, D_3 in (1, 2)
    auto drow = [](int b) { return b == 3 ? 16 : 0; };
    auto dcol = [](int b) { return b == 3 ? 32 : 16 * (b + 1); };
    {
        // column lr of D_grp: forward substitution over the block's 16 rows
        const int b = grp;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float acc = (i == lr) ? 1.f : 0.f;
#pragma unroll
            for (int s4 = 0; 4 * s4 < i; ++s4) {
                const f32x4 av = *reinterpret_cast<const f32x4*>(&sA[16 * b + i][16 * b + 4 * s4]);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (4 * s4 + e < i) acc = fmaf(-av[e], x[4 * s4 + e], acc);
            }
            x[i] = acc;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sA[drow(b) + i][dcol(b) + lr] = x[i];
    }
    __syncthreads();  // the D_b are published

    // row lr, columns 4 grp + 0..3 of the block at (r0, c0): A operand of X in X Y
    auto rows = [&](int r0, int c0) {
        return *reinterpret_cast<const f32x4*>(&sA[r0 + lr][c0 + 4 * grp]);
    };
    // rows 4 grp + 0..3 of column lr of D_b: B operand of D_b in X D_b
    auto dcolumn = [&](int b) {
        f32x4 v;
#pragma unroll
        for (int s = 0; s < 4; ++s) v[s] = sA[drow(b) + 4 * grp + s][dcol(b) + lr];
        return v;
    };
    auto neg = [](const f32x4& v) { return f32x4{-v[0], -v[1], -v[2], -v[3]}; };
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    f32x4 Dr[4], Dc[3];
#pragma unroll
    for (int b = 0; b < 4; ++b) Dr[b] = rows(drow(b), dcol(b));
#pragma unroll
    for (int b = 0; b < 3; ++b) Dc[b] = dcolumn(b);

    // Tt[i][j]: block (i, j) of T as row lr, columns 4 grp + 0..3
    f32x4 Tt[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) Tt[i][j] = i == j ? Dr[i] : z;
    // column block 0
    f32x4 Pn = neg(mfma_f32(z, rows(16, 0), Dc[0]));
    const f32x4 T10 = mfma_f32(z, Dr[1], Pn);
    Tt[1][0] = mfma_f32(z, Pn, Dr[1]);
    Pn = neg(mfma_f32(mfma_f32(z, rows(32, 0), Dc[0]), rows(32, 16), T10));
    const f32x4 T20 = mfma_f32(z, Dr[2], Pn);
    Tt[2][0] = mfma_f32(z, Pn, Dr[2]);
    Pn = neg(mfma_f32(mfma_f32(mfma_f32(z, rows(48, 0), Dc[0]), rows(48, 16), T10), rows(48, 32), T20));
    Tt[3][0] = mfma_f32(z, Pn, Dr[3]);
    // column block 1
    Pn = neg(mfma_f32(z, rows(32, 16), Dc[1]));
    const f32x4 T21 = mfma_f32(z, Dr[2], Pn);
    Tt[2][1] = mfma_f32(z, Pn, Dr[2]);
    Pn = neg(mfma_f32(mfma_f32(z, rows(48, 16), Dc[1]), rows(48, 32), T21));
    Tt[3][1] = mfma_f32(z, Pn, Dr[3]);
    // column block 2
    Pn = neg(mfma_f32(z, rows(48, 32), Dc[2]));
    Tt[3][2] = mfma_f32(z, Pn, Dr[3]);

    // T1 = T diag(beta), split hi/lo, as split-order A operands: k-step ks
    // of row tile t takes columns 4 grp + 0..3 of blocks 2 ks and 2 ks + 1
    f32x4 bt[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) bt[j] = *reinterpret_cast<const f32x4*>(&sBeta[16 * j + 4 * grp]);
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            if (2 * ks > t) continue;  // above the diagonal: zero, never read
            u32x2 hi[2], lo[2];
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int j = 2 * ks + half;
                const f32x4 v = Tt[t][j];
                split4(v[0] * bt[j][0], v[1] * bt[j][1], v[2] * bt[j][2], v[3] * bt[j][3], hi[half], lo[half]);
            }
            *reinterpret_cast<u32x4*>(wsb + L::kT1F + frag_off(t, ks, 0, lane)) =
                u32x4{hi[0][0], hi[0][1], hi[1][0], hi[1][1]};
            *reinterpret_cast<u32x4*>(wsb + L::kT1F + frag_off(t, ks, 1, lane)) =
                u32x4{lo[0][0], lo[0][1], lo[1][0], lo[1][1]};
        }
}

// Eight consecutive elements of a q/k/v row as one bf16 MFMA operand: bf16
// inputs as they are, float32 inputs rounded to nearest even.
template <bool F32>
__device__ __forceinline__ bf16x8 ld8_in(const void* base, size_t elem) {
    if constexpr (F32) {
        const float* p = static_cast<const float*>(base) + elem;
        const f32x4 a = *reinterpret_cast<const f32x4*>(p);
        const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
        return as_bf16x8(u32x4{cvt2(a[0], a[1]), cvt2(a[2], a[3]), cvt2(b[0], b[1]), cvt2(b[2], b[3])});
    } else {
        return ld16_bf16(static_cast<const uint16_t*>(base) + elem);
    }
}

// Float32 inputs: the chunk's V rows of head h as a bf16 image (zero past
// the sequence end), lane -> rows 16 t + l%16, columns 8 (l/16) + 32 c ....
// The image is stored by column block, [DV/16][64 rows][16 columns], so
// that each chain workgroup reads its block as one contiguous 2 KiB piece
// (row-major, its 32 bytes of every row shared their cache lines with the
// other column blocks, and the float32-input prefill took 4 us longer).
template <class L, int DV>
__device__ __forceinline__ void store_v_image(const void* v, char* wsb, size_t t0, int nvalid, int H,
                                              int h, int lane) {
    const int lr = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int r = 16 * t + lr;
#pragma unroll
        for (int c = 0; c < DV / 32; ++c) {
            const int d0 = 32 * c + 8 * grp;
            const bf16x8 x = r < nvalid ? ld8_in<true>(v, ((t0 + r) * H + h) * DV + d0) : zero_bf16x8();
            *reinterpret_cast<bf16x8*>(wsb + L::kVI + ((d0 / 16) * kC + r) * 32 + (d0 % 16) * 2) = x;
        }
    }
}

template <int DK, int DV, bool F32, bool SPLIT>
__global__ void __launch_bounds__(64)
prefill_prep_kernel(const void* __restrict__ q, const void* __restrict__ k,
                    const void* __restrict__ v, const float* __restrict__ g,
                    const float* __restrict__ beta, char* __restrict__ ws, SeqGeom geo, int H,
                    int Hqk, int group, bool tiled) {
    using L = WsL<DK, DV, false, F32>;
    constexpr int KS = L::KS;
    // A (fp32) during the solve, then the hi/lo transpose of T1 (bf16); a
    // barrier separates the two uses.
    __shared__ __attribute__((aligned(16))) float sA[kC][kAP];
    __shared__ float sG[kC];
    __shared__ __attribute__((aligned(16))) float sBeta[kC];

    const int lane = threadIdx.x;
    // SPLIT: two blocks per chunk, the first forming A, T1, the gate block
    // and (float32 inputs) the K and V images, the second QKm and the Q
    // image; each output takes the same instructions as in the single block
    const int blk = SPLIT ? blockIdx.x >> 1 : blockIdx.x;  // h * CT + c: workspace block of head h, chunk c
    const bool doA = !SPLIT || (blockIdx.x & 1) == 0;
    const bool doQ = !SPLIT || (blockIdx.x & 1) == 1;
    const int h = blk / geo.CT;
    const int c = blk - h * geo.CT;
    const int i = geo.owner(c);
    if (i < 0) return;  // capacity past the last sequence's chunks
    int start, len, c0, nc;
    geo.seq(i, start, len, c0, nc);
    const int n = c - c0;  // chunk of sequence i
    const int hq = qk_head(h, Hqk, group, tiled);  // the q/k head this value head reads
    const int t0 = start + n * kC;  // first token of the chunk
    const int nvalid = min(kC, len - n * kC);
    const int lr = lane & 15;  // MFMA row / column inside a tile
    const int grp = lane >> 4;
    char* wsb = ws + static_cast<size_t>(blk) * L::kBlock;

    // gates: inclusive prefix sum of the log-gates over the chunk
    float gv = 0.f, bv = 0.f;
    if (lane < nvalid) {
        const size_t bth = (static_cast<size_t>(t0) + lane) * H + h;
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
    if (doA) {
        float* e = reinterpret_cast<float*>(wsb + L::kE);
        const float Glast = __shfl(G, 63, 64);
        e[kEg + lane] = expf(G);
        e[kEr + lane] = expf(Glast - G);
        if (lane == 0) e[kEl] = expf(Glast);
        e[kEs + lane] = expf(gv);  // the token's own decay (state snapshots)
    }

    // fragments of the chunk's q and k rows (zero beyond the sequence end)
    auto row_at = [&](int r) {  // element offset of q or k row t0 + r
        return ((static_cast<size_t>(t0) + r) * Hqk + hq) * DK;
    };
    bf16x8 kf[4][KS];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int r = 16 * t + lr;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            kf[t][ks] = r < nvalid ? ld8_in<F32>(k, row_at(r) + 32 * ks + 8 * grp) : zero_bf16x8();
    }
    if constexpr (F32) {  // the bf16 K and V images for the chain
        if (doA) {
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    *reinterpret_cast<bf16x8*>(wsb + L::kKI + (static_cast<size_t>(16 * t + lr) * DK + 32 * ks + 8 * grp) * 2) =
                        kf[t][ks];
            store_v_image<L, DV>(v, wsb, t0, nvalid, H, h, lane);
        }
    }
    __syncthreads();

    // A = strict lower part of diag(beta) (exp(G_r - G_s)) o (K K^T)
    if (doA)
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
                if (col < row) a = sBeta[row] * __expf(sG[row] - sG[col]) * acc[rr];
                sA[row][col] = a;
            }
        }
    }

    if (doQ) {
    // fragments of the chunk's q rows (zero beyond the sequence end)
    bf16x8 qp[4][KS];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int r = 16 * t + lr;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qp[t][ks] = r < nvalid ? ld8_in<F32>(q, row_at(r) + 32 * ks + 8 * grp) : zero_bf16x8();
    }
    if constexpr (F32) {  // the bf16 Q image for the chain
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                *reinterpret_cast<bf16x8*>(wsb + L::kQI + (static_cast<size_t>(16 * t + lr) * DK + 32 * ks + 8 * grp) * 2) =
                    qp[t][ks];
    }

    // QKm = lower part (diagonal included) of exp(G_r - G_s) o (Q K^T), as
    // hi/lo A operands in split k order.  Each 16 x 16 tile is formed
    // transposed (K Q^T), so lane l holds row r = 16 rt + l%16 and the four
    // columns s = 16 st + 4 (l/16) + 0..3: the tiles st = 2 ks and 2 ks + 1
    // give exactly the 8 values of k-step ks in split order.
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
        const int r = 16 * rt + lr;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            if (2 * ks > rt) continue;  // above the diagonal: zero, never read
            u32x2 hi[2], lo[2];
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int st = 2 * ks + half;
                const int s0 = 16 * st + 4 * grp;
                hi[half] = u32x2{0u, 0u};
                lo[half] = u32x2{0u, 0u};
                if (st <= rt) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < KS; ++kk) acc = mfma(kf[st][kk], qp[rt][kk], acc);
                    // acc[j] = q_r . k_(s0 + j)
                    float x[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        x[j] = (s0 + j <= r) ? __expf(sG[r] - sG[s0 + j]) * acc[j] : 0.f;
                    split4(x[0], x[1], x[2], x[3], hi[half], lo[half]);
                }
            }
            *reinterpret_cast<u32x4*>(wsb + L::kQKF + frag_off(rt, ks, 0, lane)) =
                u32x4{hi[0][0], hi[0][1], hi[1][0], hi[1][1]};
            *reinterpret_cast<u32x4*>(wsb + L::kQKF + frag_off(rt, ks, 1, lane)) =
                u32x4{lo[0][0], lo[0][1], lo[1][0], lo[1][1]};
        }
    }
    }  // doQ
    if (!doA) return;
    __syncthreads();

    solve_store_t1<L>(sA, sBeta, wsb, lane);
}

// ---------------------------------------------------------------------------
// prep, KDA: the per-key-row decays enter A and QKm inside the sum over keys,
//   A[r][s]   = beta_r sum_i k_r[i] k_s[i] exp(G_r[i] - G_s[i])   (s < r)
//   QKm[r][s] =        sum_i q_r[i] k_s[i] exp(G_r[i] - G_s[i])   (s <= r)
// Each factor exp(G_r - G_s) is split at a reference row m, exp(G_r - G_m)
// exp(G_m - G_s), and the two halves scale the MFMA operands: row tile mt
// (rows 16 mt..) takes its first row m = 16 mt against every column tile.
// With decays of at most 1 (g <= 0) the row half is then at most 1, and so is
// the column half for every earlier column tile (s < m <= r): those products
// are safe for any gates, and a half that underflows belongs to a product
// that is itself below e^-87.  On the diagonal tile the column half
// exp(G_m - G_s) grows with s; while no key decays by more than e^-40 across
// the tile, it stays below e^40 and the factorised product is used.
// Otherwise the tile is formed again after the key walk, one entry at a time
// in fp32 with each entry's own decay exp(G_r - G_s) <= 1 (exact_diag_tile),
// and those entries replace the factorised ones, so the path is correct for
// every g <= 0.  The walk over the key axis goes in steps
// of 32 keys, so that only 32 of the DK gates per row are live at a time:
// the cumulative gates G of the step are an inclusive scan over the chunk's
// rows (16 lanes hold 16 rows; the totals of earlier row tiles are added).
// ---------------------------------------------------------------------------

// x + (x of the lane `off` below in the same 16-lane row; 0 for the row's
// first `off` lanes).
template <int off>
__device__ __forceinline__ float add_row_shr(float x) {
    return x + __builtin_bit_cast(
                   float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x110 + off, 0xf, 0xf, true));
}

// Inclusive prefix sum over the 16 lanes of each row of the wavefront.
__device__ __forceinline__ float scan16(float x) {
    x = add_row_shr<1>(x);
    x = add_row_shr<2>(x);
    x = add_row_shr<4>(x);
    return add_row_shr<8>(x);
}

// Eight floats -> one bf16 MFMA operand (round to nearest even).
__device__ __forceinline__ bf16x8 pack8(const float (&x)[8]) {
    return as_bf16x8(u32x4{cvt2(x[0], x[1]), cvt2(x[2], x[3]), cvt2(x[4], x[5]), cvt2(x[6], x[7])});
}

// bf16 element j of 8 packed in a u32x4.
__device__ __forceinline__ float bf16_elem(const u32x4& w, int j) {
    return __uint_as_float((j & 1) ? (w[j >> 1] & 0xffff0000u) : (w[j >> 1] << 16));
}

// Smallest decay, e^-40, that one key may take across a row tile while its
// diagonal tile still uses the factorised product (column halves below e^40).
constexpr float kExactMin = 4.248354255291589e-18f;
// Diagonal tile mt of A and QKm over keys 32 ks .. 32 ks + 31, one entry at a
// time in fp32 with each entry's exact decay exp(G_r - G_s) <= 1.  Lane
// (lr, grp) holds row 16 mt + lr at keys 32 ks + 8 grp + 0..7 and takes the
// other rows' keys from the lanes of its 16-lane row.  It adds, over its
// eight keys, P[s] = sum k_r k_s exp(-|G_r - G_s|) and Q[s] = sum q_r k_s
// exp(-|G_r - G_s|) for r = 16 mt + lr and every row s = 16 mt + 0..15 of the
// tile: P[s] is A[max(r,s)][min(r,s)] / beta and, for s <= r, Q[s] is
// QKm[r][s] (with g <= 0 the row further down has the smaller G).  Only
// differences of G inside the tile enter, so the gates are summed from the
// tile's first row.  The inputs are read again (they are in L2).
template <int DK, bool F32>
__device__ __forceinline__ void exact_diag_tile(const void* q, const void* k, const float* g, int t0,
                                                int nvalid, int H, int h, int Hqk, int hq, int mt,
                                                int ks, float (&P)[16], float (&Q)[16], int lane) {
    const int lr = lane & 15, grp = lane >> 4;
    const int r = 16 * mt + lr;
    const int d0 = 32 * ks + 8 * grp;
    float gl[8], kk[8], qv[8];
    if (r < nvalid) {
        const size_t tok = static_cast<size_t>(t0) + r;
        const f32x4 g0 = *reinterpret_cast<const f32x4*>(g + (tok * H + h) * DK + d0);
        const f32x4 g1 = *reinterpret_cast<const f32x4*>(g + (tok * H + h) * DK + d0 + 4);
        const u32x4 kb = __builtin_bit_cast(u32x4, ld8_in<F32>(k, (tok * Hqk + hq) * DK + d0));
        const u32x4 qb = __builtin_bit_cast(u32x4, ld8_in<F32>(q, (tok * Hqk + hq) * DK + d0));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            gl[j] = g0[j];
            gl[4 + j] = g1[j];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            kk[j] = bf16_elem(kb, j);
            qv[j] = bf16_elem(qb, j);
        }
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) gl[j] = kk[j] = qv[j] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) gl[j] = scan16(gl[j]);  // cumulative over the tile's rows

#pragma unroll
    for (int s = 0; s < 16; ++s) {
        const int src = (lane & 48) | s;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float ksj = __shfl(kk[j], src, 64);
            const float gsj = __shfl(gl[j], src, 64);
            const float t = ksj * __expf(-fabsf(gl[j] - gsj));
            P[s] = fmaf(t, kk[j], P[s]);
            Q[s] = fmaf(t, qv[j], Q[s]);
        }
    }
}

template <int DK, int DV, bool F32>
__global__ void __launch_bounds__(64)
prefill_prep_kda_kernel(const void* __restrict__ q, const void* __restrict__ k,
                        const void* __restrict__ v, const float* __restrict__ g,
                        const float* __restrict__ beta, char* __restrict__ ws, SeqGeom geo, int H,
                        int Hqk, int group, bool tiled) {
    using L = WsL<DK, DV, true, F32>;
    constexpr int KS = DK / 32;
    __shared__ __attribute__((aligned(16))) float sA[kC][kAP];
    __shared__ __attribute__((aligned(16))) float sBeta[kC];

    const int lane = threadIdx.x;
    const int blk = blockIdx.x;  // h * CT + c: workspace block of head h, chunk c
    const int h = blk / geo.CT;
    const int c = blk - h * geo.CT;
    const int i = geo.owner(c);
    if (i < 0) return;  // capacity past the last sequence's chunks
    int start, len, c0, nc;
    geo.seq(i, start, len, c0, nc);
    const int n = c - c0;
    const int hq = qk_head(h, Hqk, group, tiled);
    const int t0 = start + n * kC;
    const int nvalid = min(kC, len - n * kC);
    const int lr = lane & 15;
    const int grp = lane >> 4;
    char* wsb = ws + static_cast<size_t>(blk) * L::kBlock;

    sBeta[lane] = lane < nvalid ? beta[(static_cast<size_t>(t0) + lane) * H + h] : 0.f;
    if constexpr (F32) store_v_image<L, DV>(v, wsb, t0, nvalid, H, h, lane);

    // pair p = mt (mt + 1) / 2 + nt of row tile mt and column tile nt <= mt
    f32x4 accA[10], accQ[10];
#pragma unroll
    for (int p = 0; p < 10; ++p) {
        accA[p] = f32x4{0.f, 0.f, 0.f, 0.f};
        accQ[p] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float* E = reinterpret_cast<float*>(wsb + L::kE);
    // sA is free until A is formed: the transpose of one step's K o exp(G_last - G),
    // [32 keys][64 rows] bf16, rows padded to 72 so that the fragment reads
    // (16 keys x 8 bytes) meet distinct banks
    uint16_t (*sKT)[72] = reinterpret_cast<uint16_t (*)[72]>(&sA[0][0]);

    uint32_t exact_tiles = 0;  // bit mt: diagonal tile mt is formed by exact_diag_tile
#pragma unroll 1
    for (int ks = 0; ks < KS; ++ks) {
        // this lane: keys d0 + 0..7 of rows 16 t + lr
        const int d0 = 32 * ks + 8 * grp;
        float G[4][8];
        u32x4 kb[4], qb[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int r = 16 * t + lr;
            if (r < nvalid) {
                const size_t tok = static_cast<size_t>(t0) + r;
                const f32x4 g0 = *reinterpret_cast<const f32x4*>(g + (tok * H + h) * DK + d0);
                const f32x4 g1 = *reinterpret_cast<const f32x4*>(g + (tok * H + h) * DK + d0 + 4);
                kb[t] = __builtin_bit_cast(u32x4, ld8_in<F32>(k, (tok * Hqk + hq) * DK + d0));
                qb[t] = __builtin_bit_cast(u32x4, ld8_in<F32>(q, (tok * Hqk + hq) * DK + d0));
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    G[t][j] = g0[j];
                    G[t][4 + j] = g1[j];
                }
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) G[t][j] = 0.f;
                kb[t] = u32x4{0u, 0u, 0u, 0u};
                qb[t] = u32x4{0u, 0u, 0u, 0u};
            }
        }
        // cumulative gates over the chunk's rows
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float carry = 0.f;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                G[t][j] = scan16(G[t][j]) + carry;
                carry = __shfl(G[t][j], (lane & 48) | 15, 64);  // through the tile's last row
            }
        }
        float GL[8];  // G at the chunk's last row (rows past the sequence add 0)
#pragma unroll
        for (int j = 0; j < 8; ++j) GL[j] = __shfl(G[3][j], (lane & 48) | 15, 64);

        // the decayed images for the chain; K o exp(G_last - G) goes through
        // sKT (the key-major transpose of this step's 32 keys) into the state
        // update's operand fragments
        __syncthreads();  // the previous step's reads of sKT are done
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            float a[8], b[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float eg = __expf(G[t][j]);
                a[j] = bf16_elem(kb[t], j) * eg;
                b[j] = bf16_elem(qb[t], j) * eg;
                const float dk = bf16_elem(kb[t], j) * __expf(GL[j] - G[t][j]);
                sKT[8 * grp + j][16 * t + lr] = static_cast<uint16_t>(cvt2(dk, 0.f) & 0xffffu);
            }
            const size_t off = (static_cast<size_t>(16 * t + lr) * DK + d0) * 2;
            *reinterpret_cast<bf16x8*>(wsb + L::kKG + off) = pack8(a);
            *reinterpret_cast<bf16x8*>(wsb + L::kQG + off) = pack8(b);
        }
        __syncthreads();
#pragma unroll
        for (int k16 = 0; k16 < 2; ++k16) {  // keys 32 ks + 16 k16 + lr
            const int i0 = 32 * ks + 16 * k16;
            const int w = i0 / (DK / 4), mt = (i0 % (DK / 4)) / 16;  // the state wavefront and tile
#pragma unroll
            for (int ks2 = 0; ks2 < 2; ++ks2) {
                const uint16_t* src = &sKT[16 * k16 + lr][32 * ks2 + 4 * grp];
                const u32x2 lo4 = *reinterpret_cast<const u32x2*>(src);
                const u32x2 hi4 = *reinterpret_cast<const u32x2*>(src + 16);
                *reinterpret_cast<u32x4*>(wsb + L::kKDF + ((((w * (DK / 64) + mt) * 2 + ks2) * 64 + lane) * 16)) =
                    u32x4{lo4[0], lo4[1], hi4[0], hi4[1]};
            }
        }
        if (lr == 0) {
            float el[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) el[j] = __expf(GL[j]);
            *reinterpret_cast<f32x4*>(E + kEv + d0) = f32x4{el[0], el[1], el[2], el[3]};
            *reinterpret_cast<f32x4*>(E + kEv + d0 + 4) = f32x4{el[4], el[5], el[6], el[7]};
        }

        // A and QKm contributions of these 32 keys
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            float ref[8], x[8], y[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) ref[j] = __shfl(G[mt][j], lane & 48, 64);
            float emin = 1.f;  // this lane's smallest row half: its decay from the tile's first row
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float e = __expf(G[mt][j] - ref[j]);
                emin = fminf(emin, e);
                x[j] = bf16_elem(kb[mt], j) * e;
                y[j] = bf16_elem(qb[mt], j) * e;
            }
            // beyond the factorised range the diagonal tile's product below
            // is discarded and the tile is formed by exact_diag_tile
            exact_tiles |= static_cast<uint32_t>(__any(emin < kExactMin)) << mt;
            const bf16x8 a = pack8(x);
            const bf16x8 qa = pack8(y);
#pragma unroll
            for (int nt = 0; nt <= mt; ++nt) {
                float z[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) z[j] = bf16_elem(kb[nt], j) * __expf(ref[j] - G[nt][j]);
                const bf16x8 b = pack8(z);
                const int p = mt * (mt + 1) / 2 + nt;
                accA[p] = mfma(a, b, accA[p]);   // rows 16 mt + 4 grp + .., column 16 nt + lr
                accQ[p] = mfma(b, qa, accQ[p]);  // transposed: row 16 mt + lr, columns 16 nt + 4 grp + ..
            }
        }
    }
    __syncthreads();  // sBeta

    // A (strict lower part, rows scaled by beta) to LDS
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt <= mt; ++nt) {
            const f32x4 acc = accA[mt * (mt + 1) / 2 + nt];
            const int col = 16 * nt + lr;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int row = 16 * mt + 4 * grp + rr;
                sA[row][col] = col < row ? sBeta[row] * acc[rr] : 0.f;
            }
        }

    // QKm (diagonal included) as hi/lo A operands in split k order, as for GDA
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
        const int r = 16 * rt + lr;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            if (2 * ks > rt) continue;  // above the diagonal: zero, never read
            u32x2 hi[2], lo[2];
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int st = 2 * ks + half;
                const int s0 = 16 * st + 4 * grp;
                hi[half] = u32x2{0u, 0u};
                lo[half] = u32x2{0u, 0u};
                if (st <= rt) {
                    const f32x4 acc = accQ[rt * (rt + 1) / 2 + st];
                    float x[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) x[j] = (s0 + j <= r) ? acc[j] : 0.f;
                    split4(x[0], x[1], x[2], x[3], hi[half], lo[half]);
                }
            }
            *reinterpret_cast<u32x4*>(wsb + L::kQKF + frag_off(rt, ks, 0, lane)) =
                u32x4{hi[0][0], hi[0][1], hi[1][0], hi[1][1]};
            *reinterpret_cast<u32x4*>(wsb + L::kQKF + frag_off(rt, ks, 1, lane)) =
                u32x4{lo[0][0], lo[0][1], lo[1][0], lo[1][1]};
        }
    }

    // Diagonal tiles with decays beyond the factorised range: formed anew over
    // all keys, and written over the entries the factorised products gave.
    // The lane index is read again here, so that no lane-dependent value of
    // the key walk stays live through the walk for this rarely taken pass:
    // the walk needs the whole 256-register budget of two wavefronts per SIMD.
    const int xl = static_cast<int>(__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)));
#pragma unroll 1
    for (int mt = 0; mt < 4; ++mt) {
        if (!((exact_tiles >> mt) & 1u)) continue;
        float P[16], Q[16];
#pragma unroll
        for (int s = 0; s < 16; ++s) P[s] = Q[s] = 0.f;
#pragma unroll 1
        for (int ks = 0; ks < KS; ++ks) exact_diag_tile<DK, F32>(q, k, g, t0, nvalid, H, h, Hqk, hq, mt, ks, P, Q, xl);
#pragma unroll
        for (int s = 0; s < 16; ++s) {  // the sums over the four key groups
            P[s] += __shfl_xor(P[s], 16, 64);
            P[s] += __shfl_xor(P[s], 32, 64);
            Q[s] += __shfl_xor(Q[s], 16, 64);
            Q[s] += __shfl_xor(Q[s], 32, 64);
        }
        // this lane's entries in the layouts of the writes above: A rows
        // 16 mt + 4 xg + j of column 16 mt + xr, QKm row 16 mt + xr, columns
        // 16 mt + 4 xg + j
        const int xr = xl & 15, xg = xl >> 4;
        float pa[4], pq[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            pa[j] = xg == 0 ? P[j] : xg == 1 ? P[4 + j] : xg == 2 ? P[8 + j] : P[12 + j];
            pq[j] = xg == 0 ? Q[j] : xg == 1 ? Q[4 + j] : xg == 2 ? Q[8 + j] : Q[12 + j];
        }
        const int col = 16 * mt + xr;
        float x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = 16 * mt + 4 * xg + j;
            sA[row][col] = col < row ? sBeta[row] * pa[j] : 0.f;
            x[j] = 4 * xg + j <= xr ? pq[j] : 0.f;
        }
        u32x2 hi, lo;
        split4(x[0], x[1], x[2], x[3], hi, lo);
        const int half = (mt & 1) * 8;  // the diagonal tile's half of the split-order fragment
        *reinterpret_cast<u32x2*>(wsb + L::kQKF + frag_off(mt, mt >> 1, 0, xl) + half) = hi;
        *reinterpret_cast<u32x2*>(wsb + L::kQKF + frag_off(mt, mt >> 1, 1, xl) + half) = lo;
    }
    __syncthreads();
    solve_store_t1<L>(sA, sBeta, wsb, lane);
}

// ---------------------------------------------------------------------------
// chain: one workgroup (two wavefronts) per (sequence, head, 16-column block)
// ---------------------------------------------------------------------------

// LDS image of a K chunk: row-major [64][DK] bf16 with the 16-byte pieces of
// row r permuted by an XOR with sw(r), so that both the row reads of the
// X = K S operand (16 rows, one piece each) and the transposing reads of the
// K^T operand (8 rows, two adjacent pieces each) touch every bank once.
template <int DK>
__device__ __forceinline__ int k_swz(int r) {
    if constexpr (DK == 128) return ((r & 7) << 1) | ((r >> 3) & 1);
    else return (((r >> 1) & 3) << 1) | ((r >> 3) & 1);
}
// Element offset of (r, c) in the K image, c a multiple of 4.
template <int DK>
__device__ __forceinline__ int k_at(int r, int c) {
    return r * DK + 8 * ((c >> 3) ^ k_swz<DK>(r)) + (c & 7);
}

// Direct-to-LDS load of 16 bytes per lane: lane l's bytes land at
// lds + 16 l (lds must be the same for the whole wavefront).  Loads past the
// end of the resource write zeros.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* lds, int voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff,
                                             0, 0, 0);
}

// LDS layout of the chain kernel.  A ring of slots holds, for consecutive
// chunks, the operands that arrive as whole rows: the gate block as it is in
// the workspace and the K and Q images (k_at layout).  Loader wavefronts fill
// the slot of chunk n + kAhead while the others compute on chunk n.  Operands
// that one wavefront reads alone (its T1 or QKm rows in fragment order, the
// state lanes' V values) go straight from memory to its registers.
// KDA: the K and Q images are the decayed images KG and QG of the
// workspace (the state update's K^T operand goes from the workspace straight
// to the state wavefronts' registers).
//
// Four slots: the loads of a chunk go out three chunks ahead of its use,
// which covers the latency of the direct-to-LDS loads from memory; the V
// block (four values per state lane) goes to registers instead, so that
// four slots fit.
template <int DK, bool KDA>
struct ChainLds {
    static constexpr int kImages = 2;
    static constexpr int kE = 0;                           // gate block (Ws<DK>::kE layout)
    static constexpr int kK = kE + 1024;                   // K image (KDA: KG)
    static constexpr int kQ = kK + kC * DK * 2;            // Q image (KDA: QG)
    static constexpr int kSlot = kK + kImages * kC * DK * 2;
    static constexpr int kLoads = 1 + kImages * (kC * DK * 2 / 1024);  // 1 KiB loads per chunk
    static constexpr int kRing = 4;
    static constexpr int kAhead = kRing - 1;  // chunks loaded ahead of the one in use
};

constexpr int kStateWaves = 4;   // chunk rows 16 w.., state rows (d_k / 4) w..
constexpr int kOutWaves = 4;     // chunk rows 16 w.. of the output
constexpr int kLoadWaves = 4;
constexpr int kChainThreads = 64 * (kStateWaves + kOutWaves + kLoadWaves + 1);  // + the storer

// Two 8-byte LDS reads -> one split-order operand (k = c + 0..3 and c + 16 + 0..3).
__device__ __forceinline__ bf16x8 ld_split(const uint16_t* p0, const uint16_t* p1) {
    return join(*reinterpret_cast<const u32x2*>(p0), *reinterpret_cast<const u32x2*>(p1));
}

template <int DK, int DV, bool KDA, bool F32>
__global__ void __launch_bounds__(kChainThreads)
prefill_chain_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                     const uint16_t* __restrict__ v, float* __restrict__ state,
                     float* __restrict__ o, const char* __restrict__ ws, SeqGeom geo, int H,
                     int Hqk, int group, bool tiled, int K, float* __restrict__ final_state,
                     const void* __restrict__ k_in, const float* __restrict__ g,
                     const int32_t* __restrict__ accepted, int32_t* __restrict__ err_flag) {
    using L = WsL<DK, DV, KDA, F32>;
    using M = ChainLds<DK, KDA>;
    // K and Q come from the workspace's images for KDA and for float32
    // inputs, V for float32 inputs; otherwise straight from the bf16 inputs
    constexpr bool kImgKQ = KDA || F32;
    constexpr int kRing = M::kRing;
    constexpr int NCB = DV / 16;       // column blocks per head
    constexpr int KS = L::KS;          // k-steps over d_k
    constexpr int SRW = DK / 4;        // state rows per state wavefront
    constexpr int SMT = SRW / 16;      // state tiles per state wavefront
    constexpr int PPR = DK / 8;        // 16-byte pieces per K row
    constexpr int KPT = kC * PPR / 64; // 1 KiB loads of the K image
    constexpr int SLD = DK + 8;        // padded row of sS (bf16)
    constexpr int CLD = kC + 8;        // padded row of sR, sW, sWp (bf16)
    constexpr int OLD = 20;            // padded row of sO (fp32)

    __shared__ __attribute__((aligned(16))) char sL[kRing][M::kSlot];
    __shared__ __attribute__((aligned(16))) uint16_t sS[16][SLD];       // chunk start state, [col][d_k]
    __shared__ __attribute__((aligned(16))) uint16_t sR[2][16][CLD];    // R hi/lo, [col][chunk row]
    __shared__ __attribute__((aligned(16))) uint16_t sW[2][16][CLD];    // W hi/lo
    __shared__ __attribute__((aligned(16))) uint16_t sWp[2][16][CLD];   // W' = exp(G_last - G) W hi/lo
    __shared__ __attribute__((aligned(16))) float sO[kC][OLD];           // the chunk's output block
    __shared__ __attribute__((aligned(16))) uint16_t sV[kStateWaves][16][16];  // V rows of each state wavefront

    const int lane = threadIdx.x & 63;
    // the role of a wavefront is uniform across it: keep it in a scalar
    // register so that the roles are separate branches of the program
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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
    const int b = bh / H;  // the sequence
    const int h = bh - b * H;
    const int col = cb * 16 + lr;
    int start, len, c0, NC;
    geo.seq(b, start, len, c0, NC);
    if (NC == 0) return;  // an empty sequence leaves its state as it is
    const char* wsh = ws + (static_cast<size_t>(h) * geo.CT + c0) * L::kBlock;
    auto ws_rsrc = [&](int n) { return make_rsrc(wsh + static_cast<size_t>(n) * L::kBlock, L::kBlock); };

    if (wave < kStateWaves) {
        // ======================= state wavefronts ==========================
        const int w = wave;
        // slot 0 of the sequence's K slots holds the start state; slots
        // 1..nsnap receive the state after that many tokens, and the final
        // state goes back to slot 0 when K == 1, else to final_state (if given)
        float* st = state + static_cast<size_t>(bh) * K * DK * DV;
        float* fin = K == 1 ? st : (final_state ? final_state + static_cast<size_t>(bh) * DK * DV : nullptr);
        const int nsnap = K > 1 ? min(len, K - 1) : 0;
        // the input state: slot 0, or after a rollback fused into this call
        // the accepted slot (an invalid index is flagged, as by the rollback,
        // and the sequence starts from slot 0)
        int src = 0;
        if (accepted != nullptr) {
            const int a = accepted[b];
            if (a >= 0 && a < K)
                src = a;
            else if (h == 0 && cb == 0 && w == 0 && lane == 0 && err_flag != nullptr)
                atomicOr(err_flag, 1);
        }
        const float* s_in = st + static_cast<size_t>(src) * DK * DV;
        // tile mt: d_k rows SRW w + 16 mt + 4 grp + 0..3 of column `col`
        f32x4 S[SMT];
#pragma unroll
        for (int mt = 0; mt < SMT; ++mt)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                S[mt][rr] = s_in[static_cast<size_t>(SRW * w + 16 * mt + 4 * grp + rr) * DV + col];
        if (src != 0) {
            // the rollback itself: slot 0 <- slot src for this wavefront's
            // rows and this workgroup's columns (the only ones it reads or
            // writes; the snapshot slots are written after the first chunk's
            // third barrier)
#pragma unroll
            for (int mt = 0; mt < SMT; ++mt)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                    st[static_cast<size_t>(SRW * w + 16 * mt + 4 * grp + rr) * DV + col] = S[mt][rr];
        }
        auto publish_state = [&]() {  // bf16 state rows -> sS (B operand of K S and Q S)
#pragma unroll
            for (int mt = 0; mt < SMT; ++mt)
                *reinterpret_cast<u32x2*>(&sS[lr][SRW * w + 16 * mt + 4 * grp]) =
                    to_bf16x4(S[mt][0], S[mt][1], S[mt][2], S[mt][3]);
        };
        // T1 rows 16 w.. of a chunk, hi/lo, split k order (read by this wavefront only)
        bf16x8 t1[2][2];
        auto load_t1 = [&](int n) {
            const __amdgpu_buffer_rsrc_t rw = ws_rsrc(n);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                if (2 * ks > w) continue;  // T1 is zero there (and not stored)
#pragma unroll
                for (int hl = 0; hl < 2; ++hl)
                    t1[ks][hl] = as_bf16x8(buf_ld16(rw, L::kT1F + frag_off(w, ks, hl, lane)));
            }
        };
        load_t1(0);
        // The wavefront's 16 rows of V of a chunk in one 8-byte load per
        // lane: row 16 w + l/4, columns 4 (l%4) + 0..3 of the column block
        // (zero past the sequence end).  Staged through sV, a transposing read
        // gives each lane its rows 16 w + 4 grp + 0..3 at column `col`.
        u32x2 vr;
        auto load_v = [&](int n) {
            const int r0 = n * kC;
            __amdgpu_buffer_rsrc_t rv;
            int rowb, off0;
            if constexpr (F32) {  // the workspace's bf16 V image, this column block's piece
                rv = ws_rsrc(n);
                rowb = 32;
                off0 = L::kVI + cb * kC * 32;
            } else {
                const int row_b16 = H * DV * 2;
                rv = make_rsrc(v + (static_cast<size_t>(start + r0) * H + h) * DV,
                               (len - 1 - r0) * row_b16 + DV * 2);
                rowb = row_b16;
                off0 = cb * 32;
            }
            vr = __builtin_bit_cast(
                u32x2, __builtin_amdgcn_raw_buffer_load_b64(rv, off0 + 8 * (lane & 3) + (16 * w + (lane >> 2)) * rowb, 0, 0));
        };
        load_v(0);
        bf16x8 kt[SMT][2];
        // KDA: the state update's K^T operands, in fragment order in the workspace
        auto load_kt = [&](int n) {
            const __amdgpu_buffer_rsrc_t rw = ws_rsrc(n);
#pragma unroll
            for (int mt = 0; mt < SMT; ++mt)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    kt[mt][ks] = as_bf16x8(
                        buf_ld16(rw, WsKda<DK>::kKDF + (((w * SMT + mt) * 2 + ks) * 64 + lane) * 16));
        };
        if constexpr (KDA) load_kt(0);
        publish_state();

        for (int n = 0; n < NC; ++n) {
            const char* slot = sL[n % kRing];
            const uint16_t* sK = reinterpret_cast<const uint16_t*>(slot + M::kK);
            const float* E = reinterpret_cast<const float*>(slot + M::kE);
            lds_barrier();  // B1: chunk n's operands and start state are in LDS

            // X = K S for chunk rows 16 w + l%16 (split k order over d_k)
            f32x4 X = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int c = 32 * ks + 4 * grp;
                const int r = 16 * w + lr;
                X = mfma(ld_split(&sK[k_at<DK>(r, c)], &sK[k_at<DK>(r, c + 16)]),
                         ld_split(&sS[lr][c], &sS[lr][c + 16]), X);
            }
            // GDA: exp(G_r) for the rows of X, exp(G_last - G_r) for W', and
            // exp(G_last) for S; KDA: exp(G_last[i]) for this wavefront's state rows
            f32x4 eg = {1.f, 1.f, 1.f, 1.f}, er = {1.f, 1.f, 1.f, 1.f};
            float el = 1.f;
            f32x4 egl[SMT];
            if constexpr (KDA) {
#pragma unroll
                for (int mt = 0; mt < SMT; ++mt)
                    egl[mt] = *reinterpret_cast<const f32x4*>(&E[kEv + SRW * w + 16 * mt + 4 * grp]);
            } else {
                eg = *reinterpret_cast<const f32x4*>(&E[kEg + 16 * w + 4 * grp]);
                er = *reinterpret_cast<const f32x4*>(&E[kEr + 16 * w + 4 * grp]);
                el = E[kEl];
            }

            // R = V - exp(G) X (KDA: V - X, the decay is inside KG) for this
            // wavefront's rows, hi/lo to LDS
            {
                // sV[w] is this wavefront's alone: its previous reads came
                // before these writes in program order
                uint16_t* const pv = &sV[w][0][0] + 4 * lane;  // row l/4, columns 4 (l%4)..
                *reinterpret_cast<u32x2*>(pv) = vr;
                const u32x2 vt = ld_tr(pv);
                u32x2 rh, rl;
                split4(__uint_as_float(vt[0] << 16) - eg[0] * X[0],
                       __uint_as_float(vt[0] & 0xffff0000u) - eg[1] * X[1],
                       __uint_as_float(vt[1] << 16) - eg[2] * X[2],
                       __uint_as_float(vt[1] & 0xffff0000u) - eg[3] * X[3], rh, rl);
                *reinterpret_cast<u32x2*>(&sR[0][lr][16 * w + 4 * grp]) = rh;
                *reinterpret_cast<u32x2*>(&sR[1][lr][16 * w + 4 * grp]) = rl;
            }
            lds_barrier();  // B2: all of R is in LDS

            // W = T1 R for rows 16 w + l%16 (three hi/lo products, split k
            // order; T1 is zero above the diagonal)
            f32x4 W = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                if (2 * ks > w) continue;
                const int c = 32 * ks + 4 * grp;
                const bf16x8 rh = ld_split(&sR[0][lr][c], &sR[0][lr][c + 16]);
                const bf16x8 rl = ld_split(&sR[1][lr][c], &sR[1][lr][c + 16]);
                W = mfma(t1[ks][0], rh, W);
                W = mfma(t1[ks][0], rl, W);
                W = mfma(t1[ks][1], rh, W);
            }
            load_t1(min(n + 1, NC - 1));  // t1 is not read again in this chunk
            load_v(min(n + 1, NC - 1));   // nor vr (it is in sV)
            // K^T operands of the state update (d_k rows SRW w + 16 mt + l%16,
            // chunk rows in split order), read while W forms (KDA: loaded
            // during the previous chunk)
            if constexpr (!KDA) {
#pragma unroll
                for (int mt = 0; mt < SMT; ++mt)
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) {
                        const int r = 32 * ks + 4 * grp + (lr >> 2);
                        const int cc = SRW * w + 16 * mt + 4 * (lr & 3);
                        kt[mt][ks] = join(ld_tr(&sK[k_at<DK>(r, cc)]), ld_tr(&sK[k_at<DK>(r + 16, cc)]));
                    }
            }
            {
                u32x2 wh, wl, ph, pl;
                split4(W, wh, wl);
                *reinterpret_cast<u32x2*>(&sW[0][lr][16 * w + 4 * grp]) = wh;
                *reinterpret_cast<u32x2*>(&sW[1][lr][16 * w + 4 * grp]) = wl;
                if constexpr (!KDA) {  // KDA: the decay to the chunk end is inside KD
                    split4(er[0] * W[0], er[1] * W[1], er[2] * W[2], er[3] * W[3], ph, pl);
                    *reinterpret_cast<u32x2*>(&sWp[0][lr][16 * w + 4 * grp]) = ph;
                    *reinterpret_cast<u32x2*>(&sWp[1][lr][16 * w + 4 * grp]) = pl;
                }
            }
            lds_barrier();  // B3: all of W and W' are in LDS

            // Snapshots inside this chunk: row r of W is token r's delta
            // beta (v - u), so the token recurrence S <- exp(g_r) S + k_r w_r^T,
            // run from the chunk's start state, gives the state after each
            // token.  K image and W stay in LDS until the next chunk's B1.
            if (!KDA && n * kC < nsnap) {
                const int rn = min(kC, nsnap - n * kC);
                f32x4 X[SMT];
#pragma unroll
                for (int mt = 0; mt < SMT; ++mt) X[mt] = S[mt];
                for (int r = 0; r < rn; ++r) {
                    const float a = E[kEs + r];
                    const float wv = __uint_as_float(static_cast<uint32_t>(sW[0][lr][r]) << 16) +
                                     __uint_as_float(static_cast<uint32_t>(sW[1][lr][r]) << 16);
                    float* dst = st + static_cast<size_t>(n * kC + r + 1) * DK * DV;
#pragma unroll
                    for (int mt = 0; mt < SMT; ++mt) {
                        const int i0 = SRW * w + 16 * mt + 4 * grp;
                        const u32x2 kk = *reinterpret_cast<const u32x2*>(&sK[k_at<DK>(r, i0)]);
                        const float kv[4] = {__uint_as_float(kk[0] << 16), __uint_as_float(kk[0] & 0xffff0000u),
                                             __uint_as_float(kk[1] << 16), __uint_as_float(kk[1] & 0xffff0000u)};
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr) {
                            X[mt][rr] = fmaf(kv[rr], wv, a * X[mt][rr]);
                            dst[static_cast<size_t>(i0 + rr) * DV + col] = X[mt][rr];
                        }
                    }
                }
            }

            // KDA snapshots start from the chunk's start state (below)
            f32x4 Y[KDA ? SMT : 1];
            if (KDA && n * kC < nsnap) {
#pragma unroll
                for (int mt = 0; mt < SMT; ++mt) Y[mt] = S[mt];
            }

            // S <- exp(G_last) S + K^T W' for this wavefront's state rows
            // (KDA: S[i,:] <- exp(G_last[i]) S[i,:] + KD^T W)
#pragma unroll
            for (int mt = 0; mt < SMT; ++mt)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) S[mt][rr] *= KDA ? egl[mt][rr] : el;
            uint16_t (*const sU)[16][CLD] = KDA ? sW : sWp;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int c = 32 * ks + 4 * grp;
                const bf16x8 ph = ld_split(&sU[0][lr][c], &sU[0][lr][c + 16]);
                const bf16x8 pl = ld_split(&sU[1][lr][c], &sU[1][lr][c + 16]);
#pragma unroll
                for (int mt = 0; mt < SMT; ++mt) {
                    S[mt] = mfma(kt[mt][ks], ph, S[mt]);
                    S[mt] = mfma(kt[mt][ks], pl, S[mt]);
                }
            }
            // (the KDA snapshots run after the update, when its K^T operands
            // are dead: with them live the leg spilled at d_k = 128)
            // KDA: each state row decays by its own exp(g_r[i]), and the
            // chunk's images hold decayed keys, so the token's key values and
            // log-gates at this lane's state rows come from the inputs,
            // kSnapBatch tokens at a time (the key values rounded to bf16 as
            // everywhere on this path).
            if (KDA && n * kC < nsnap) {
                constexpr int kSnapBatch = 2;  // four spilled at d_k = 128
                constexpr int EB = F32 ? 4 : 2;  // bytes per key value
                const int rn = min(kC, nsnap - n * kC);
                const int hq = qk_head(h, Hqk, group, tiled);
                const size_t tok0 = static_cast<size_t>(start) + n * kC;
                // Buffer views of the chunk's gates and keys and of its
                // snapshot slots, so that the lane's offsets are 32-bit
                // (4 grp rows in, column `col`) and the rest is scalar.
                const __amdgpu_buffer_rsrc_t rg = make_rsrc(g + (tok0 * H + h) * DK, ((rn - 1) * H + 1) * DK * 4);
                const __amdgpu_buffer_rsrc_t rk =
                    make_rsrc(static_cast<const char*>(k_in) + (tok0 * Hqk + hq) * DK * EB, ((rn - 1) * Hqk + 1) * DK * EB);
                const __amdgpu_buffer_rsrc_t rs = make_rsrc(st + static_cast<size_t>(n * kC + 1) * DK * DV, rn * DK * DV * 4);
                for (int r0 = 0; r0 < rn; r0 += kSnapBatch) {
                    f32x4 kv[kSnapBatch][SMT], ag[kSnapBatch][SMT];
#pragma unroll
                    for (int j = 0; j < kSnapBatch; ++j) {
                        const int r = min(r0 + j, rn - 1);
#pragma unroll
                        for (int mt = 0; mt < SMT; ++mt) {
                            const int i0s = SRW * w + 16 * mt;  // + 4 grp in the lane's offset
                            ag[j][mt] = __builtin_bit_cast(
                                f32x4, __builtin_amdgcn_raw_buffer_load_b128(rg, 16 * grp, (r * H * DK + i0s) * 4, 0));
                            const int ko = (r * Hqk * DK + i0s) * EB;
                            if constexpr (F32) {
                                const f32x4 x =
                                    __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, 16 * grp, ko, 0));
                                const uint32_t lo = cvt2(x[0], x[1]), hi = cvt2(x[2], x[3]);
                                kv[j][mt] = f32x4{__uint_as_float(lo << 16), __uint_as_float(lo & 0xffff0000u),
                                                  __uint_as_float(hi << 16), __uint_as_float(hi & 0xffff0000u)};
                            } else {
                                const u32x2 x =
                                    __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rk, 8 * grp, ko, 0));
                                kv[j][mt] = f32x4{__uint_as_float(x[0] << 16), __uint_as_float(x[0] & 0xffff0000u),
                                                  __uint_as_float(x[1] << 16), __uint_as_float(x[1] & 0xffff0000u)};
                            }
                        }
                    }
#pragma unroll
                    for (int j = 0; j < kSnapBatch; ++j) {
                        const int r = r0 + j;
                        if (r >= rn) break;
                        const float wv = __uint_as_float(static_cast<uint32_t>(sW[0][lr][r]) << 16) +
                                         __uint_as_float(static_cast<uint32_t>(sW[1][lr][r]) << 16);
#pragma unroll
                        for (int mt = 0; mt < SMT; ++mt) {
#pragma unroll
                            for (int rr = 0; rr < 4; ++rr) {
                                Y[mt][rr] = fmaf(kv[j][mt][rr], wv, __expf(ag[j][mt][rr]) * Y[mt][rr]);
                                // slot n kC + r + 1, state row SRW w + 16 mt + 4 grp + rr, column col
                                __builtin_amdgcn_raw_buffer_store_b32(
                                    __float_as_uint(Y[mt][rr]), rs, (4 * grp * DV + col) * 4,
                                    (r * DK * DV + (SRW * w + 16 * mt + rr) * DV) * 4, 0);
                            }
                        }
                    }
                }
            }
            if constexpr (KDA) load_kt(min(n + 1, NC - 1));  // kt is not read again in this chunk
            // sS was last read before B2 (by every wavefront)
            publish_state();
        }
        lds_barrier();  // final barrier, matched by every wavefront

        if (fin != nullptr) {
#pragma unroll
            for (int mt = 0; mt < SMT; ++mt)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                    fin[static_cast<size_t>(SRW * w + 16 * mt + 4 * grp + rr) * DV + col] = S[mt][rr];
        }
        return;
    }
    if (wave < kStateWaves + kOutWaves) {
        // ====================== output wavefronts ==========================
        const int w = wave - kStateWaves;
        // QKm rows 16 w.. hi/lo, split k order (read by this wavefront only)
        bf16x8 qk[2][2];
        auto load_q = [&](int n) {
            const __amdgpu_buffer_rsrc_t rw = ws_rsrc(n);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                if (2 * ks > w) continue;  // QKm is zero there (and not read)
#pragma unroll
                for (int hl = 0; hl < 2; ++hl)
                    qk[ks][hl] = as_bf16x8(buf_ld16(rw, L::kQKF + frag_off(w, ks, hl, lane)));
            }
        };
        load_q(0);
        for (int n = 0; n < NC; ++n) {
            const char* slot = sL[n % kRing];
            const uint16_t* sQ = reinterpret_cast<const uint16_t*>(slot + M::kQ);
            const float* E = reinterpret_cast<const float*>(slot + M::kE);
            lds_barrier();  // B1
            // P = Q S for chunk rows 16 w + l%16 (split k order over d_k)
            f32x4 P = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int c = 32 * ks + 4 * grp;
                const int rq = 16 * w + lr;
                P = mfma(ld_split(&sQ[k_at<DK>(rq, c)], &sQ[k_at<DK>(rq, c + 16)]),
                         ld_split(&sS[lr][c], &sS[lr][c + 16]), P);
            }
            f32x4 eg = {1.f, 1.f, 1.f, 1.f};  // KDA: the decay is inside QG
            if constexpr (!KDA) eg = *reinterpret_cast<const f32x4*>(&E[kEg + 16 * w + 4 * grp]);
            lds_barrier();  // B2
            lds_barrier();  // B3: W is in LDS
            // O = exp(G) P + QKm W
            f32x4 O;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) O[rr] = eg[rr] * P[rr];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                if (2 * ks > w) continue;  // QKm is zero there
                const int c = 32 * ks + 4 * grp;
                const bf16x8 wh = ld_split(&sW[0][lr][c], &sW[0][lr][c + 16]);
                const bf16x8 wl = ld_split(&sW[1][lr][c], &sW[1][lr][c + 16]);
                O = mfma(qk[ks][0], wh, O);
                O = mfma(qk[ks][0], wl, O);
                O = mfma(qk[ks][1], wh, O);
            }
            load_q(min(n + 1, NC - 1));  // qk is not read again in this chunk
            // to LDS; the storer writes the block during the next chunk
            // (it read the previous block before this chunk's B2)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) sO[16 * w + 4 * grp + rr][lr] = O[rr];
        }
        lds_barrier();  // final barrier: the last chunk's output is in LDS
        return;
    }
    if (wave < kStateWaves + kOutWaves + kLoadWaves) {
        // ====================== loader wavefronts ==========================
        // Each loader issues its own run of the chunk's 1 KiB direct-to-LDS
        // loads (kPer of them, the last loader the rest: every load is
        // issued once), in three parts, one after each barrier.  The loads of chunk
        // n + kAhead (= 3) go out during chunk n, and before chunk n + 1's
        // first barrier each loader waits until chunk n + 1's loads are done:
        // only its loads of chunks n + 2 and n + 3 may stay outstanding.
        // Slot (n + 3) % 4 held chunk n - 1, whose last reads come before
        // chunk n's first barrier.
        const int l = wave - kStateWaves - kOutWaves;
        const int hq = qk_head(h, Hqk, group, tiled);  // the q/k head this value head reads
        const size_t headq0 = (static_cast<size_t>(start) * Hqk + hq) * DK;  // q/k element (start, hq, 0)
        const int rowq_b16 = Hqk * DK * 2;                                   // bytes per token of q, k
        const int seqq_b16 = (len - 1) * rowq_b16 + DK * 2;  // end of the last valid row of q, k
        constexpr int kPer = (M::kLoads + kLoadWaves - 1) / kLoadWaves;
        constexpr int kLast = M::kLoads - kPer * (kLoadWaves - 1);  // loads of the last loader
        static_assert(kLast > 0 && kLast <= kPer, "every loader has loads");
        // parts of kP01, kP01 and the rest: little is left for after B3, so
        // that a loader reaches B1 (after waiting for the next chunk) early
        constexpr int kP01 = kPer / 2;
        auto load = [&](int n, int qt) {
            char* slot = sL[n % kRing];
            const int r0 = n * kC;
            const __amdgpu_buffer_rsrc_t rw = ws_rsrc(n);
            const __amdgpu_buffer_rsrc_t rk =
                make_rsrc(k + headq0 + static_cast<size_t>(r0) * Hqk * DK, seqq_b16 - r0 * rowq_b16);
            const __amdgpu_buffer_rsrc_t rq =
                make_rsrc(q + headq0 + static_cast<size_t>(r0) * Hqk * DK, seqq_b16 - r0 * rowq_b16);
            const int j0 = qt * kP01, j1 = qt == 2 ? kPer : (qt + 1) * kP01;
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                const int i = kPer * l + j;
                if (j < j0 || j >= j1 || i >= M::kLoads) continue;
                if (i == 0) {
                    dma16(rw, slot + M::kE, L::kE + 16 * lane);
                } else {
                    const int im = (i - 1) / KPT;  // image: K (KG), then Q (QG)
                    const int pi = i - 1 - im * KPT;
                    const int p = 64 * pi + lane;  // image piece: row p / PPR, slot p % PPR
                    const int rr = p / PPR;
                    const int piece = 16 * ((p % PPR) ^ k_swz<DK>(rr));
                    char* dst = slot + M::kK + im * (kC * DK * 2) + 1024 * pi;
                    if constexpr (kImgKQ) {  // the workspace's row-major images
                        dma16(rw, dst, (im == 0 ? L::kKI : L::kQI) + rr * (DK * 2) + piece);
                    } else {
                        dma16(im == 1 ? rq : rk, dst, rr * rowq_b16 + piece);
                    }
                }
            }
        };
        constexpr int A = M::kAhead;
        for (int a = 0; a < A; ++a)
            if (a < NC)
                for (int qt = 0; qt < 3; ++qt) load(a, qt);
        // chunk 0's loads are done; those of chunks 1 and 2 may stay
        // outstanding (each is waited for at the end of the chunk before it).
        // Measured against waiting for all three: 128 tokens of 16 heads
        // 12.8 us against 13.0, 1024 tokens 32.3 against 33.0
        static_assert(A == 3, "the start-up waits count three chunks");
        if (NC >= 3) {
            if (l < kLoadWaves - 1)
                vm_wait_keep<2 * kPer>();
            else
                vm_wait_keep<2 * kLast>();
        } else if (NC == 2) {
            if (l < kLoadWaves - 1)
                vm_wait_keep<kPer>();
            else
                vm_wait_keep<kLast>();
        } else {
            vm_wait_all();
        }
        for (int n = 0; n < NC; ++n) {
            const bool more = n + A < NC;  // slot (n + A) % kRing was last read before B1
            lds_barrier();  // B1
            if (more) load(n + A, 0);
            lds_barrier();  // B2
            if (more) load(n + A, 1);
            lds_barrier();  // B3
            if (more) {
                load(n + A, 2);
                // chunk n + 1's loads are done
                if (l < kLoadWaves - 1)
                    vm_wait_keep<(A - 1) * kPer>();
                else
                    vm_wait_keep<(A - 1) * kLast>();
            } else {
                vm_wait_all();
            }
        }
        lds_barrier();  // final barrier
        return;
    }
    {
        // ======================= storer wavefront ==========================
        constexpr int kNonTemporal = 2;  // buffer store cache policy: nt
        // chunk n's output block from sO to o: lane -> row lane / 4 + 16 i,
        // columns 4 (lane % 4) + 0..3 of the block, read as two 8-byte halves.
        // The stores go through a buffer view of the chunk's rows with the
        // non-temporal bit: nothing reads o again here, and the prefill ran
        // 3.5 us faster than with plain stores, which keep the lines in L2.
        auto store_o = [&](int n, int i0) {  // rows 16 i + lane / 4, i = i0, i0 + 1
            const int rows = min(kC, len - n * kC);
            const __amdgpu_buffer_rsrc_t ro =
                make_rsrc(o + ((static_cast<size_t>(start) + n * kC) * H + h) * DV + cb * 16,
                          ((rows - 1) * H * DV + 16) * 4);
#pragma unroll
            for (int i = i0; i < i0 + 2; ++i) {
                const int rr = 16 * i + (lane >> 2);
                const float* src = &sO[rr][4 * (lane & 3)];
                const f32x2 a = *reinterpret_cast<const f32x2*>(src);
                const f32x2 c = *reinterpret_cast<const f32x2*>(src + 2);
                if (rr < rows)
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{a[0], a[1], c[0], c[1]}),
                                                           ro, (rr * H * DV + 4 * (lane & 3)) * 4, 0, kNonTemporal);
            }
        };
        // half of the block after B1, half after B2: sO is rewritten after B3
        for (int n = 0; n < NC; ++n) {
            lds_barrier();  // B1: chunk n - 1's output is in sO
            if (n > 0) store_o(n - 1, 0);
            lds_barrier();  // B2
            if (n > 0) store_o(n - 1, 2);
            lds_barrier();  // B3
        }
        lds_barrier();  // final barrier
        store_o(NC - 1, 0);
        store_o(NC - 1, 2);
    }
}

template <int DK, int DV, bool KDA, bool F32>
static hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t stream) {
    char* ws = static_cast<char*>(a.workspace);
    SeqGeom geo;
    if (a.cu_seqlens != nullptr) {  // variable lengths: the table first
        geo.tab = reinterpret_cast<const int32_t*>(ws);
        geo.N = a.B;
        geo.T = 0;
        geo.NC = 0;
        geo.CT = (a.T + kC - 1) / kC + a.B;
        hipLaunchKernelGGL(prefill_table_kernel, dim3(1), dim3(64), 0, stream, a.cu_seqlens, a.B, a.T,
                           reinterpret_cast<int32_t*>(ws));
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        ws += table_bytes(a.B);
    } else {
        geo.tab = nullptr;
        geo.N = a.B;
        geo.T = a.T;
        geo.NC = (a.T + kC - 1) / kC;
        geo.CT = a.B * geo.NC;
    }
    const dim3 prep_grid(static_cast<unsigned>(a.H) * geo.CT);
    if (KDA)
        hipLaunchKernelGGL((prefill_prep_kda_kernel<DK, DV, F32>), prep_grid, dim3(64), 0, stream, a.q, a.k,
                           a.v, a.g, a.beta, ws, geo, a.H, a.Hqk, a.group, a.tiled);
    else if (prep_grid.x <= 2u * static_cast<unsigned>(cu_count()))
        // few blocks: each block's latency sets the prep's time, so a chunk's
        // A and T1 and its QKm go to two blocks (B=1 H=16 d=128: 64 tokens
        // 11.4 us against 14.3 us, 256 tokens 16.0 against 19.4, 1024 tokens
        // 33.3 against 36.5; at 4096 tokens, 1024 blocks, 98 against 95)
        hipLaunchKernelGGL((prefill_prep_kernel<DK, DV, F32, true>), dim3(2 * prep_grid.x), dim3(64), 0, stream,
                           a.q, a.k, a.v, a.g, a.beta, ws, geo, a.H, a.Hqk, a.group, a.tiled);
    else
        hipLaunchKernelGGL((prefill_prep_kernel<DK, DV, F32, false>), prep_grid, dim3(64), 0, stream, a.q, a.k,
                           a.v, a.g, a.beta, ws, geo, a.H, a.Hqk, a.group, a.tiled);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // with float32 inputs the chain reads only the workspace's bf16 images
    // (the input pointers are passed but never read)
    const auto* q = static_cast<const uint16_t*>(a.q);
    const auto* k = static_cast<const uint16_t*>(a.k);
    const auto* v = static_cast<const uint16_t*>(a.v);
    const unsigned bh = static_cast<unsigned>(a.B) * static_cast<unsigned>(a.H);
    hipLaunchKernelGGL((prefill_chain_kernel<DK, DV, KDA, F32>), dim3(bh * (DV / 16)), dim3(kChainThreads), 0,
                       stream, q, k, v, a.state, a.o, ws, geo, a.H, a.Hqk, a.group, a.tiled, a.K,
                       a.final_state, a.k, a.g, a.accepted, a.err_flag);
    return hipGetLastError();
}

template <bool KDA, bool F32>
static hipError_t launch_prefill_d(const PrefillArgs& a, hipStream_t stream) {
    if (a.dk == 128)
        return a.dv == 128 ? launch_prefill_t<128, 128, KDA, F32>(a, stream) : launch_prefill_t<128, 64, KDA, F32>(a, stream);
    return a.dv == 128 ? launch_prefill_t<64, 128, KDA, F32>(a, stream) : launch_prefill_t<64, 64, KDA, F32>(a, stream);
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
    if (a.kda) return a.f32 ? launch_prefill_d<true, true>(a, stream) : launch_prefill_d<true, false>(a, stream);
    return a.f32 ? launch_prefill_d<false, true>(a, stream) : launch_prefill_d<false, false>(a, stream);
}

}  // namespace gdn
