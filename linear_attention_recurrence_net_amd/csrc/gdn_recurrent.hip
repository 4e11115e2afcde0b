// gdn_recurrent.hip -- token-by-token GDN kernel for decode and speculative
// verification (gfx950).
//
// What it computes is the gated delta rule of gdn.h, token after token, with
// the K-slot snapshot semantics of the partial-rollback kernels (koboldcpp
// commit log, tag v1.113.1, bullet "metal: add GDN partial rollback").
//
// Work mapping (HBM-bound: one read and one write of each fp32 state tile
// dominate the bytes):
//  * one workgroup per (sequence, head) -- or, when the grid would fill less
//    than one resident round, per (sequence, head, column block) with NCB = 2
//    or 4 blocks of CW = d_v / NCB columns (the columns of S are independent:
//    u_j and p_j sum column j only); its WPH wavefronts split the d_k state
//    rows into blocks of RW = d_k / WPH rows of the workgroup's columns;
//  * inside a wavefront, lane = CG * sub + cg with CG = CW / 4 lanes across
//    a row (4 consecutive columns each, one 128-bit access) and RS = 64 / CG
//    row sub-groups; sub-group `sub` holds the L = RW / RS consecutive rows
//    sub * L .. sub * L + L - 1 of the block.  One load instruction thus
//    moves RS row pieces of 4 * CW bytes (whole 128-byte lines at least),
//    and a lane's k and q rows are contiguous;
//  * a single-token launch uses two wavefronts per head (32 rows of a
//    128 x 128 tile per lane) while the grid fits one resident round, four
//    beyond it; several tokens use four for 128 x 128 tiles, two otherwise.
//    Measured on the MI355X with in-place copies of a 64 MiB state: column
//    blocks of 128-byte row pieces 24.6 us, whole rows with four wavefronts
//    per head 24.1 us, whole rows with two wavefronts per head meeting at a
//    barrier between their loads and stores 22.5 us;
//  * the whole row block is loaded before the first token, so every lane
//    has L independent 128-bit loads in flight;
//  * the decay is folded into the reductions (k' = a.k, q' = a.q, applied
//    once on the update), so S is read from registers once per token;
//  * S^T k' and S^T q' are summed inside the lane over its rows, across the
//    row sub-groups with permlane butterflies, and across the wavefronts of
//    the head through LDS (one LDS-only barrier per token, two buffers by
//    token parity).  Every wavefront adds the partial sums in the same order,
//    so all of them hold bit-identical totals.
//
// Per token the arithmetic is (folded form, equal to decay -> delta ->
// readout):   u = S^T (a.k), p = S^T (a.q), w = beta (v - u),
//             o = p + (k.q) w,  S <- a.S + k w^T.

#include "device_common.hpp"
#include "gdn_internal.hpp"

#include <atomic>
#include <type_traits>

namespace gdn {

namespace {

// Fixed launch choices, each measured on the MI355X (reasons at the launcher
// and at TileIO):
constexpr bool kNtLoad = true;    // state loads and stores are non-temporal
constexpr bool kNtStore = true;
constexpr int kWphOne = 2;        // wavefronts per head for one token
constexpr int kWphMulti = 2;      // ... for several tokens, tiles below 128 x 128
constexpr int kWphMulti128 = 4;   // ... for several tokens, 128 x 128 tiles
constexpr int kDraft = 4;         // 128 x 128 launches of 1..kDraft tokens load all inputs up front

// One head's d_k x d_v state tile, read and written through a buffer
// resource: each lane keeps one byte offset (that of its first row).  Stores,
// and loads with SOFF_LD, pass the row's distance from it (a compile-time
// constant) in the scalar offset; other loads put the row's 4 KiB window in
// the scalar offset and the row inside the window in the vector offset.
// Flat addressing spent a 64-bit address per row beyond the first 4 KiB.
// Measured: the single-token decode (B=64 H=16 d=128) runs 23.2 us with
// scalar-offset loads against 23.9 us without; the four-token verify
// (B=32 H=16) 25.2 us with window loads against 25.8 us with scalar-offset
// loads, and 25.0 us with scalar-offset snapshot stores against 25.2 us
// with window stores.  Accesses are streaming (non-temporal) unless the
// tuning knobs say otherwise.
template <int DK, int DV, bool SOFF_LD>
struct TileIO {
    static constexpr int WIN = 1024 / DV;  // rows per 4 KiB window
    static constexpr int CP = 2;           // cache policy: nt
    __amdgpu_buffer_rsrc_t r;

    __device__ __forceinline__ explicit TileIO(float* tile)
        : r(__builtin_amdgcn_make_buffer_rsrc(tile, 0, DK * DV * 4, 0x00020000)) {}

    // row i of this lane's block; off = byte offset of the lane's first row
    __device__ __forceinline__ f32x4 load(uint32_t off, int i) const {
        const uint32_t vo = SOFF_LD ? off : off + (i % WIN) * DV * 4;
        const int so = SOFF_LD ? i * DV * 4 : (i / WIN) * 4096;
        return __builtin_bit_cast(f32x4,
                                  __builtin_amdgcn_raw_buffer_load_b128(r, vo, so, kNtLoad ? CP : 0));
    }
    __device__ __forceinline__ void store(uint32_t off, int i, f32x4 v) const {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, i * DV * 4,
                                               kNtStore ? CP : 0);
    }
};

// The inputs one lane needs for one token: its RPL rows of k and q, its 4
// columns of v, beta, and one log-gate: the head's, or for per-row gates the
// gate of key row `grow`, whose exponential this lane evaluates for the
// whole wavefront.
template <int RPL, bool KDA, bool BF16>
struct TokenRaw {
    static constexpr int KW = BF16 ? RPL / 2 : RPL;  // 32-bit words per k (or q) slice
    uint32_t kw[KW];
    uint32_t qw[KW];
    uint32_t vw[BF16 ? 2 : 4];
    float g;
    float beta;

    // bth indexes the (sequence, token, value head) of v, g, beta; bthq the
    // (sequence, token, q/k head) of q and k.
    __device__ __forceinline__ void load(const void* q, const void* k, const void* v,
                                         const float* gp, const float* bp, size_t bth,
                                         size_t bthq, int row0, int col0, int grow, int DK, int DV) {
        static_assert(KW % 2 == 0, "row slices are loaded 64 or 128 bits at a time");
        const size_t ko = bthq * DK + row0;  // key index row0 of q and k
        const size_t vo = bth * DV + col0;   // value index col0 of v
        const uint32_t* kp = reinterpret_cast<const uint32_t*>(
            static_cast<const char*>(k) + ko * (BF16 ? 2 : 4));
        const uint32_t* qp = reinterpret_cast<const uint32_t*>(
            static_cast<const char*>(q) + ko * (BF16 ? 2 : 4));
        if constexpr (KW % 4 == 0) {
#pragma unroll
            for (int i = 0; i < KW / 4; ++i) {
                uint4 a = reinterpret_cast<const uint4*>(kp)[i];
                uint4 c = reinterpret_cast<const uint4*>(qp)[i];
                kw[4 * i] = a.x; kw[4 * i + 1] = a.y; kw[4 * i + 2] = a.z; kw[4 * i + 3] = a.w;
                qw[4 * i] = c.x; qw[4 * i + 1] = c.y; qw[4 * i + 2] = c.z; qw[4 * i + 3] = c.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < KW / 2; ++i) {
                uint2 a = reinterpret_cast<const uint2*>(kp)[i];
                uint2 c = reinterpret_cast<const uint2*>(qp)[i];
                kw[2 * i] = a.x; kw[2 * i + 1] = a.y;
                qw[2 * i] = c.x; qw[2 * i + 1] = c.y;
            }
        }
        if constexpr (BF16) {
            uint2 a = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(v) + vo);
            vw[0] = a.x; vw[1] = a.y;
        } else {
            uint4 a = *reinterpret_cast<const uint4*>(static_cast<const float*>(v) + vo);
            vw[0] = a.x; vw[1] = a.y; vw[2] = a.z; vw[3] = a.w;
        }
        g = KDA ? gp[bth * DK + grow] : gp[bth];
        beta = bp[bth];
    }

    __device__ __forceinline__ void unpack_kq(float (&kv)[RPL], float (&qv)[RPL]) const {
        if constexpr (BF16) {
#pragma unroll
            for (int i = 0; i < KW; ++i) {
                unpack_bf16x2(kw[i], kv[2 * i], kv[2 * i + 1]);
                unpack_bf16x2(qw[i], qv[2 * i], qv[2 * i + 1]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < RPL; ++i) {
                kv[i] = __uint_as_float(kw[i]);
                qv[i] = __uint_as_float(qw[i]);
            }
        }
    }

    __device__ __forceinline__ f32x4 vvec() const {
        if constexpr (BF16) {
            float a, b, c, d;
            unpack_bf16x2(vw[0], a, b);
            unpack_bf16x2(vw[1], c, d);
            return f32x4{a, b, c, d};
        } else {
            return f32x4{__uint_as_float(vw[0]), __uint_as_float(vw[1]), __uint_as_float(vw[2]),
                         __uint_as_float(vw[3])};
        }
    }
};

}  // namespace

// Sum of x over the lanes that share lane % FROM (the row sub-groups of a
// wavefront): butterflies over lane bits log2(FROM)..5.
template <int FROM>
__device__ __forceinline__ float sum_subgroups(float x) {
    static_assert(FROM == 8 || FROM == 16 || FROM == 32, "rows of 32, 64 or 128 columns");
    if constexpr (FROM == 8) x = add_xor8(x);
    if constexpr (FROM <= 16) x = add_xor16(x);
    return add_xor32(x);
}

// ONE: the launch has exactly one token and no snapshot (plain decode).
// ROLL: the input state of sequence b is slot accepted[b] (the rollback of
// the previous draft, fused into this launch), copied to slot 0 as well.
// DK and DV: key and value head sizes (state rows and columns).  WPH:
// wavefronts per head, one workgroup per head.  TB > 0: the launch has 1..TB
// tokens, whose inputs are all loaded before the first token is computed.  Two wavefronts per SIMD are
// requested (at most 256 registers), so a 1024-head decode grid of 2048
// wavefronts is resident at once.
template <int DK, int DV, bool KDA, bool BF16, bool ONE, int WPH, int TB, bool ROLL, int NCB>
__global__ void __launch_bounds__((WPH * kWave)) __attribute__((amdgpu_waves_per_eu(2)))
recurrent_kernel(const void* __restrict__ q, const void* __restrict__ k,
                 const void* __restrict__ v, const float* __restrict__ g,
                 const float* __restrict__ beta, float* __restrict__ state,
                 float* __restrict__ final_state, float* __restrict__ o, int T, int H, int K,
                 int n_snap, int Hqk, int group, bool tiled, const int32_t* __restrict__ accepted,
                 int32_t* __restrict__ err_flag) {
    static_assert(!(ROLL && ONE), "a fused rollback runs on the multi-token path");
    constexpr int CW = DV / NCB;      // columns of the workgroup's block
    constexpr int CG = CW / 4;        // lanes across one state row of the block
    constexpr int RS = kWave / CG;    // row sub-groups (rows per load instruction)
    constexpr int RW = DK / WPH;      // rows per wavefront
    constexpr int L = RW / RS;        // rows per lane
    constexpr int RED = 2 * CW + 4;   // one wavefront's partial sums in LDS: u, p, k.q
    static_assert(NCB >= 1 && DV % NCB == 0 && CW >= 32, "column blocks of whole 128-byte lines");
    constexpr size_t TILE = static_cast<size_t>(DK) * DV;
    static_assert(L >= 4 && L % 4 == 0 && RW % RS == 0 && DK % WPH == 0, "tiling");
    static_assert(!KDA || RW <= kWave, "KDA: each lane evaluates one key row's decay");

    // partial sums of each wavefront, two buffers by token parity
    __shared__ __attribute__((aligned(16))) float red[WPH > 1 ? 2 * WPH * RED : 4];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x >> 6;
    const int cg = lane % CG;
    const int sub = lane / CG;
    const int bh = static_cast<int>(blockIdx.x) / NCB;  // b * H + h
    const int lc0 = cg * 4;                             // first column of the lane in the block
    const int col0 = (static_cast<int>(blockIdx.x) % NCB) * CW + lc0;
    const int row0 = wave * RW + sub * L;
    const int grow = wave * RW + lane % RW;  // key row whose decay this lane evaluates (KDA)
    const int b = bh / H;
    const int h = bh - b * H;
    const int hq = qk_head(h, Hqk, group, tiled);  // the q/k head this value head reads

    float* slots = state + static_cast<size_t>(bh) * K * TILE;
    const uint32_t off0 = static_cast<uint32_t>(row0 * DV + col0) * 4u;  // byte offset in a tile

    // Raw inputs of one token, as loaded (bf16 stays packed until used).
    // The first token's are requested before the state rows: the memory
    // counter is in order, so the row reduction can then start on the first
    // rows while later ones are still arriving.
    using Raw = TokenRaw<L, KDA, BF16>;
    const int n_tok = ONE ? 1 : T;
    auto load_token = [&](Raw& r, int t) {
        r.load(q, k, v, g, beta, (static_cast<size_t>(b) * T + t) * H + h,
               (static_cast<size_t>(b) * T + t) * Hqk + hq, row0, col0, grow, DK, DV);
    };
    Raw cur;
    Raw all[TB > 0 ? TB : 1];
    if constexpr (TB > 0) {
        // every token's inputs now (a short draft): no token then waits for a
        // load issued behind an earlier token's snapshot stores
#pragma unroll
        for (int j = 0; j < TB; ++j) load_token(all[j], j < n_tok ? j : n_tok - 1);
    } else if (n_tok > 0) {
        load_token(cur, 0);
    }

    // the slot the input state is read from: 0, or with ROLL the accepted
    // draft length of the sequence (an invalid one is flagged, as by the
    // rollback, and the sequence starts from slot 0)
    int src = 0;
    if constexpr (ROLL) {
        const int a = accepted[b];
        if (a >= 0 && a < K)
            src = a;
        else if (h == 0 && threadIdx.x == 0 && err_flag != nullptr)
            atomicOr(err_flag, 1);
    }
    f32x4 s[L];
    {
        const TileIO<DK, DV, ONE> in(slots + static_cast<size_t>(src) * TILE);
#pragma unroll
        for (int i = 0; i < L; ++i) s[i] = in.load(off0, i);
    }
    // The first token needs the whole row block and its own inputs, so wait
    // for them here.  Without this wait the loop head would see the first
    // token's input registers as still loading on every iteration; the
    // memory counter is in order, so the wait it then emits there would also
    // drain the previous token's snapshot stores.  After it, the in-loop
    // waits cover only the prefetched inputs and the stores stay in flight.
    if (!ONE) __builtin_amdgcn_s_waitcnt(0);
    if constexpr (ROLL) {
        // the rollback itself: slot 0 <- slot src, bit for bit.  No wavefront
        // of the head reads slot 0 here, and the snapshot slots (src among
        // them) are written only after the first token's exchange, which
        // every wavefront of the head reaches with all of its rows loaded.
        if (src != 0) {
            const TileIO<DK, DV, ONE> out(slots);
#pragma unroll
            for (int i = 0; i < L; ++i) out.store(off0, i, s[i]);
        }
    }
    const bool keep_last = K == 1 || final_state != nullptr;

    // One token from its inputs `cur`: the folded update of the row block,
    // the readout, and the store of the new state to slot t + 1 (SNAP 1:
    // always, 2: if t < n_snap).  In the streaming form snapshot and plain
    // tokens run in separate loops, so no snapshot store sits behind a branch
    // and the wait the compiler places for the prefetched inputs leaves the
    // previous token's snapshot stores in flight.
    auto step = [&](int t, const Raw& cur, auto snap_tag) {
        constexpr int SNAP = decltype(snap_tag)::value;
        const bool snap = SNAP == 1 || (SNAP == 2 && t < n_snap);
        const size_t bth = (static_cast<size_t>(b) * T + t) * H + h;

        float kv[L], qv[L];
        cur.unpack_kq(kv, qv);
        const f32x4 vv = cur.vvec();
        const float bt = cur.beta;

        float a_row[KDA ? L : 1];
        float a_head = 1.0f;
        if constexpr (KDA) {
            // one exponential per key row of the block, then each lane
            // gathers the decays of its own rows (row r of the block sits in
            // lane r)
            const float ae = expf(cur.g);
#pragma unroll
            for (int i = 0; i < L; ++i)
                a_row[i] = __int_as_float(__builtin_amdgcn_ds_bpermute((sub * L + i) * 4, __float_as_int(ae)));
        } else {
            a_head = expf(cur.g);
        }

        // in-lane partial sums over this lane's rows
        float u0 = 0.f, u1 = 0.f, u2 = 0.f, u3 = 0.f;
        float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
        float kq = 0.f;
#pragma unroll
        for (int i = 0; i < L; ++i) {
            float kk = kv[i], qq = qv[i];
            kq = fmaf(kv[i], qv[i], kq);
            if constexpr (KDA) {
                kk *= a_row[i];
                qq *= a_row[i];
            }
            u0 = fmaf(s[i].x, kk, u0);
            u1 = fmaf(s[i].y, kk, u1);
            u2 = fmaf(s[i].z, kk, u2);
            u3 = fmaf(s[i].w, kk, u3);
            p0 = fmaf(s[i].x, qq, p0);
            p1 = fmaf(s[i].y, qq, p1);
            p2 = fmaf(s[i].z, qq, p2);
            p3 = fmaf(s[i].w, qq, p3);
        }
        // across the row sub-groups of the wavefront, then across the
        // wavefronts of the head through LDS: each wavefront writes its
        // partials and every lane sums those of its own columns in order
        // 0..WPH-1.  With 64 columns (four row sub-groups) paired butterflies
        // finish two sums per swap and leave each lane with two adjacent
        // column totals of u or p, which it writes; otherwise every lane
        // holds its sub-group's totals of all four columns and writes those.
        // Measured on the 64 x 64 KDA verify (B=32 H=32 T=4 K=4): 14.0 us
        // against 14.6 us; with 128 columns the paired form was neutral on
        // the verify and 1.1 us slower on the decode.
        constexpr bool PAIRED = WPH > 1 && CG == 16;
        kq = sum_subgroups<CG>(kq);
        if constexpr (!PAIRED) {
            u0 = sum_subgroups<CG>(u0);
            u1 = sum_subgroups<CG>(u1);
            u2 = sum_subgroups<CG>(u2);
            u3 = sum_subgroups<CG>(u3);
            p0 = sum_subgroups<CG>(p0);
            p1 = sum_subgroups<CG>(p1);
            p2 = sum_subgroups<CG>(p2);
            p3 = sum_subgroups<CG>(p3);
        }
        if constexpr (WPH > 1) {
            float* buf = red + (t & 1) * (WPH * RED);
            float* mine = buf + wave * RED;
            if constexpr (PAIRED) {
                // sub 0, 1 | 2, 3 -> u0 u1 p0 p1 | u2 u3 p2 p3, then
                // sub 0 | 1 | 2 | 3 -> u0 u1 | p0 p1 | u2 u3 | p2 p3
                const float ra = add_xor32_pair(u0, u2), rb = add_xor32_pair(u1, u3);
                const float rc = add_xor32_pair(p0, p2), rd = add_xor32_pair(p1, p3);
                const float x = add_xor16_pair(ra, rc), y = add_xor16_pair(rb, rd);
                *reinterpret_cast<f32x2*>(mine + (sub & 1) * CW + lc0 + (sub >> 1) * 2) = f32x2{x, y};
            } else {
                *reinterpret_cast<f32x4*>(mine + lc0) = f32x4{u0, u1, u2, u3};
                *reinterpret_cast<f32x4*>(mine + CW + lc0) = f32x4{p0, p1, p2, p3};
            }
            mine[2 * CW] = kq;
            lds_barrier();
            f32x4 ut = *reinterpret_cast<const f32x4*>(buf + lc0);
            f32x4 pt = *reinterpret_cast<const f32x4*>(buf + CW + lc0);
            float kqt = buf[2 * CW];
#pragma unroll
            for (int w = 1; w < WPH; ++w) {
                ut += *reinterpret_cast<const f32x4*>(buf + w * RED + lc0);
                pt += *reinterpret_cast<const f32x4*>(buf + w * RED + CW + lc0);
                kqt += buf[w * RED + 2 * CW];
            }
            u0 = ut.x; u1 = ut.y; u2 = ut.z; u3 = ut.w;
            p0 = pt.x; p1 = pt.y; p2 = pt.z; p3 = pt.w;
            kq = kqt;
        }
        if constexpr (!KDA) {
            u0 *= a_head; u1 *= a_head; u2 *= a_head; u3 *= a_head;
            p0 *= a_head; p1 *= a_head; p2 *= a_head; p3 *= a_head;
        }

        const float w0 = bt * (vv.x - u0);
        const float w1 = bt * (vv.y - u1);
        const float w2 = bt * (vv.z - u2);
        const float w3 = bt * (vv.w - u3);

        // Every lane of the head holds the bit-identical o for its columns.
        // Row sub-group 0 of wavefront 0 stores it, except over several
        // tokens of a tile smaller than 128 x 128, where every lane stores it
        // (the same values to the same addresses) and the body keeps no
        // branch.  Measured on the verify workloads (four tokens): 128 x 128
        // 25.4 us against 25.9 us with every lane storing, 64 x 64 KDA
        // 14.8 us against 15.0 us with one lane group storing.
        constexpr bool O_ALL = !ONE && DK * DV < 128 * 128;
        const f32x4 ov{fmaf(kq, w0, p0), fmaf(kq, w1, p1), fmaf(kq, w2, p2), fmaf(kq, w3, p3)};
        if (O_ALL || (wave == 0 && sub == 0)) st4(o + bth * DV + col0, ov);

        // The state after the last token is needed only if it is stored (in
        // place for K = 1, or as the final state); o needs none of it.  For
        // 128 x 128 tiles the update is then skipped (verify B=32 H=16 T=4
        // K=4: 25.3 us against 25.6 us); smaller tiles keep the body free of
        // the branch (64 x 64 KDA verify: 14.6 us against 15.2 us with it).
        constexpr bool TRIM = DK * DV == 128 * 128;
        if (ONE || snap || !TRIM || keep_last || t + 1 < n_tok) {
            // decay in place, then fuse the rank-1 term into it: each element
            // stays in its register (fusing the decay into a separate k*w
            // product made the compiler copy every element back, one extra
            // instruction per element and token)
#pragma unroll
            for (int i = 0; i < L; ++i) {
                const float a = KDA ? a_row[i] : a_head;
                const float kk = kv[i];
                s[i].x = fmaf(kk, w0, a * s[i].x);
                s[i].y = fmaf(kk, w1, a * s[i].y);
                s[i].z = fmaf(kk, w2, a * s[i].z);
                s[i].w = fmaf(kk, w3, a * s[i].w);
            }
        }

        if (snap) {
            const TileIO<DK, DV, ONE> out(slots + static_cast<size_t>(t + 1) * TILE);
#pragma unroll
            for (int i = 0; i < L; ++i) out.store(off0, i, s[i]);
        }
    };
    using Plain = std::integral_constant<int, 0>;
    using Snap = std::integral_constant<int, 1>;
    using SnapIf = std::integral_constant<int, 2>;

    if constexpr (ONE) {
        step(0, cur, Plain{});
    } else if constexpr (TB > 0) {
#pragma unroll
        for (int j = 0; j < TB; ++j)
            if (j < n_tok) step(j, all[j], SnapIf{});
    } else {
        // prefetch the next token while this one is computed (the last token
        // reloads itself, so the load needs no branch)
        int t = 0;
        for (; t < n_snap; ++t) {
            Raw nxt;
            load_token(nxt, t + 1 < n_tok ? t + 1 : t);
            step(t, cur, Snap{});
            cur = nxt;
        }
        for (; t < n_tok; ++t) {
            Raw nxt;
            load_token(nxt, t + 1 < n_tok ? t + 1 : t);
            step(t, cur, Plain{});
            cur = nxt;
        }
    }

    if (K == 1) {
#pragma unroll
        for (int i = 0; i < L; ++i) TileIO<DK, DV, ONE>(slots).store(off0, i, s[i]);
    }
    if (final_state != nullptr) {
        const TileIO<DK, DV, ONE> out(final_state + static_cast<size_t>(bh) * TILE);
#pragma unroll
        for (int i = 0; i < L; ++i) out.store(off0, i, s[i]);
    }
}

template <int DK, int DV, bool KDA, bool BF16, bool ONE, int WPH, int TB = 0, bool ROLL = false, int NCB = 1>
static void launch_recurrent_shape(const RecurrentArgs& a, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(a.B) * static_cast<unsigned>(a.H) * NCB);
    hipLaunchKernelGGL((recurrent_kernel<DK, DV, KDA, BF16, ONE, WPH, TB, ROLL, NCB>), grid, dim3(WPH * kWave), 0, stream,
                       a.q, a.k, a.v, a.g, a.beta, a.state, a.final_state, a.o, a.T, a.H, a.K,
                       a.n_snap, a.Hqk, a.group, a.tiled, a.accepted, a.err_flag);
}

// Read once per device (host threads may race to fill an entry; they all
// store the same value).
int cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int cu = cache[dev].load(std::memory_order_relaxed);
    if (cu == 0) {
        if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0)
            cu = 256;
        cache[dev].store(cu, std::memory_order_relaxed);
    }
    return cu;
}

// Heads that one round of the single-token 128 x 128 kernel holds at two
// wavefronts per head and two wavefronts per SIMD: four per compute unit.
static long resident_heads() { return 4L * cu_count(); }

// Column blocks per head: a grid that would fill less than one resident
// round (two wavefronts per SIMD) is split into 4 or 2 blocks of whole
// 128-byte row pieces, so that more compute units share the head's state.
// Measured on decode GDA H=16 d=128 (one token): B=1 3.1 us against 4.7 us
// with whole rows, B=8 4.9 against 6.0, B=16 6.8 against 8.4, B=32 (two
// blocks) 11.8 against 12.9; at B=64 two blocks took 24.2 us against 23.1.
template <int DK, int DV, bool KDA, bool BF16, bool ONE, int WPH, int TB = 0, bool ROLL = false>
static void launch_cols(const RecurrentArgs& a, hipStream_t stream) {
    const long waves = static_cast<long>(a.B) * a.H * WPH;
    // wavefronts of one resident round; half of it for the 128 x 128 draft
    // form, whose fused-rollback launches lost 0.2-0.8 us when column blocks
    // filled a whole round (B=8 and 16 of H=16)
    const long round = (TB > 0 ? 1 : 2) * resident_heads();
    if constexpr (DV >= 128) {
        if (4 * waves <= round) {
            launch_recurrent_shape<DK, DV, KDA, BF16, ONE, WPH, TB, ROLL, 4>(a, stream);
            return;
        }
    }
    if (2 * waves <= round) {
        launch_recurrent_shape<DK, DV, KDA, BF16, ONE, WPH, TB, ROLL, 2>(a, stream);
        return;
    }
    launch_recurrent_shape<DK, DV, KDA, BF16, ONE, WPH, TB, ROLL, 1>(a, stream);
}

// Wavefronts per head for a requested count: KDA evaluates one key row's decay
// per lane, so its wavefronts own at most 64 rows each.
template <int DK, bool KDA>
constexpr int heads_split(int wph) { return KDA && DK / wph > kWave ? DK / kWave : wph; }

template <int DK, int DV, bool KDA, bool BF16>
static hipError_t launch_recurrent_t(const RecurrentArgs& a, hipStream_t stream) {
    if (a.accepted != nullptr) {
        // rollback fused into the launch: the multi-token shapes, any T >= 1
        constexpr int WPH = heads_split<DK, KDA>(DK == 128 && DV == 128 ? kWphMulti128 : kWphMulti);
        constexpr bool DRAFT = DK == 128 && DV == 128;
        if (DRAFT && a.T >= 1 && a.T <= kDraft)
            launch_cols<DK, DV, KDA, BF16, false, WPH, DRAFT ? kDraft : 0, true>(a, stream);
        else
            launch_cols<DK, DV, KDA, BF16, false, WPH, 0, true>(a, stream);
        return hipGetLastError();
    }
    if (a.T == 1 && a.n_snap == 0) {
        // Single token: two wavefronts per head while the grid fits one
        // resident round (64 MiB of 128 x 128 state: 23.7 us against 25.1 us
        // at four), four beyond it (2048 heads: 48.6 us against 51.5 us).
        if constexpr (DK == 128 && DV == 128) {
            if (static_cast<long>(a.B) * a.H > resident_heads()) {
                launch_recurrent_shape<DK, DV, KDA, BF16, true, 4>(a, stream);
                return hipGetLastError();
            }
        }
        launch_cols<DK, DV, KDA, BF16, true, heads_split<DK, KDA>(kWphOne)>(a, stream);
    } else {
        // Over several tokens a 128 x 128 tile is split four ways: at two
        // wavefronts per head the prefetched inputs no longer fit in registers.
        constexpr int WPH = heads_split<DK, KDA>(DK == 128 && DV == 128 ? kWphMulti128 : kWphMulti);
        // Short drafts of a 128 x 128 tile load all their inputs up front
        // (verify B=32 H=16 T=4 K=4: 25.0 us against 25.2 us streamed); the
        // 64 x 64 KDA verify measured 0.3-0.6 us slower that way.
        constexpr bool DRAFT = DK == 128 && DV == 128;
        if (DRAFT && a.T >= 1 && a.T <= kDraft)
            launch_cols<DK, DV, KDA, BF16, false, WPH, DRAFT ? kDraft : 0>(a, stream);
        else
            launch_cols<DK, DV, KDA, BF16, false, WPH>(a, stream);
    }
    return hipGetLastError();
}

template <int DK, int DV>
static hipError_t launch_recurrent_d(const RecurrentArgs& a, hipStream_t stream) {
    if (a.kda)
        return a.bf16 ? launch_recurrent_t<DK, DV, true, true>(a, stream) : launch_recurrent_t<DK, DV, true, false>(a, stream);
    return a.bf16 ? launch_recurrent_t<DK, DV, false, true>(a, stream) : launch_recurrent_t<DK, DV, false, false>(a, stream);
}

hipError_t launch_recurrent(const RecurrentArgs& a, hipStream_t stream) {
    if (a.dk == 128)
        return a.dv == 128 ? launch_recurrent_d<128, 128>(a, stream) : launch_recurrent_d<128, 64>(a, stream);
    return a.dv == 128 ? launch_recurrent_d<64, 128>(a, stream) : launch_recurrent_d<64, 64>(a, stream);
}

}  // namespace gdn
