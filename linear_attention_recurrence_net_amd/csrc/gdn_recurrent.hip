// gdn_recurrent.hip -- token-by-token GDN kernel for decode and speculative
// verification (gfx950).
//
// What it computes is the gated delta rule of gdn.h, token after token, with
// the K-slot snapshot semantics of the partial-rollback kernels (koboldcpp
// commit log, tag v1.113.1, bullet "metal: add GDN partial rollback").
//
// Work mapping (HBM-bound: one read and one write of each fp32 state tile
// dominate the bytes):
//  * columns of S evolve independently, so each wavefront owns a block of
//    CPW state columns across all d_k rows and needs no communication with
//    other wavefronts (the pages' CUDA kernel shards columns across warps
//    for the same register-pressure reason: llama.cpp commit log, tag b9752,
//    bullet "Shard columns across warps");
//  * a workgroup holds WPG such wavefronts of one (sequence, head);
//  * inside a wavefront, lane = CG * rowgroup + colgroup with CG = CPW/4:
//    the lane holds 4 consecutive columns (one 128-bit load per row) of
//    RPL = d_k / (64/CG) consecutive rows;
//  * the whole column block is loaded before the first token, so every lane
//    has RPL independent 128-bit loads in flight;
//  * the decay is folded into the reductions (k' = a.k, q' = a.q, applied
//    once on the update), so S is read from registers once per token;
//  * S^T k' and S^T q' are summed inside the lane over its rows, then across
//    the row groups with swizzle / DPP / permlane butterflies (no LDS).
//
// Per token the arithmetic is (folded form, equal to decay -> delta ->
// readout):   u = S^T (a.k), p = S^T (a.q), w = beta (v - u),
//             o = p + (k.q) w,  S <- a.S + k w^T.

#include "device_common.hpp"
#include "gdn_internal.hpp"

// Tuning knobs (columns per wavefront, wavefronts per workgroup, minimum
// waves per SIMD requested from the register allocator, streaming loads).
#ifndef GDN_DEC_CPW
#define GDN_DEC_CPW 32
#endif
#ifndef GDN_DEC_WPG
#define GDN_DEC_WPG 2
#endif
#ifndef GDN_DEC_WAVES_PER_EU
#define GDN_DEC_WAVES_PER_EU 0
#endif
#ifndef GDN_DEC_NT_LOAD
#define GDN_DEC_NT_LOAD 1
#endif
#ifndef GDN_DEC_NT_STORE
#define GDN_DEC_NT_STORE 1
#endif

namespace gdn {

namespace {

constexpr int kCPW = GDN_DEC_CPW;

// Wavefronts per workgroup (each owns kCPW state columns): GDN_DEC_WPG for
// the single-token decode, twice that for launches over several tokens,
// where the longer-lived workgroups measured faster (16-token-head verify at
// d = 128: 25.3 us against 26.5 us), both capped by the column count.
template <int DV, bool ONE>
constexpr int waves_per_group() {
    constexpr int want = ONE ? GDN_DEC_WPG : 2 * GDN_DEC_WPG;
    return (DV / kCPW) < want ? (DV / kCPW) : want;
}

__device__ __forceinline__ f32x4 load_state(const float* p) {
#if GDN_DEC_NT_LOAD
    return ld4_nt(p);
#else
    return ld4(p);
#endif
}

__device__ __forceinline__ void store_state(float* p, f32x4 v) {
#if GDN_DEC_NT_STORE
    st4_nt(p, v);
#else
    st4(p, v);
#endif
}

// The inputs one lane needs for one token: its RPL rows of k and q, its 4
// columns of v, beta, and the log-gate (one, or RPL for per-row gates).
template <int RPL, bool KDA, bool BF16>
struct TokenRaw {
    static constexpr int KW = BF16 ? RPL / 2 : RPL;  // 32-bit words per k (or q) slice
    uint32_t kw[KW];
    uint32_t qw[KW];
    uint32_t vw[BF16 ? 2 : 4];
    float g[KDA ? RPL : 1];
    float beta;

    // bth indexes the (sequence, token, value head) of v, g, beta; bthq the
    // (sequence, token, q/k head) of q and k.
    __device__ __forceinline__ void load(const void* q, const void* k, const void* v,
                                         const float* gp, const float* bp, size_t bth,
                                         size_t bthq, int row0, int col0, int DK, int DV) {
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
        if constexpr (KDA) {
            float tmp[RPL];
            load_vec<RPL, false>(gp, bth * DK + row0, tmp);
#pragma unroll
            for (int i = 0; i < RPL; ++i) g[i] = tmp[i];
        } else {
            g[0] = gp[bth];
        }
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

// ONE: the launch has exactly one token and no snapshot (plain decode); the
// token loop is then straight-line code.  DK and DV: key and value head
// sizes (state rows and columns).
template <int DK, int DV, bool KDA, bool BF16, bool ONE>
__global__ void __launch_bounds__((waves_per_group<DV, ONE>() * kWave))
#if GDN_DEC_WAVES_PER_EU > 0
__attribute__((amdgpu_waves_per_eu(GDN_DEC_WAVES_PER_EU)))
#endif
recurrent_kernel(const void* __restrict__ q, const void* __restrict__ k,
                 const void* __restrict__ v, const float* __restrict__ g,
                 const float* __restrict__ beta, float* __restrict__ state,
                 float* __restrict__ final_state, float* __restrict__ o, int T, int H, int K,
                 int n_snap, int Hqk, int group, bool tiled) {
    constexpr int CG = kCPW / 4;     // lanes across one row segment
    constexpr int RG = kWave / CG;   // row groups
    constexpr int RPL = DK / RG;     // rows held per lane
    constexpr int WPG = waves_per_group<DV, ONE>();
    constexpr int NB = DV / (kCPW * WPG);  // workgroups per head
    constexpr size_t TILE = static_cast<size_t>(DK) * DV;
    static_assert(RPL >= 1 && DK % RG == 0 && DV % (kCPW * WPG) == 0, "tiling");

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x >> 6;
    const int cg = lane % CG;
    const int rg = lane / CG;
    const int bh = blockIdx.x / NB;  // b * H + h
    const int cb = blockIdx.x - bh * NB;
    const int col0 = (cb * WPG + wave) * kCPW + cg * 4;
    const int row0 = rg * RPL;
    const int b = bh / H;
    const int h = bh - b * H;
    const int hq = qk_head(h, Hqk, group, tiled);  // the q/k head this value head reads

    float* slots = state + static_cast<size_t>(bh) * K * TILE;

    f32x4 s[RPL];
#pragma unroll
    for (int i = 0; i < RPL; ++i) s[i] = load_state(slots + static_cast<size_t>(row0 + i) * DV + col0);

    // Raw inputs of one token, as loaded (bf16 stays packed until used).
    using Raw = TokenRaw<RPL, KDA, BF16>;
    const int n_tok = ONE ? 1 : T;
    Raw cur;
    if (n_tok > 0)
        cur.load(q, k, v, g, beta, (static_cast<size_t>(b) * T) * H + h,
                 (static_cast<size_t>(b) * T) * Hqk + hq, row0, col0, DK, DV);

    for (int t = 0; t < n_tok; ++t) {
        const size_t bth = (static_cast<size_t>(b) * T + t) * H + h;
        const size_t bthq = (static_cast<size_t>(b) * T + t) * Hqk + hq;
        // prefetch the next token while this one is computed
        Raw nxt;
        if (!ONE && t + 1 < n_tok) nxt.load(q, k, v, g, beta, bth + H, bthq + Hqk, row0, col0, DK, DV);

        float kv[RPL], qv[RPL];
        cur.unpack_kq(kv, qv);
        const f32x4 vv = cur.vvec();
        const float bt = cur.beta;

        float a_row[KDA ? RPL : 1];
        float a_head = 1.0f;
        if constexpr (KDA) {
#pragma unroll
            for (int i = 0; i < RPL; ++i) a_row[i] = expf(cur.g[i]);
        } else {
            a_head = expf(cur.g[0]);
        }

        // in-lane partial sums over this lane's rows
        float u0 = 0.f, u1 = 0.f, u2 = 0.f, u3 = 0.f;
        float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
        float kq = 0.f;
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
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
        u0 = sum_lanes_from<CG>(u0);
        u1 = sum_lanes_from<CG>(u1);
        u2 = sum_lanes_from<CG>(u2);
        u3 = sum_lanes_from<CG>(u3);
        p0 = sum_lanes_from<CG>(p0);
        p1 = sum_lanes_from<CG>(p1);
        p2 = sum_lanes_from<CG>(p2);
        p3 = sum_lanes_from<CG>(p3);
        kq = sum_lanes_from<CG>(kq);
        if constexpr (!KDA) {
            u0 *= a_head; u1 *= a_head; u2 *= a_head; u3 *= a_head;
            p0 *= a_head; p1 *= a_head; p2 *= a_head; p3 *= a_head;
        }

        const float w0 = bt * (vv.x - u0);
        const float w1 = bt * (vv.y - u1);
        const float w2 = bt * (vv.z - u2);
        const float w3 = bt * (vv.w - u3);

        if (rg == 0) {
            st4(o + bth * DV + col0,
                f32x4{fmaf(kq, w0, p0), fmaf(kq, w1, p1), fmaf(kq, w2, p2), fmaf(kq, w3, p3)});
        }

#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            const float a = KDA ? a_row[i] : a_head;
            const float kk = kv[i];
            s[i].x = fmaf(a, s[i].x, kk * w0);
            s[i].y = fmaf(a, s[i].y, kk * w1);
            s[i].z = fmaf(a, s[i].z, kk * w2);
            s[i].w = fmaf(a, s[i].w, kk * w3);
        }

        if (!ONE && t < n_snap) {
            float* dst = slots + static_cast<size_t>(t + 1) * TILE;
#pragma unroll
            for (int i = 0; i < RPL; ++i) store_state(dst + static_cast<size_t>(row0 + i) * DV + col0, s[i]);
        }
        if (!ONE) cur = nxt;
    }

    if (K == 1) {
#pragma unroll
        for (int i = 0; i < RPL; ++i) store_state(slots + static_cast<size_t>(row0 + i) * DV + col0, s[i]);
    }
    if (final_state != nullptr) {
        float* dst = final_state + static_cast<size_t>(bh) * TILE;
#pragma unroll
        for (int i = 0; i < RPL; ++i) store_state(dst + static_cast<size_t>(row0 + i) * DV + col0, s[i]);
    }
}

template <int DK, int DV, bool KDA, bool BF16, bool ONE>
static void launch_recurrent_shape(const RecurrentArgs& a, hipStream_t stream) {
    constexpr int WPG = waves_per_group<DV, ONE>();
    constexpr int NB = DV / (kCPW * WPG);
    const dim3 grid(static_cast<unsigned>(a.B) * static_cast<unsigned>(a.H) * NB);
    hipLaunchKernelGGL((recurrent_kernel<DK, DV, KDA, BF16, ONE>), grid, dim3(WPG * kWave), 0, stream,
                       a.q, a.k, a.v, a.g, a.beta, a.state, a.final_state, a.o, a.T, a.H, a.K,
                       a.n_snap, a.Hqk, a.group, a.tiled);
}

template <int DK, int DV, bool KDA, bool BF16>
static hipError_t launch_recurrent_t(const RecurrentArgs& a, hipStream_t stream) {
    if (a.T == 1 && a.n_snap == 0)
        launch_recurrent_shape<DK, DV, KDA, BF16, true>(a, stream);
    else
        launch_recurrent_shape<DK, DV, KDA, BF16, false>(a, stream);
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
