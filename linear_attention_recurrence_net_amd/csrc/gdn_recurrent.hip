// gdn_recurrent.hip -- token-by-token GDN kernel for decode and speculative
// verification (gfx950).
//
// What it computes is the gated delta rule of gdn.h, token after token, with
// the K-slot snapshot semantics of the partial-rollback kernels (koboldcpp
// commit log, tag v1.113.1, bullet "metal: add GDN partial rollback").
//
// Work mapping (HBM-bound: one read and one write of each fp32 state tile
// dominate the bytes):
//  * one workgroup per (sequence, head); DV/32 wavefronts, each owning a
//    block of 32 state columns -- columns of S evolve independently, so the
//    split needs no communication between wavefronts (the pages' CUDA kernel
//    shards columns across warps for the same register-pressure reason:
//    llama.cpp commit log, tag b9752, bullet "Shard columns across warps");
//  * inside a wavefront, lane = 8 * rowgroup + colgroup: the lane holds 4
//    consecutive columns (one 128-bit load per row) of DK/8 consecutive rows,
//    i.e. 64 fp32 registers at d = 128; every state load/store instruction
//    of a wavefront moves 8 full 128-byte rows segments;
//  * the decay is folded into the reductions (k' = a.k, q' = a.q, applied
//    once on the update), so S is read from registers once per token;
//  * S^T k' and S^T q' are summed inside the lane over its rows, then across
//    the 8 row groups with DPP / permlane butterflies (no LDS).
//  * the whole tile is loaded before the first token, so every lane has 16
//    independent 128-bit loads in flight.
//
// Per token the arithmetic is (folded form, equal to decay -> delta ->
// readout):   u = S^T (a.k), p = S^T (a.q), w = beta (v - u),
//             o = p + (k.q) w,  S <- a.S + k w^T.

#include "device_common.hpp"
#include "gdn_internal.hpp"

namespace gdn {

template <int D, bool KDA, bool BF16>
__global__ void __launch_bounds__(D / 32 * kWave)
recurrent_kernel(const void* __restrict__ q, const void* __restrict__ k,
                 const void* __restrict__ v, const float* __restrict__ g,
                 const float* __restrict__ beta, float* __restrict__ state,
                 float* __restrict__ final_state, float* __restrict__ o, int T, int H, int K,
                 int n_snap) {
    constexpr int RPL = D / 8;  // rows held per lane
    constexpr size_t TILE = static_cast<size_t>(D) * D;

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x >> 6;
    const int cg = lane & 7;         // column group inside the wave
    const int rg = lane >> 3;        // row group
    const int col0 = wave * 32 + cg * 4;
    const int row0 = rg * RPL;

    const int bh = blockIdx.x;       // b * H + h
    const int b = bh / H;
    const int h = bh - b * H;

    float* slots = state + static_cast<size_t>(bh) * K * TILE;

    f32x4 s[RPL];
#pragma unroll
    for (int i = 0; i < RPL; ++i) s[i] = ld4(slots + static_cast<size_t>(row0 + i) * D + col0);

    for (int t = 0; t < T; ++t) {
        const size_t bth = (static_cast<size_t>(b) * T + t) * H + h;

        float kv[RPL], qv[RPL];
        load_vec<RPL, BF16>(k, bth * D + row0, kv);
        load_vec<RPL, BF16>(q, bth * D + row0, qv);
        const f32x4 vv = load4<BF16>(v, bth * D + col0);
        const float bt = beta[bth];

        float a_row[KDA ? RPL : 1];
        float a_head = 1.0f;
        if constexpr (KDA) {
            float graw[RPL];
            load_vec<RPL, false>(g, bth * D + row0, graw);
#pragma unroll
            for (int i = 0; i < RPL; ++i) a_row[i] = expf(graw[i]);
        } else {
            a_head = expf(g[bth]);
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
        u0 = sum_over_rowgroups(u0);
        u1 = sum_over_rowgroups(u1);
        u2 = sum_over_rowgroups(u2);
        u3 = sum_over_rowgroups(u3);
        p0 = sum_over_rowgroups(p0);
        p1 = sum_over_rowgroups(p1);
        p2 = sum_over_rowgroups(p2);
        p3 = sum_over_rowgroups(p3);
        kq = sum_over_rowgroups(kq);
        if constexpr (!KDA) {
            u0 *= a_head; u1 *= a_head; u2 *= a_head; u3 *= a_head;
            p0 *= a_head; p1 *= a_head; p2 *= a_head; p3 *= a_head;
        }

        const float w0 = bt * (vv.x - u0);
        const float w1 = bt * (vv.y - u1);
        const float w2 = bt * (vv.z - u2);
        const float w3 = bt * (vv.w - u3);

        if (rg == 0) {
            st4(o + bth * D + col0,
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

        if (t < n_snap) {
            float* dst = slots + static_cast<size_t>(t + 1) * TILE;
#pragma unroll
            for (int i = 0; i < RPL; ++i)
                st4_nt(dst + static_cast<size_t>(row0 + i) * D + col0, s[i]);
        }
    }

    if (K == 1) {
#pragma unroll
        for (int i = 0; i < RPL; ++i)
            st4_nt(slots + static_cast<size_t>(row0 + i) * D + col0, s[i]);
    }
    if (final_state != nullptr) {
        float* dst = final_state + static_cast<size_t>(bh) * TILE;
#pragma unroll
        for (int i = 0; i < RPL; ++i)
            st4_nt(dst + static_cast<size_t>(row0 + i) * D + col0, s[i]);
    }
}

template <int D, bool KDA, bool BF16>
static hipError_t launch_recurrent_t(const RecurrentArgs& a, hipStream_t stream) {
    dim3 grid(static_cast<unsigned>(a.B) * static_cast<unsigned>(a.H));
    dim3 block(D / 32 * kWave);
    hipLaunchKernelGGL((recurrent_kernel<D, KDA, BF16>), grid, block, 0, stream, a.q, a.k, a.v,
                       a.g, a.beta, a.state, a.final_state, a.o, a.T, a.H, a.K, a.n_snap);
    return hipGetLastError();
}

hipError_t launch_recurrent(const RecurrentArgs& a, hipStream_t stream) {
    const bool bf = a.bf16, kda = a.kda;
    if (a.d == 128) {
        if (kda) return bf ? launch_recurrent_t<128, true, true>(a, stream) : launch_recurrent_t<128, true, false>(a, stream);
        return bf ? launch_recurrent_t<128, false, true>(a, stream) : launch_recurrent_t<128, false, false>(a, stream);
    }
    if (kda) return bf ? launch_recurrent_t<64, true, true>(a, stream) : launch_recurrent_t<64, true, false>(a, stream);
    return bf ? launch_recurrent_t<64, false, true>(a, stream) : launch_recurrent_t<64, false, false>(a, stream);
}

}  // namespace gdn
