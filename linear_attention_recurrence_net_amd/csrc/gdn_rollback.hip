// gdn_rollback.hip -- restore the accepted snapshot slot into slot 0.
//
// After speculative verification a sequence keeps the state after its
// accepted tokens (koboldcpp commit log, tag v1.113.1, bullet "llama: allow
// partial seq_rm for GDN models for speculative decoding").  The snapshot
// kernel left S_a in slot a, so the rollback is a bitwise copy slot a -> 0
// for every head of the sequence: a pure streaming copy, bound by HBM.
//
// One workgroup of two wavefronts copies one (sequence, head) tile (a quarter
// of one when there are few 64 KiB tiles); each lane issues all of its 128-bit
// loads, the workgroup meets at a barrier once they have landed, then every
// lane stores.  On the MI355X this shape copied
// the 24 rolled-back sequences of the B=32 H=16 d=128 verify workload in
// 9.2 us, against 10.3 us for four-wavefront groups without the barrier.
// Workgroups of sequences with a == 0 exit at once.

#include "device_common.hpp"
#include "gdn_internal.hpp"

namespace gdn {

// Two wavefronts per (sequence, head) tile.
constexpr int kCopyThreads = 128;

template <int PER_LANE>
__global__ void __launch_bounds__(kCopyThreads)
rollback_kernel(const int32_t* __restrict__ accepted, float* __restrict__ state, int H, int K,
                size_t tile_vec4, int32_t* __restrict__ err_flag, int parts) {
    // `parts` workgroups per tile (PER_LANE > 0), each copying its own
    // contiguous PER_LANE * kCopyThreads 16-byte pieces of it
    const int bh = static_cast<int>(blockIdx.x) / parts;
    const int part = static_cast<int>(blockIdx.x) - bh * parts;
    const int b = bh / H;
    const int h = bh - b * H;
    const int a = accepted[b];
    if (a < 0 || a >= K) {
        if (h == 0 && part == 0 && threadIdx.x == 0 && err_flag != nullptr) atomicOr(err_flag, 1);
        return;
    }
    if (a == 0) return;
    float* base = state + static_cast<size_t>(bh) * K * tile_vec4 * 4 +
                  static_cast<size_t>(part) * (PER_LANE > 0 ? PER_LANE : 0) * kCopyThreads * 4;
    const float* src = base + static_cast<size_t>(a) * tile_vec4 * 4;
    if constexpr (PER_LANE > 0) {
        // tile_vec4 == PER_LANE * kCopyThreads
        f32x4 r[PER_LANE];
#pragma unroll
        for (int i = 0; i < PER_LANE; ++i) r[i] = ld4_nt(src + 4 * (i * kCopyThreads + threadIdx.x));
        // every load has landed before any lane of the group stores
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_s_barrier();
#pragma unroll
        for (int i = 0; i < PER_LANE; ++i) st4_nt(base + 4 * (i * kCopyThreads + threadIdx.x), r[i]);
    } else {
        for (size_t i = threadIdx.x; i < tile_vec4; i += kCopyThreads) st4(base + 4 * i, ld4(src + 4 * i));
    }
}

hipError_t launch_rollback(int B, int H, int K, size_t tile_elems, const int32_t* accepted,
                           float* state, int32_t* err_flag, hipStream_t stream) {
    const size_t tile_vec4 = tile_elems / 4;
    const unsigned heads = static_cast<unsigned>(B) * static_cast<unsigned>(H);
    dim3 grid(heads);
    dim3 block(kCopyThreads);
    constexpr int big = 4096 / kCopyThreads, small = 1024 / kCopyThreads;  // 64 KiB and 16 KiB tiles
    if (tile_vec4 == big * kCopyThreads && 4 * heads <= static_cast<unsigned>(cu_count()))
        // few tiles: four workgroups per tile (all 16 heads of one sequence
        // at d = 128: 2.5 us against 3.5 us, four sequences 3.1 against 3.8;
        // eight sequences 4.6 against 4.5)
        hipLaunchKernelGGL(rollback_kernel<small>, dim3(4 * heads), block, 0, stream, accepted, state, H, K, tile_vec4,
                           err_flag, 4);
    else if (tile_vec4 == big * kCopyThreads)
        hipLaunchKernelGGL(rollback_kernel<big>, grid, block, 0, stream, accepted, state, H, K, tile_vec4, err_flag, 1);
    else if (tile_vec4 == small * kCopyThreads)
        hipLaunchKernelGGL(rollback_kernel<small>, grid, block, 0, stream, accepted, state, H, K, tile_vec4, err_flag, 1);
    else
        hipLaunchKernelGGL(rollback_kernel<0>, grid, block, 0, stream, accepted, state, H, K, tile_vec4, err_flag, 1);
    return hipGetLastError();
}

}  // namespace gdn
