// gdn_internal.hpp -- launch descriptors of the token kernels (recurrent,
// rollback) shared by the host entry points and the kernel translation units
// (not part of the public ABI).  The prefill's are in gdn_prefill_args.hpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

// The q/k head that value head h reads (h / group, or h % Hqk when tiled).
__host__ __device__ inline int qk_head(int h, int Hqk, int group, bool tiled) {
    return tiled ? h % Hqk : h / group;
}

struct RecurrentArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    float* state;        // [B,H,K,dk,dv]
    float* final_state;  // [B,H,dk,dv] or nullptr
    float* o;            // [B,T,H,dv]
    int B, T, H, K;
    int dk, dv;          // key and value head sizes, each 64 or 128
    int Hqk;             // q/k heads: value head h reads q/k head qk_head(h)
    int group;           // H / Hqk
    bool tiled;          // qk_head(h) = tiled ? h % Hqk : h / group
    int n_snap;          // snapshot slots written: K > 1 ? min(T, K-1) : 0
    bool bf16, kda;
    // Rollback of the previous draft before this call (nullptr: none): the
    // input state of sequence b is slot accepted[b], which is also copied to
    // slot 0; an index outside 0..K-1 sets *err_flag (if given) and the
    // sequence starts from slot 0.
    const int32_t* accepted = nullptr;
    int32_t* err_flag = nullptr;
};

hipError_t launch_recurrent(const RecurrentArgs& a, hipStream_t stream);

// Compute units of the current device (read once per device; 256 if the
// runtime cannot say).
int cu_count();

hipError_t launch_rollback(int B, int H, int K, size_t tile_elems, const int32_t* accepted,
                           float* state, int32_t* err_flag, hipStream_t stream);

}  // namespace gdn
