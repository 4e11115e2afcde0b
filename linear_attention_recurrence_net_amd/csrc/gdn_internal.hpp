// gdn_internal.hpp -- launch descriptors shared by the host entry points and
// the kernel translation units (not part of the public ABI).
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
    float* state;        // [B,H,K,d,d]
    float* final_state;  // [B,H,d,d] or nullptr
    float* o;            // [B,T,H,d]
    int B, T, H, K, d;
    int Hqk;             // q/k heads: value head h reads q/k head qk_head(h)
    int group;           // H / Hqk
    bool tiled;          // qk_head(h) = tiled ? h % Hqk : h / group
    int n_snap;          // snapshot slots written: K > 1 ? min(T, K-1) : 0
    bool bf16, kda;
};

hipError_t launch_recurrent(const RecurrentArgs& a, hipStream_t stream);

hipError_t launch_rollback(int B, int H, int K, size_t tile_elems, const int32_t* accepted,
                           float* state, int32_t* err_flag, hipStream_t stream);

struct PrefillArgs {
    const void* q;  // bf16 or f32 [B,T,H,d], or [total tokens, H, d] with cu_seqlens
    const void* k;
    const void* v;
    const float* g;     // [B,T,H], or [B,T,H,d] for KDA
    const float* beta;  // [B,T,H]
    float* state;       // [B,H,K,d,d]: slot 0 in (and out when K == 1), snapshots in 1..K-1
    float* final_state; // [B,H,d,d] or nullptr; written when K > 1
    float* o;           // [B,T,H,d]
    void* workspace;
    const int32_t* cu_seqlens;  // device [B+1] token offsets, or nullptr: B sequences of T tokens
    int B, T, H, d;             // with cu_seqlens: B sequences, T = total tokens
    int Hqk, group;      // q/k heads, as in RecurrentArgs
    bool tiled;
    int K;               // state slots per (sequence, head)
    bool kda;            // g is [.., H, d] (one log-gate per key row)
    bool f32;            // q, k, v are float32 (else bf16)
};

size_t prefill_workspace_bytes(int B, int T, int H, int d, bool kda = false, bool f32 = false);
size_t prefill_varlen_workspace_bytes(int N, int total, int H, int d);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);

}  // namespace gdn
