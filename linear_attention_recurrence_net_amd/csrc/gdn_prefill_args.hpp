// gdn_prefill_args.hpp -- launch descriptor of the chunked prefill, shared
// by the host entry points and gdn_prefill.hip (not part of the public ABI).
#pragma once

#include "gdn_internal.hpp"

namespace gdn {

struct PrefillArgs {
    const void* q;  // bf16 or f32 [B,T,H_qk,dk], or [total tokens, H_qk, dk] with cu_seqlens
    const void* k;
    const void* v;
    const float* g;     // [B,T,H], or [B,T,H,dk] for KDA
    const float* beta;  // [B,T,H]
    float* state;       // [B,H,K,dk,dv]: slot 0 in (and out when K == 1), snapshots in 1..K-1
    float* final_state; // [B,H,dk,dv] or nullptr; written when K > 1
    float* o;           // [B,T,H,dv]
    void* workspace;
    const int32_t* cu_seqlens;  // device [B+1] token offsets, or nullptr: B sequences of T tokens
    int B, T, H;                // with cu_seqlens: B sequences, T = total tokens
    int dk, dv;                 // key and value head sizes, each 64 or 128
    int Hqk, group;      // q/k heads, as in RecurrentArgs
    bool tiled;
    int K;               // state slots per (sequence, head)
    bool kda;            // g is [.., H, dk] (one log-gate per key row)
    bool f32;            // q, k, v are float32 (else bf16)
    // Rollback of the previous draft before this call (nullptr: none; K > 1
    // and no cu_seqlens): the input state of sequence b is slot accepted[b],
    // also copied to slot 0; an index outside 0..K-1 sets *err_flag (if
    // given) and the sequence starts from slot 0.
    const int32_t* accepted = nullptr;
    int32_t* err_flag = nullptr;
};

size_t prefill_workspace_bytes(int B, int T, int H, int dk, int dv, bool kda = false, bool f32 = false);
size_t prefill_varlen_workspace_bytes(int N, int total, int H, int dk, int dv, bool kda = false,
                                      bool f32 = false);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);

}  // namespace gdn
