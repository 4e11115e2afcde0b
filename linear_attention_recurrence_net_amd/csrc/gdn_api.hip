// gdn_api.hip -- the extern "C" entry points of gdn.h (all but the no-alloc
// prefill, in gdn_noalloc.hip): host-side validation, kernel selection and
// launch on the caller's stream.  Nothing here allocates, synchronises or
// keeps state between calls.

#include "gdn.h"
#include "gdn_internal.hpp"
#include "gdn_prefill_args.hpp"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool head_size(int d) { return d == 64 || d == 128; }
// Every kernel takes any pairing of the two head sizes.
bool supported_head(int d_k, int d_v) { return head_size(d_k) && head_size(d_v); }

int check_launch(hipError_t e) { return e == hipSuccess ? GDN_OK : GDN_ERR_HIP; }

// The bytes [p, p + n) of one array of a call; `out` if the call writes it.
struct Span {
    const void* p;
    size_t n;
    bool out;
};

// GDN_ERR_ALIAS if an array the call writes shares a byte with any other of
// its arrays (inputs may share memory with each other); NULL or empty arrays
// take no part.
int check_disjoint(const Span* s, int n) {
    for (int i = 0; i < n; ++i)
        for (int j = i + 1; j < n; ++j) {
            if (!(s[i].out || s[j].out) || !s[i].p || !s[j].p || s[i].n == 0 || s[j].n == 0) continue;
            const uintptr_t a = reinterpret_cast<uintptr_t>(s[i].p), b = reinterpret_cast<uintptr_t>(s[j].p);
            if (a < b + s[j].n && b < a + s[i].n) return GDN_ERR_ALIAS;
        }
    return GDN_OK;
}

// The arrays of a token-kernel call (q, k [B,T,H_qk,d_k]; v, o [B,T,H,d_v];
// g, beta; the K-slot state and the final state), plus the accepted lengths
// and the error flag of a fused rollback.
int check_recurrent_disjoint(int B, int T, int H, int H_qk, int d_k, int d_v, int qkv_dtype, int gate,
                             int K, const void* q, const void* k, const void* v, const void* g,
                             const void* beta, const void* state, const void* final_state, const void* o,
                             const void* accepted = nullptr, const void* err_flag = nullptr) {
    const size_t bt = static_cast<size_t>(B) * T, e = qkv_dtype == GDN_BF16 ? 2 : 4;
    const size_t tile = static_cast<size_t>(d_k) * d_v * 4;
    const Span s[] = {
        {q, bt * H_qk * d_k * e, false},
        {k, bt * H_qk * d_k * e, false},
        {v, bt * H * d_v * e, false},
        {g, bt * H * (gate == GDN_GATE_KEY ? d_k : 1) * 4, false},
        {beta, bt * H * 4, false},
        {accepted, static_cast<size_t>(B) * 4, false},
        {o, bt * H * d_v * 4, true},
        {state, static_cast<size_t>(B) * H * K * tile, true},
        {final_state, static_cast<size_t>(B) * H * tile, true},
        {err_flag, 4, true},
    };
    return check_disjoint(s, sizeof(s) / sizeof(s[0]));
}

// H value heads read H_qk query/key heads (H a multiple of H_qk).
int validate_heads(int H, int H_qk, int head_map) {
    if (H_qk < 1 || (H > 0 && H % H_qk != 0)) return GDN_ERR_SHAPE;
    if (head_map != GDN_HEADS_GROUPED && head_map != GDN_HEADS_TILED) return GDN_ERR_UNSUPPORTED;
    return GDN_OK;
}

int validate_recurrent(int B, int T, int H, int d_k, int d_v, int qkv_dtype, int gate, int K,
                       const void* q, const void* k, const void* v, const float* g,
                       const float* beta, const float* state, const float* final_state,
                       const float* o) {
    if (B < 0 || T < 0 || H < 0 || K < 1) return GDN_ERR_SHAPE;
    // Empty token arrays (T == 0) and empty batches may come with NULL pointers.
    const bool tokens = B > 0 && H > 0 && T > 0;
    if (tokens && (!q || !k || !v || !g || !beta || !o)) return GDN_ERR_NULL;
    if (B > 0 && H > 0 && !state) return GDN_ERR_NULL;
    if (!supported_head(d_k, d_v)) return GDN_ERR_UNSUPPORTED;
    if (qkv_dtype != GDN_F32 && qkv_dtype != GDN_BF16) return GDN_ERR_UNSUPPORTED;
    if (gate != GDN_GATE_HEAD && gate != GDN_GATE_KEY) return GDN_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) || !aligned16(state) ||
        !aligned16(o) || (final_state && !aligned16(final_state)))
        return GDN_ERR_UNSUPPORTED;
    return GDN_OK;
}

int launch_forward(int B, int T, int H, int H_qk, int head_map, int d_k, int d_v, int qkv_dtype,
                   int gate, int K, const void* q, const void* k, const void* v, const float* g,
                   const float* beta, float* state, float* final_state, float* o,
                   const int32_t* accepted, int32_t* err_flag, void* stream);

}  // namespace

extern "C" {

int gdn_forward_qk_broadcast(int32_t B, int32_t T, int32_t H, int32_t H_qk, int32_t head_map,
                             int32_t d_k, int32_t d_v, int32_t qkv_dtype, int32_t gate,
                             int32_t K, const void* q, const void* k, const void* v,
                             const float* g, const float* beta, float* state,
                             float* final_state, float* o, void* stream) {
    int st = validate_recurrent(B, T, H, d_k, d_v, qkv_dtype, gate, K, q, k, v, g, beta, state,
                                final_state, o);
    if (st != GDN_OK) return st;
    st = validate_heads(H, H_qk, head_map);
    if (st != GDN_OK) return st;
    if (B == 0 || H == 0) return GDN_OK;
    st = check_recurrent_disjoint(B, T, H, H_qk, d_k, d_v, qkv_dtype, gate, K, q, k, v, g, beta, state,
                                  final_state, o);
    if (st != GDN_OK) return st;
    // With no token, nothing changes unless a final_state copy is requested.
    if (T == 0 && final_state == nullptr) return GDN_OK;
    return launch_forward(B, T, H, H_qk, head_map, d_k, d_v, qkv_dtype, gate, K, q, k, v, g, beta, state,
                          final_state, o, nullptr, nullptr, stream);
}

int gdn_forward_snapshots_after_rollback(int32_t B, int32_t T, int32_t H, int32_t H_qk,
                                         int32_t head_map, int32_t d_k, int32_t d_v,
                                         int32_t qkv_dtype, int32_t gate, int32_t K,
                                         const int32_t* accepted, const void* q, const void* k,
                                         const void* v, const float* g, const float* beta,
                                         float* state, float* final_state, float* o,
                                         int32_t* err_flag, void* stream) {
    int st = validate_recurrent(B, T, H, d_k, d_v, qkv_dtype, gate, K, q, k, v, g, beta, state,
                                final_state, o);
    if (st != GDN_OK) return st;
    st = validate_heads(H, H_qk, head_map);
    if (st != GDN_OK) return st;
    if (B > 0 && !accepted) return GDN_ERR_NULL;
    if (B == 0 || H == 0) return GDN_OK;
    st = check_recurrent_disjoint(B, T, H, H_qk, d_k, d_v, qkv_dtype, gate, K, q, k, v, g, beta, state,
                                  final_state, o, accepted, err_flag);
    if (st != GDN_OK) return st;
    if (T == 0 || K == 1) {
        // no token, or a single slot (nothing to roll back; an index other
        // than 0 is only flagged): the two calls themselves
        st = gdn_rollback_select(B, H, K, d_k, d_v, accepted, state, err_flag, stream);
        if (st != GDN_OK) return st;
        return gdn_forward_qk_broadcast(B, T, H, H_qk, head_map, d_k, d_v, qkv_dtype, gate, K, q, k, v, g,
                                        beta, state, final_state, o, stream);
    }
    return launch_forward(B, T, H, H_qk, head_map, d_k, d_v, qkv_dtype, gate, K, q, k, v, g, beta, state,
                          final_state, o, accepted, err_flag, stream);
}

}  // extern "C"

namespace {

int launch_forward(int B, int T, int H, int H_qk, int head_map, int d_k, int d_v, int qkv_dtype,
                   int gate, int K, const void* q, const void* k, const void* v, const float* g,
                   const float* beta, float* state, float* final_state, float* o,
                   const int32_t* accepted, int32_t* err_flag, void* stream) {
    gdn::RecurrentArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.state = state;
    a.final_state = final_state;
    a.o = o;
    a.B = B;
    a.T = T;
    a.H = H;
    a.K = K;
    a.dk = d_k;
    a.dv = d_v;
    a.Hqk = H_qk;
    a.group = H / H_qk;
    a.tiled = head_map == GDN_HEADS_TILED;
    a.n_snap = K > 1 ? (T < K - 1 ? T : K - 1) : 0;
    a.bf16 = qkv_dtype == GDN_BF16;
    a.kda = gate == GDN_GATE_KEY;
    a.accepted = accepted;
    a.err_flag = err_flag;
    return check_launch(gdn::launch_recurrent(a, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int gdn_forward_snapshots(int32_t B, int32_t T, int32_t H, int32_t d_k, int32_t d_v,
                          int32_t qkv_dtype, int32_t gate, int32_t K, const void* q,
                          const void* k, const void* v, const float* g, const float* beta,
                          float* state, float* final_state, float* o, void* stream) {
    return gdn_forward_qk_broadcast(B, T, H, H > 0 ? H : 1, GDN_HEADS_GROUPED, d_k, d_v,
                                    qkv_dtype, gate, K, q, k, v, g, beta, state, final_state, o,
                                    stream);
}

int gdn_forward(int32_t B, int32_t T, int32_t H, int32_t d_k, int32_t d_v, int32_t qkv_dtype,
                int32_t gate, const void* q, const void* k, const void* v, const float* g,
                const float* beta, float* state, float* o, void* stream) {
    return gdn_forward_snapshots(B, T, H, d_k, d_v, qkv_dtype, gate, 1, q, k, v, g, beta, state,
                                 nullptr, o, stream);
}

int gdn_rollback_select(int32_t B, int32_t H, int32_t K, int32_t d_k, int32_t d_v,
                        const int32_t* accepted, float* state, int32_t* err_flag, void* stream) {
    if (B < 0 || H < 0 || K < 1 || d_k < 1 || d_v < 1) return GDN_ERR_SHAPE;
    if (B > 0 && (!accepted || (H > 0 && !state))) return GDN_ERR_NULL;
    const size_t tile = static_cast<size_t>(d_k) * static_cast<size_t>(d_v);
    if (tile % 4 != 0 || !aligned16(state)) return GDN_ERR_UNSUPPORTED;
    if (B == 0 || H == 0) return GDN_OK;
    const Span s[] = {{accepted, static_cast<size_t>(B) * 4, false},
                      {state, static_cast<size_t>(B) * H * K * tile * 4, true},
                      {err_flag, 4, true}};
    const int st = check_disjoint(s, 3);
    if (st != GDN_OK) return st;
    return check_launch(gdn::launch_rollback(B, H, K, tile, accepted, state, err_flag,
                                             static_cast<hipStream_t>(stream)));
}

size_t gdn_prefill_workspace_size(int32_t B, int32_t T, int32_t H, int32_t d_k, int32_t d_v,
                                  int32_t chunk) {
    if (B < 0 || T < 0 || H < 0 || chunk != 64 || !supported_head(d_k, d_v)) return 0;
    return gdn::prefill_workspace_bytes(B, T, H, d_k, d_v);
}

size_t gdn_prefill_workspace_size_ex(int32_t B, int32_t T, int32_t H, int32_t d_k, int32_t d_v,
                                     int32_t chunk, int32_t qkv_dtype, int32_t gate) {
    if (B < 0 || T < 0 || H < 0 || chunk != 64 || !supported_head(d_k, d_v)) return 0;
    if ((qkv_dtype != GDN_F32 && qkv_dtype != GDN_BF16) || (gate != GDN_GATE_HEAD && gate != GDN_GATE_KEY))
        return 0;
    return gdn::prefill_workspace_bytes(B, T, H, d_k, d_v, gate == GDN_GATE_KEY, qkv_dtype == GDN_F32);
}

}  // extern "C"

namespace {

// Every check gdn_prefill_chunked_ex makes before it launches anything.
int check_prefill_ex(int32_t B, int32_t T, int32_t H, int32_t H_qk, int32_t head_map, int32_t d_k,
                     int32_t d_v, int32_t chunk, int32_t qkv_dtype, int32_t gate, int32_t K, const void* q,
                     const void* k, const void* v, const float* g, const float* beta, const float* state,
                     const float* final_state, const float* o, const void* workspace,
                     size_t workspace_bytes) {
    if (B < 0 || T < 0 || H < 0 || chunk < 1 || K < 1) return GDN_ERR_SHAPE;
    const int hs = validate_heads(H, H_qk, head_map);
    if (hs != GDN_OK) return hs;
    const bool tokens = B > 0 && H > 0 && T > 0;
    if (tokens && (!q || !k || !v || !g || !beta || !o)) return GDN_ERR_NULL;
    if (B > 0 && H > 0 && !state) return GDN_ERR_NULL;
    if (chunk != 64 || !supported_head(d_k, d_v)) return GDN_ERR_UNSUPPORTED;
    if (qkv_dtype != GDN_F32 && qkv_dtype != GDN_BF16) return GDN_ERR_UNSUPPORTED;
    if (gate != GDN_GATE_HEAD && gate != GDN_GATE_KEY) return GDN_ERR_UNSUPPORTED;
    // (KDA reads g in 16-byte pieces; GDA reads it as single floats)
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || (gate == GDN_GATE_KEY && !aligned16(g)) ||
        !aligned16(state) || !aligned16(o) || (final_state && !aligned16(final_state)))
        return GDN_ERR_UNSUPPORTED;
    if (B == 0 || H == 0) return GDN_OK;
    if (T == 0)
        return check_recurrent_disjoint(B, T, H, H_qk, d_k, d_v, qkv_dtype, gate, K, q, k, v, g, beta, state,
                                        K > 1 ? final_state : nullptr, o);
    // the kernels address one sequence's [T,H,d] rows with 32-bit byte offsets
    if (static_cast<int64_t>(T) * H * (d_k > d_v ? d_k : d_v) * 4 >= (int64_t(1) << 31))
        return GDN_ERR_UNSUPPORTED;
    const size_t need = gdn::prefill_workspace_bytes(B, T, H, d_k, d_v, gate == GDN_GATE_KEY, qkv_dtype == GDN_F32);
    {
        // the workspace bytes the kernels write, against every other array
        const size_t bt = static_cast<size_t>(B) * T, e = qkv_dtype == GDN_BF16 ? 2 : 4;
        const Span s[] = {
            {workspace, need, true},
            {q, bt * H_qk * d_k * e, false},
            {k, bt * H_qk * d_k * e, false},
            {v, bt * H * d_v * e, false},
            {g, bt * H * (gate == GDN_GATE_KEY ? d_k : 1) * 4, false},
            {beta, bt * H * 4, false},
            {o, bt * H * d_v * 4, true},
            {state, static_cast<size_t>(B) * H * K * d_k * d_v * 4, true},
            {K > 1 ? final_state : nullptr, static_cast<size_t>(B) * H * d_k * d_v * 4, true},
        };
        const int st = check_disjoint(s, sizeof(s) / sizeof(s[0]));
        if (st != GDN_OK) return st;
    }
    if (workspace == nullptr || workspace_bytes < need ||
        (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return GDN_ERR_WORKSPACE;
    return GDN_OK;
}

// gdn_prefill_chunked_ex after check_prefill_ex, with the rollback of the
// previous draft fused into the chain when `accepted` is given (K > 1, T > 0).
int launch_prefill_ex(int32_t B, int32_t T, int32_t H, int32_t H_qk, int32_t head_map, int32_t d_k,
                      int32_t d_v, int32_t qkv_dtype, int32_t gate, int32_t K, const void* q, const void* k,
                      const void* v, const float* g, const float* beta, float* state, float* final_state,
                      float* o, void* workspace, const int32_t* accepted, int32_t* err_flag, void* stream) {
    if (B == 0 || H == 0) return GDN_OK;
    if (T == 0) {
        // no token: only a requested final_state copy of slot 0 remains, which
        // is exactly the recurrent entry point's T = 0 case
        if (K == 1 || final_state == nullptr) return GDN_OK;
        return gdn_forward_qk_broadcast(B, 0, H, H_qk, head_map, d_k, d_v, qkv_dtype, gate, K,
                                        nullptr, nullptr, nullptr, nullptr, nullptr, state,
                                        final_state, nullptr, stream);
    }
    gdn::PrefillArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.state = state;
    a.final_state = K > 1 ? final_state : nullptr;
    a.o = o;
    a.workspace = workspace;
    a.cu_seqlens = nullptr;
    a.B = B;
    a.T = T;
    a.H = H;
    a.dk = d_k;
    a.dv = d_v;
    a.Hqk = H_qk;
    a.group = H / H_qk;
    a.tiled = head_map == GDN_HEADS_TILED;
    a.K = K;
    a.kda = gate == GDN_GATE_KEY;
    a.f32 = qkv_dtype == GDN_F32;
    a.accepted = accepted;
    a.err_flag = err_flag;
    return check_launch(gdn::launch_prefill(a, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int gdn_prefill_chunked_ex(int32_t B, int32_t T, int32_t H, int32_t H_qk, int32_t head_map,
                           int32_t d_k, int32_t d_v, int32_t chunk, int32_t qkv_dtype, int32_t gate,
                           int32_t K, const void* q, const void* k, const void* v, const float* g,
                           const float* beta, float* state, float* final_state, float* o,
                           void* workspace, size_t workspace_bytes, void* stream) {
    const int st = check_prefill_ex(B, T, H, H_qk, head_map, d_k, d_v, chunk, qkv_dtype, gate, K, q, k, v, g,
                                    beta, state, final_state, o, workspace, workspace_bytes);
    if (st != GDN_OK) return st;
    return launch_prefill_ex(B, T, H, H_qk, head_map, d_k, d_v, qkv_dtype, gate, K, q, k, v, g, beta, state,
                             final_state, o, workspace, nullptr, nullptr, stream);
}

int gdn_prefill_chunked_ex_after_rollback(int32_t B, int32_t T, int32_t H, int32_t H_qk,
                                          int32_t head_map, int32_t d_k, int32_t d_v, int32_t chunk,
                                          int32_t qkv_dtype, int32_t gate, int32_t K,
                                          const int32_t* accepted, const void* q, const void* k,
                                          const void* v, const float* g, const float* beta,
                                          float* state, float* final_state, float* o,
                                          void* workspace, size_t workspace_bytes, int32_t* err_flag,
                                          void* stream) {
    if (B > 0 && !accepted) return GDN_ERR_NULL;
    int st = check_prefill_ex(B, T, H, H_qk, head_map, d_k, d_v, chunk, qkv_dtype, gate, K, q, k, v, g, beta,
                              state, final_state, o, workspace, workspace_bytes);
    if (st != GDN_OK) return st;
    if (B == 0 || H == 0) return GDN_OK;
    st = check_recurrent_disjoint(B, T, H, H_qk, d_k, d_v, qkv_dtype, gate, K, q, k, v, g, beta, state,
                                  K > 1 ? final_state : nullptr, o, accepted, err_flag);
    if (st != GDN_OK) return st;
    if (T == 0 || K == 1) {
        // no token, or a single slot (nothing to roll back; an index other
        // than 0 is only flagged): the two calls themselves
        st = gdn_rollback_select(B, H, K, d_k, d_v, accepted, state, err_flag, stream);
        if (st != GDN_OK) return st;
        return launch_prefill_ex(B, T, H, H_qk, head_map, d_k, d_v, qkv_dtype, gate, K, q, k, v, g, beta, state,
                                 final_state, o, workspace, nullptr, nullptr, stream);
    }
    return launch_prefill_ex(B, T, H, H_qk, head_map, d_k, d_v, qkv_dtype, gate, K, q, k, v, g, beta, state,
                             final_state, o, workspace, accepted, err_flag, stream);
}

int gdn_prefill_chunked_snapshots(int32_t B, int32_t T, int32_t H, int32_t H_qk,
                                  int32_t head_map, int32_t d_k, int32_t d_v, int32_t chunk,
                                  int32_t K, const void* q, const void* k, const void* v,
                                  const float* g, const float* beta, float* state,
                                  float* final_state, float* o, void* workspace,
                                  size_t workspace_bytes, void* stream) {
    return gdn_prefill_chunked_ex(B, T, H, H_qk, head_map, d_k, d_v, chunk, GDN_BF16, GDN_GATE_HEAD,
                                  K, q, k, v, g, beta, state, final_state, o, workspace,
                                  workspace_bytes, stream);
}

int gdn_prefill_chunked_qk_broadcast(int32_t B, int32_t T, int32_t H, int32_t H_qk,
                                     int32_t head_map, int32_t d_k, int32_t d_v, int32_t chunk,
                                     const void* q, const void* k, const void* v,
                                     const float* g, const float* beta, float* state, float* o,
                                     void* workspace, size_t workspace_bytes, void* stream) {
    return gdn_prefill_chunked_snapshots(B, T, H, H_qk, head_map, d_k, d_v, chunk, 1, q, k, v, g,
                                         beta, state, nullptr, o, workspace, workspace_bytes,
                                         stream);
}

size_t gdn_prefill_varlen_workspace_size_ex(int32_t N, int32_t total_T, int32_t H, int32_t d_k,
                                            int32_t d_v, int32_t chunk, int32_t qkv_dtype,
                                            int32_t gate) {
    if (N < 0 || total_T < 0 || H < 0 || chunk != 64 || !supported_head(d_k, d_v)) return 0;
    if (qkv_dtype != GDN_F32 && qkv_dtype != GDN_BF16) return 0;
    if (gate != GDN_GATE_HEAD && gate != GDN_GATE_KEY) return 0;
    return gdn::prefill_varlen_workspace_bytes(N, total_T, H, d_k, d_v, gate == GDN_GATE_KEY,
                                               qkv_dtype == GDN_F32);
}

size_t gdn_prefill_varlen_workspace_size(int32_t N, int32_t total_T, int32_t H, int32_t d_k,
                                         int32_t d_v, int32_t chunk) {
    return gdn_prefill_varlen_workspace_size_ex(N, total_T, H, d_k, d_v, chunk, GDN_BF16, GDN_GATE_HEAD);
}

int gdn_prefill_chunked_varlen_ex(int32_t N, int32_t total_T, int32_t H, int32_t H_qk,
                                  int32_t head_map, int32_t d_k, int32_t d_v, int32_t chunk,
                                  int32_t qkv_dtype, int32_t gate, const int32_t* cu_seqlens,
                                  const void* q, const void* k, const void* v, const float* g,
                                  const float* beta, float* state, float* o, void* workspace,
                                  size_t workspace_bytes, void* stream) {
    if (N < 0 || total_T < 0 || H < 0 || chunk < 1) return GDN_ERR_SHAPE;
    const int hs = validate_heads(H, H_qk, head_map);
    if (hs != GDN_OK) return hs;
    if (N > 0 && !cu_seqlens) return GDN_ERR_NULL;
    const bool tokens = N > 0 && H > 0 && total_T > 0;
    if (tokens && (!q || !k || !v || !g || !beta || !o)) return GDN_ERR_NULL;
    if (N > 0 && H > 0 && !state) return GDN_ERR_NULL;
    if (chunk != 64 || !supported_head(d_k, d_v)) return GDN_ERR_UNSUPPORTED;
    if (qkv_dtype != GDN_F32 && qkv_dtype != GDN_BF16) return GDN_ERR_UNSUPPORTED;
    if (gate != GDN_GATE_HEAD && gate != GDN_GATE_KEY) return GDN_ERR_UNSUPPORTED;
    // (KDA reads g in 16-byte pieces; GDA reads it as single floats)
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || (gate == GDN_GATE_KEY && !aligned16(g)) ||
        !aligned16(state) || !aligned16(o))
        return GDN_ERR_UNSUPPORTED;
    if (N == 0 || H == 0 || total_T == 0) return GDN_OK;
    // the kernels address one sequence's [T,H,d] rows with 32-bit byte offsets
    if (static_cast<int64_t>(total_T) * H * (d_k > d_v ? d_k : d_v) * 4 >= (int64_t(1) << 31))
        return GDN_ERR_UNSUPPORTED;
    const bool kda = gate == GDN_GATE_KEY, f32 = qkv_dtype == GDN_F32;
    const size_t need = gdn::prefill_varlen_workspace_bytes(N, total_T, H, d_k, d_v, kda, f32);
    {
        const size_t t = static_cast<size_t>(total_T), e = f32 ? 4 : 2;
        const Span s[] = {
            {cu_seqlens, (static_cast<size_t>(N) + 1) * 4, false},
            {q, t * H_qk * d_k * e, false},
            {k, t * H_qk * d_k * e, false},
            {v, t * H * d_v * e, false},
            {g, t * H * (kda ? d_k : 1) * 4, false},
            {beta, t * H * 4, false},
            {o, t * H * d_v * 4, true},
            {state, static_cast<size_t>(N) * H * d_k * d_v * 4, true},
            {workspace, need, true},
        };
        const int st = check_disjoint(s, sizeof(s) / sizeof(s[0]));
        if (st != GDN_OK) return st;
    }
    if (workspace == nullptr || workspace_bytes < need ||
        (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return GDN_ERR_WORKSPACE;
    gdn::PrefillArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.state = state;
    a.o = o;
    a.workspace = workspace;
    a.cu_seqlens = cu_seqlens;
    a.final_state = nullptr;
    a.K = 1;
    a.kda = kda;
    a.f32 = f32;
    a.B = N;
    a.T = total_T;
    a.H = H;
    a.dk = d_k;
    a.dv = d_v;
    a.Hqk = H_qk;
    a.group = H / H_qk;
    a.tiled = head_map == GDN_HEADS_TILED;
    return check_launch(gdn::launch_prefill(a, static_cast<hipStream_t>(stream)));
}

int gdn_prefill_chunked_varlen(int32_t N, int32_t total_T, int32_t H, int32_t H_qk,
                               int32_t head_map, int32_t d_k, int32_t d_v, int32_t chunk,
                               const int32_t* cu_seqlens, const void* q, const void* k,
                               const void* v, const float* g, const float* beta, float* state,
                               float* o, void* workspace, size_t workspace_bytes, void* stream) {
    return gdn_prefill_chunked_varlen_ex(N, total_T, H, H_qk, head_map, d_k, d_v, chunk, GDN_BF16,
                                         GDN_GATE_HEAD, cu_seqlens, q, k, v, g, beta, state, o,
                                         workspace, workspace_bytes, stream);
}

int gdn_prefill_chunked(int32_t B, int32_t T, int32_t H, int32_t d_k, int32_t d_v,
                        int32_t chunk, const void* q, const void* k, const void* v,
                        const float* g, const float* beta, float* state, float* o,
                        void* workspace, size_t workspace_bytes, void* stream) {
    return gdn_prefill_chunked_qk_broadcast(B, T, H, H > 0 ? H : 1, GDN_HEADS_GROUPED, d_k, d_v,
                                            chunk, q, k, v, g, beta, state, o, workspace,
                                            workspace_bytes, stream);
}

size_t gdn_prefill_kda_workspace_size(int32_t B, int32_t T, int32_t H, int32_t d_k, int32_t d_v,
                                      int32_t chunk) {
    return gdn_prefill_workspace_size_ex(B, T, H, d_k, d_v, chunk, GDN_BF16, GDN_GATE_KEY);
}

int gdn_prefill_chunked_kda(int32_t B, int32_t T, int32_t H, int32_t H_qk, int32_t head_map,
                            int32_t d_k, int32_t d_v, int32_t chunk, const void* q, const void* k,
                            const void* v, const float* g, const float* beta, float* state,
                            float* o, void* workspace, size_t workspace_bytes, void* stream) {
    return gdn_prefill_chunked_ex(B, T, H, H_qk, head_map, d_k, d_v, chunk, GDN_BF16, GDN_GATE_KEY, 1,
                                  q, k, v, g, beta, state, nullptr, o, workspace, workspace_bytes,
                                  stream);
}

const char* gdn_status_str(int status) {
    switch (status) {
        case GDN_OK: return "ok";
        case GDN_ERR_NULL: return "a required pointer is NULL";
        case GDN_ERR_SHAPE: return "invalid size (negative B/T/H, K < 1, chunk < 1 or H_qk not dividing H)";
        case GDN_ERR_UNSUPPORTED:
            return "unsupported configuration (head size, dtype, gate mode, chunk or alignment)";
        case GDN_ERR_WORKSPACE: return "prefill workspace missing, misaligned or too small";
        case GDN_ERR_HIP: return "HIP runtime error at launch";
        case GDN_ERR_SCRATCH:
            return "prefill workspace exceeds the library's fixed scratch array (GDN_PREFILL_SCRATCH_BYTES)";
        case GDN_ERR_ALIAS: return "an array the call writes overlaps another of its arrays";
        default: return "unknown status";
    }
}

}  // extern "C"
