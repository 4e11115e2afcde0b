/*
 * gdn.h -- C ABI of the MI355X (gfx950) gated delta net (GDN) library.
 *
 * The operation (the gated delta rule; the commit-log pages name it as the
 * GGML_OP_GATED_DELTA_NET recurrence without writing it out -- llama.cpp
 * commit log, tag b9752, bullet "metal : add Metal backend for
 * GGML_OP_GATED_DELTA_NET"): per sequence b and head h the state S is a
 * d_k x d_v float32 matrix (row i = key index, column j = value index).  For
 * each token t in order:
 *
 *   decay    GDA: S <- exp(g_t) S            (one log-gate per head and token)
 *            KDA: S[i,:] <- exp(g_t[i]) S[i,:]  (one log-gate per key row)
 *   delta    u = S^T k_t,   w = beta_t (v_t - u),   S <- S + k_t w^T
 *   readout  o_t = S^T q_t   (the state after this token's update)
 *
 * No scale is applied to q; a caller that wants 1/sqrt(d_k) scales q first.
 *
 * Conventions shared by every entry point:
 *  - Every tensor pointer is a DEVICE pointer to a contiguous row-major array
 *    (last axis contiguous) owned by the caller.  The library keeps no
 *    global state beyond each device's compute-unit count, read once per
 *    device to choose a launch shape, and the address of each device's
 *    scratch array for gdn_prefill_chunked_ex_noalloc; it never
 *    synchronises and launches only on `stream` (a hipStream_t passed as
 *    void*; NULL means the default stream).
 *  - Layouts: q, k [B,T,H,d_k]; v, o [B,T,H,d_v]; g [B,T,H] (GDA) or
 *    [B,T,H,d_k] (KDA); beta [B,T,H]; state [B,H,K,d_k,d_v] (slot 0 = input).
 *    q/k/v are float32 or bfloat16 (qkv_dtype); g, beta, state and o are
 *    float32.  g holds LOG-gates (the decay is exp(g)).
 *  - Head sizes d_k and d_v each 64 or 128, in any pairing (the sizes the
 *    pages' fused kernels support; other sizes are reported as unsupported,
 *    never computed).
 *  - Empty problems (B, H or T equal to 0) are valid; the pointers of empty
 *    arrays may then be NULL.
 *  - All validation happens on the host before any launch.  On an error
 *    nothing is launched and no output is touched.  A launch failure is
 *    reported as GDN_ERR_HIP.  Calls are asynchronous.
 *  - No array a call writes (o, state, final_state, the workspace,
 *    err_flag) may share a byte with any other of its arrays; the host
 *    checks the byte ranges the call's sizes give and returns GDN_ERR_ALIAS
 *    (inputs may share memory with each other).
 *    NaN/Inf inputs propagate; they are not checked.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDN_OK = 0,
    GDN_ERR_NULL = 1,        /* a required pointer is NULL                      */
    GDN_ERR_SHAPE = 2,       /* a size is negative, K < 1, chunk < 1, or H_qk
                                does not divide H                               */
    GDN_ERR_UNSUPPORTED = 3, /* d_k or d_v not in {64,128}, bad dtype/gate     */
    GDN_ERR_WORKSPACE = 4,   /* prefill workspace missing or too small          */
    GDN_ERR_HIP = 5,         /* the HIP runtime reported a launch error         */
    GDN_ERR_SCRATCH = 6,     /* the problem needs more than the library's fixed
                                scratch array (gdn_prefill_chunked_ex_noalloc)  */
    GDN_ERR_ALIAS = 7        /* an array the call writes (o, state, final_state,
                                workspace, err_flag) overlaps another array of
                                the call                                        */
} gdn_status;

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype; /* dtype of q, k, v only */
typedef enum { GDN_GATE_HEAD = 0 /* GDA */, GDN_GATE_KEY = 1 /* KDA */ } gdn_gate;

/*
 * Decode / multi-token forward with a single state slot, in place: the fused
 * recurrence of the llama.cpp commit log, tag b9752, bullet "metal : add
 * Metal backend for GGML_OP_GATED_DELTA_NET" (GDA or KDA gates, head sizes
 * 64 and 128), with the single-slot state that the koboldcpp commit log, tag
 * v1.113.1, bullet "metal: add GDN partial rollback", keeps for K = 1.
 * state [B,H,d_k,d_v] holds S_0 on entry and S_T on return; o [B,T,H,d_v].
 * Equivalent to gdn_forward_snapshots with K = 1 and final_state = NULL
 * (same kernel, bit-identical results).  T = 0 leaves the state unchanged.
 */
int gdn_forward(int32_t B, int32_t T, int32_t H, int32_t d_k, int32_t d_v, int32_t qkv_dtype,
                int32_t gate, const void* q, const void* k, const void* v, const float* g,
                const float* beta, float* state, float* o, void* stream);

/*
 * Forward with K snapshot slots for speculative verification (koboldcpp
 * commit log, tag v1.113.1, bullet "metal: add GDN partial rollback": K is
 * the slot count, the input state is read from slot 0 of the 3-D state
 * tensor, intermediate states are written to the slots inside the token
 * loop, K = 1 keeps the single-slot behaviour).
 * state [B,H,K,d_k,d_v].  Writes:
 *   K == 1 : slot 0 <- S_T (exactly gdn_forward);
 *   K  > 1 : slot t <- S_t (the state after the first t tokens) for
 *            1 <= t <= min(T, K-1); slot 0 and slots above T are untouched;
 *   final_state [B,H,d_k,d_v] <- S_T when final_state is not NULL.
 *   o [B,T,H,d_v] for every token.
 */
int gdn_forward_snapshots(int32_t B, int32_t T, int32_t H, int32_t d_k, int32_t d_v,
                          int32_t qkv_dtype, int32_t gate, int32_t K, const void* q,
                          const void* k, const void* v, const float* g, const float* beta,
                          float* state, float* final_state, float* o, void* stream);

/*
 * Rollback to the accepted draft length (koboldcpp commit log, tag v1.113.1,
 * bullets "llama: allow partial seq_rm for GDN models for speculative
 * decoding" -- roll back up to draft_max by keeping the GDN intermediates --
 * and "llama-memory-recurrent: clear rs_idx in clear").
 * accepted: device int32 [B].  For each sequence b, a = accepted[b]:
 *   1 <= a <= K-1 : slot 0 of every head <- slot a, bit for bit;
 *   a == 0        : no change;
 *   a < 0, a >= K : the sequence is left untouched and, when err_flag is not
 *                   NULL, *err_flag (a device int32 the caller zeroes) is
 *                   set to 1.
 * state [B,H,K,d_k,d_v].  Any d_k, d_v >= 1 with d_k*d_v a multiple of 4.
 */
int gdn_rollback_select(int32_t B, int32_t H, int32_t K, int32_t d_k, int32_t d_v,
                        const int32_t* accepted, float* state, int32_t* err_flag, void* stream);

/*
 * The rollback of the previous draft fused into the next verification: the
 * results of gdn_rollback_select(accepted) followed by
 * gdn_forward_qk_broadcast on the same state, in one launch (koboldcpp
 * commit log, tag v1.113.1, bullets "llama: allow partial seq_rm for GDN
 * models for speculative decoding" and "metal: add GDN partial rollback":
 * the accepted intermediate state becomes the input of the next step).
 * For each sequence b with a = accepted[b] in 1..K-1, every head reads its
 * input state from slot a and also copies it to slot 0, bit for bit; a == 0
 * reads slot 0; an index outside 0..K-1 sets *err_flag (a device int32 the
 * caller zeroes; may be NULL) and the sequence starts from slot 0, as after
 * a rollback that left it untouched.  Then slots 1..min(T, K-1), o and
 * final_state are written as by gdn_forward_qk_broadcast (K = 1: the final
 * state goes to slot 0).  Every argument, layout and error as there, plus
 * accepted (device int32 [B]; NULL with B > 0 -> GDN_ERR_NULL).  The
 * results are bit-identical to the two calls.  With T = 0 or K = 1 (one
 * slot: nothing to roll back, an index other than 0 is only flagged) the
 * entry point makes the two calls itself.
 */
int gdn_forward_snapshots_after_rollback(int32_t B, int32_t T, int32_t H, int32_t H_qk,
                                         int32_t head_map, int32_t d_k, int32_t d_v,
                                         int32_t qkv_dtype, int32_t gate, int32_t K,
                                         const int32_t* accepted, const void* q, const void* k,
                                         const void* v, const float* g, const float* beta,
                                         float* state, float* final_state, float* o,
                                         int32_t* err_flag, void* stream);

/*
 * Chunked prefill (llama.cpp commit log, tag b9752, bullet "llama : enable
 * chunked fused GDN path"; the chunk algebra is the WY/UT form of the same
 * recurrence and gives the same result up to rounding).
 * GDA only, q/k/v bfloat16, d_k and d_v in {64,128}, chunk = 64, any T >= 0
 * with T*H*max(d_k,d_v)*4 < 2^31 bytes per sequence (a short final chunk behaves as if
 * padded with beta = 0, g = 0, k = q = v = 0).
 * state [B,H,d_k,d_v] float32 holds S_0 on entry and S_T on return;
 * o [B,T,H,d_v] float32.  Contractions run on bf16 MFMA with float32
 * accumulation; the carried state stays float32.
 * workspace: device memory of at least gdn_prefill_workspace_size(...)
 * bytes, 256-byte aligned, owned by the caller; its contents on entry are
 * ignored and on return are unspecified.
 */
size_t gdn_prefill_workspace_size(int32_t B, int32_t T, int32_t H, int32_t d_k, int32_t d_v,
                                  int32_t chunk);
int gdn_prefill_chunked(int32_t B, int32_t T, int32_t H, int32_t d_k, int32_t d_v,
                        int32_t chunk, const void* q, const void* k, const void* v,
                        const float* g, const float* beta, float* state, float* o,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * q/k shared between value heads, without materialising the repeats
 * (llama.cpp commit log, tag b9752, bullet "models : avoid Q and K repeats
 * when using fused GDA").  H value heads (v, g, beta, state, o) read H_qk
 * query/key heads, H a multiple of H_qk, in one of two orders (the same
 * page's bullet "reorder v heads for linear attention to avoid expensive
 * interleaved repeat" names both: the interleaved repeat, and the value-head
 * order that replaces it):
 */
typedef enum {
    GDN_HEADS_GROUPED = 0, /* value head h reads q/k head h / (H / H_qk)      */
    GDN_HEADS_TILED = 1    /* value head h reads q/k head h % H_qk            */
} gdn_head_map;

/*
 * gdn_forward_snapshots with shared q/k heads: q, k [B,T,H_qk,d_k]; every
 * other argument as in gdn_forward_snapshots (K = 1 is the in-place
 * single-slot forward).  The results are bit-identical to
 * gdn_forward_snapshots on q and k repeated to H heads in the given order.
 * H_qk < 1 or H not a multiple of H_qk (with H > 0) -> GDN_ERR_SHAPE;
 * head_map not a gdn_head_map -> GDN_ERR_UNSUPPORTED.
 */
int gdn_forward_qk_broadcast(int32_t B, int32_t T, int32_t H, int32_t H_qk, int32_t head_map,
                             int32_t d_k, int32_t d_v, int32_t qkv_dtype, int32_t gate,
                             int32_t K, const void* q, const void* k, const void* v,
                             const float* g, const float* beta, float* state,
                             float* final_state, float* o, void* stream);

/*
 * gdn_prefill_chunked with shared q/k heads: q, k [B,T,H_qk,d_k]; every
 * other argument, the workspace size (gdn_prefill_workspace_size with the H
 * value heads) and the errors as above.  The results are bit-identical to
 * gdn_prefill_chunked on q and k repeated to H heads in the given order.
 */
int gdn_prefill_chunked_qk_broadcast(int32_t B, int32_t T, int32_t H, int32_t H_qk,
                                     int32_t head_map, int32_t d_k, int32_t d_v, int32_t chunk,
                                     const void* q, const void* k, const void* v,
                                     const float* g, const float* beta, float* state, float* o,
                                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Chunked prefill of N sequences of different lengths packed along the
 * token axis (the variable-length batches a serving engine prefills; the
 * chunk algebra and the limits are those of gdn_prefill_chunked, with the
 * shared q/k heads of gdn_prefill_chunked_qk_broadcast; pass H_qk = H and
 * GDN_HEADS_GROUPED for plain heads).
 * cu_seqlens: DEVICE int32 [N+1]; sequence i is tokens
 *   [cu_seqlens[i], cu_seqlens[i+1]).  The host never reads it.  On the
 *   device each offset is clamped to [0, total_T] and raised to the largest
 *   offset before it, so malformed offsets shrink sequences (possibly to
 *   nothing) but never overlap them or leave [0, total_T).  Output rows of
 *   tokens outside every sequence are not written.
 * q, k [total_T,H_qk,d_k]; v, o [total_T,H,d_v]; g, beta [total_T,H]
 * (GDA log-gates); state [N,H,d_k,d_v] float32, one slot per sequence, in
 * place (an empty sequence leaves its state unchanged).
 * workspace: at least gdn_prefill_varlen_workspace_size(...) bytes, 256-byte
 * aligned, owned by the caller.  Each sequence's result is bit-identical to
 * gdn_prefill_chunked on that sequence alone.
 */
size_t gdn_prefill_varlen_workspace_size(int32_t N, int32_t total_T, int32_t H, int32_t d_k,
                                         int32_t d_v, int32_t chunk);
int gdn_prefill_chunked_varlen(int32_t N, int32_t total_T, int32_t H, int32_t H_qk,
                               int32_t head_map, int32_t d_k, int32_t d_v, int32_t chunk,
                               const int32_t* cu_seqlens, const void* q, const void* k,
                               const void* v, const float* g, const float* beta, float* state,
                               float* o, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Chunked prefill that also emits state snapshots: the slot semantics of
 * gdn_forward_snapshots (koboldcpp commit log, tag v1.113.1, bullet "metal:
 * add GDN partial rollback") computed by the chunked path of
 * gdn_prefill_chunked (llama.cpp commit log, tag b9752, bullet "llama :
 * enable chunked fused GDN path"), so that a long draft can be verified by
 * the chunked kernels and then rolled back with gdn_rollback_select.
 * state [B,H,K,d_k,d_v] float32: slot 0 is the input and, for K > 1, is not
 *   written; slot t (1 <= t <= min(T, K-1)) receives the state after t
 *   tokens; slots past T are untouched.  K == 1 writes the final state back
 *   to slot 0 (this is then exactly gdn_prefill_chunked_qk_broadcast).
 * final_state [B,H,d_k,d_v] or NULL: for K > 1, the state after all T tokens
 *   (with T == 0, a copy of slot 0).  Ignored when K == 1.
 * q, k [B,T,H_qk,d_k] and head_map as in gdn_prefill_chunked_qk_broadcast;
 * every other argument, the workspace and the limits as in
 * gdn_prefill_chunked.  K < 1 -> GDN_ERR_SHAPE.  Outputs and snapshots are
 * within the prefill tolerance of the token recurrence (the snapshots come
 * from the chunk's own W rows, advanced token by token in float32).
 */
int gdn_prefill_chunked_snapshots(int32_t B, int32_t T, int32_t H, int32_t H_qk,
                                  int32_t head_map, int32_t d_k, int32_t d_v, int32_t chunk,
                                  int32_t K, const void* q, const void* k, const void* v,
                                  const float* g, const float* beta, float* state,
                                  float* final_state, float* o, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * Chunked prefill with KDA gates: one log-gate per key row, so that row i of
 * the state decays by exp(g_t[i]) at token t (llama.cpp commit log, tag
 * b9752, bullets "metal : add Metal backend for GGML_OP_GATED_DELTA_NET" for
 * the gate kinds and "llama : enable chunked fused GDN path" for the chunked
 * path).  Arguments as in gdn_prefill_chunked_qk_broadcast, except
 * g [B,T,H,d_k] float32 log-gates and the workspace size, which comes from
 * gdn_prefill_kda_workspace_size.  Every log-gate g <= 0 (each decay at most
 * 1) is in range, however strong: within the prefill tolerance of the token
 * recurrence.  Chunks in which a key row decays by more than e^-40 across 16
 * tokens take a slower exact path for their 16 x 16 diagonal blocks.
 */
size_t gdn_prefill_kda_workspace_size(int32_t B, int32_t T, int32_t H, int32_t d_k, int32_t d_v,
                                      int32_t chunk);
int gdn_prefill_chunked_kda(int32_t B, int32_t T, int32_t H, int32_t H_qk, int32_t head_map,
                            int32_t d_k, int32_t d_v, int32_t chunk, const void* q, const void* k,
                            const void* v, const float* g, const float* beta, float* state,
                            float* o, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The general chunked prefill: every choice the specialised prefill entry
 * points fix, as arguments (llama.cpp commit log, tag b9752, bullets
 * "metal : add Metal backend for GGML_OP_GATED_DELTA_NET" -- GDA or KDA,
 * head sizes 64 and 128 -- and "llama : enable chunked fused GDN path").
 * qkv_dtype: GDN_BF16, or GDN_F32 -- q, k and v float32, rounded to bf16 for
 *   the MFMA products (round to nearest even), so that the result is the
 *   bf16 path's on the rounded inputs and within the prefill tolerance of
 *   the token recurrence on the float32 inputs.
 * gate: GDN_GATE_HEAD (g [B,T,H]) or GDN_GATE_KEY (g [B,T,H,d_k], log-gates
 *   g <= 0 as for gdn_prefill_chunked_kda).
 * K, state, final_state: as in gdn_prefill_chunked_snapshots, for GDA and
 *   for KDA (slot t then holds the state after t tokens with every key row
 *   decayed by its own gates; the same gdn_rollback_select applies).
 * q, k [B,T,H_qk,d_k] and head_map as in gdn_prefill_chunked_qk_broadcast;
 * v, o, beta as in gdn_prefill_chunked.  The workspace holds at least
 * gdn_prefill_workspace_size_ex(...) bytes (larger for KDA and for float32
 * inputs), 256-byte aligned, owned by the caller.
 */
size_t gdn_prefill_workspace_size_ex(int32_t B, int32_t T, int32_t H, int32_t d_k, int32_t d_v,
                                     int32_t chunk, int32_t qkv_dtype, int32_t gate);
int gdn_prefill_chunked_ex(int32_t B, int32_t T, int32_t H, int32_t H_qk, int32_t head_map,
                           int32_t d_k, int32_t d_v, int32_t chunk, int32_t qkv_dtype, int32_t gate,
                           int32_t K, const void* q, const void* k, const void* v, const float* g,
                           const float* beta, float* state, float* final_state, float* o,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * The rollback of the previous draft fused into a chunked prefill with
 * snapshots: the results of gdn_rollback_select(accepted) followed by
 * gdn_prefill_chunked_ex on the same state (koboldcpp commit log, tag
 * v1.113.1, bullets "llama: allow partial seq_rm for GDN models for
 * speculative decoding" and "metal: add GDN partial rollback": the accepted
 * intermediate state becomes the input of the next step).  For each
 * sequence b with a = accepted[b] in 1..K-1, every head reads its input
 * state from slot a and also copies it to slot 0, bit for bit; a == 0 reads
 * slot 0; an index outside 0..K-1 sets *err_flag (a device int32 the caller
 * zeroes; may be NULL) and the sequence starts from slot 0.  Then slots
 * 1..min(T, K-1), o and final_state are written as by
 * gdn_prefill_chunked_ex.  Every other argument, layout, limit and error as
 * there, plus accepted (device int32 [B]; NULL with B > 0 -> GDN_ERR_NULL);
 * nothing is launched when a check fails.  The results are bit-identical to
 * the two calls.  With T = 0 or K = 1 the entry point makes the two calls
 * itself.
 */
int gdn_prefill_chunked_ex_after_rollback(int32_t B, int32_t T, int32_t H, int32_t H_qk,
                                          int32_t head_map, int32_t d_k, int32_t d_v, int32_t chunk,
                                          int32_t qkv_dtype, int32_t gate, int32_t K,
                                          const int32_t* accepted, const void* q, const void* k,
                                          const void* v, const float* g, const float* beta,
                                          float* state, float* final_state, float* o,
                                          void* workspace, size_t workspace_bytes, int32_t* err_flag,
                                          void* stream);

/*
 * The variable-length prefill of gdn_prefill_chunked_varlen with the gate
 * kind and input type of gdn_prefill_chunked_ex (the same pages' bullets):
 * qkv_dtype GDN_BF16 or GDN_F32, gate GDN_GATE_HEAD (g [total_T,H]) or
 * GDN_GATE_KEY (g [total_T,H,d_k], 16-byte aligned).  Every other argument,
 * the offsets' clamping and the limits as in gdn_prefill_chunked_varlen;
 * the workspace holds at least gdn_prefill_varlen_workspace_size_ex(...)
 * bytes, 256-byte aligned.  Each sequence's result is bit-identical to
 * gdn_prefill_chunked_ex on that sequence alone (K = 1).
 */
size_t gdn_prefill_varlen_workspace_size_ex(int32_t N, int32_t total_T, int32_t H, int32_t d_k,
                                            int32_t d_v, int32_t chunk, int32_t qkv_dtype,
                                            int32_t gate);
int gdn_prefill_chunked_varlen_ex(int32_t N, int32_t total_T, int32_t H, int32_t H_qk,
                                  int32_t head_map, int32_t d_k, int32_t d_v, int32_t chunk,
                                  int32_t qkv_dtype, int32_t gate, const int32_t* cu_seqlens,
                                  const void* q, const void* k, const void* v, const float* g,
                                  const float* beta, float* state, float* o, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * gdn_prefill_chunked_ex for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Arguments, results and errors are those of
 * gdn_prefill_chunked_ex without the workspace, which is instead a fixed
 * array of GDN_PREFILL_SCRATCH_BYTES in the library's own device memory.
 * Each device that loads the library holds that array until the process
 * ends; its address is looked up on the first call on a device (with that
 * device current).  The call allocates nothing.
 * A problem whose workspace (gdn_prefill_workspace_size_ex) exceeds
 * GDN_PREFILL_SCRATCH_BYTES returns GDN_ERR_SCRATCH, and nothing is launched
 * (256 MiB holds, for example, T = 8192 tokens of 16 heads at d = 128 in
 * every gate kind and input type).  The results are bit-identical to
 * gdn_prefill_chunked_ex with a caller workspace.
 * Every call on one device uses the same array, which keeps the last call's
 * contents (the kernels write every workspace byte they read, so nothing has
 * to be cleared): calls that may overlap on one device -- on different
 * streams, or from different host threads -- race and must be ordered by the
 * caller.
 */
#define GDN_PREFILL_SCRATCH_BYTES (256u * 1024u * 1024u)
int gdn_prefill_chunked_ex_noalloc(int32_t B, int32_t T, int32_t H, int32_t H_qk, int32_t head_map,
                                   int32_t d_k, int32_t d_v, int32_t chunk, int32_t qkv_dtype,
                                   int32_t gate, int32_t K, const void* q, const void* k,
                                   const void* v, const float* g, const float* beta, float* state,
                                   float* final_state, float* o, void* stream);

/* Static description of a status code. */
const char* gdn_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
