/*
 * tailreplay.h -- C ABI of the MI355X (gfx950) Tail-Replay state-rebuild library.
 *
 * Tail-Replay rebuilds the recurrent states of a hybrid model's linear-attention
 * (Gated DeltaNet) layers on a prefix-cache hit: it replays only the last
 * k = ceil(r m) tokens of the m matched tokens, from a zero state (reading notes
 * "Tail-Replay：混合 LLM 前缀缓存的短尾重放机制", section 2.2, steps 1-4; explainer
 * "Tail-Replay: Escaping the Curse of Linear Attention in Prefix Caching for Hybrid
 * LLMs", Technical Summary, "Key Mechanisms").
 *
 * Conventions shared by every entry point
 *   - Pointers marked [device] are device memory on the current HIP device;
 *     [host] pointers are ordinary host memory.  The caller owns every buffer.
 *   - Compute entry points enqueue work on `stream` (a hipStream_t; NULL is the
 *     null stream) and return without waiting.  Setting TR_DEBUG_SYNC=1 in the
 *     environment makes them synchronise and check for errors before returning.
 *   - Every argument is validated on the host before any HIP call; a call that
 *     returns anything but TR_OK has enqueued nothing (TR_ERR_HIP excepted: a
 *     launch was attempted).  tr_last_error() then returns a message
 *     (thread-local; valid until the thread's next call).
 *   - Inputs are read-only; outputs are fully overwritten.  Buffers must not
 *     overlap, except that state_in may equal state_out.
 *   - bf16 is IEEE-style bfloat16 (1-8-7), fp32 is IEEE binary32.
 *   - No entry point allocates device memory; scratch space comes from the
 *     caller's workspace argument where one is needed.
 *   - Thread safety: calls on different streams may run concurrently.
 */
#ifndef TAILREPLAY_H
#define TAILREPLAY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TR_OK = 0,
    TR_ERR_INVALID_ARG = 1,   /* null pointer, bad size, inconsistent cu_seqlens, ... */
    TR_ERR_UNSUPPORTED = 2,   /* valid request outside the supported set (head dims, dtype) */
    TR_ERR_WORKSPACE = 3,     /* workspace smaller than the matching *_workspace_size() */
    TR_ERR_HIP = 4            /* a HIP call failed; see tr_last_error() */
} tr_status;

typedef enum {
    TR_BF16 = 0,              /* q, k, v, o in bf16; chunked MFMA path */
    TR_F32 = 1                /* q, k, v, o in fp32; fp32 arithmetic throughout */
} tr_dtype;

typedef enum {
    TR_SCHEDULE_AUTO = 0,     /* split when the request has few heads (the default) */
    TR_SCHEDULE_FUSED = 1,    /* always one workgroup per (sequence, value head) */
    TR_SCHEDULE_SPLIT = 2     /* always the split schedule (bf16) */
} tr_schedule;

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* tr_last_error(void);

/* Library version string. */
const char* tr_version(void);

/* ---------------------------------------------------------------------------------
 * Tail selection (reading notes, section 2.1 symbol table: k = ceil(r m); section 2.2
 * step 2 and its worked example: the tail is h_{m-k+1..m}, 1-based).
 *
 * tr_tail_length: k = ceil(m * r_num / r_den) in exact integer arithmetic, for
 *   m >= 0 and 0 < r_num <= r_den.  Returns k (0 when m == 0; 1 <= k <= m
 *   otherwise), or -1 for invalid arguments (then tr_last_error() says why).
 *
 * tr_tail_seqlens: for B cache hits with matched lengths m_host[b], writes
 *   cu_seqlens_host[0..B] (the packed offsets of the B tails, cu[0] = 0,
 *   cu[b+1] - cu[b] = k_b) and, if tail_start_host is not NULL, the 0-based first
 *   position m_b - k_b of each tail inside its prefix.  All arrays [host].
 *   Fails (TR_ERR_INVALID_ARG) on negative m, invalid r, or a total above INT32_MAX.
 * ------------------------------------------------------------------------------- */
int64_t tr_tail_length(int64_t m, int32_t r_num, int32_t r_den);
tr_status tr_tail_seqlens(const int64_t* m_host, int32_t B, int32_t r_num, int32_t r_den,
                          int32_t* cu_seqlens_host, int64_t* tail_start_host);

/* ---------------------------------------------------------------------------------
 * tr_gdn_replay -- varlen Gated DeltaNet recurrence over packed sequences.
 *
 * Computes, for every sequence b and value head h, token by token
 *     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,  alpha_t = exp(g_t),
 *     o_t = S_t (q_scale q_t)                     (read-out after the update)
 * starting from state_in[b, h] (or zero when state_in is NULL), and writes the final
 * state.  Reading notes, section 2.3, Eq. (1), with the state stored dv x dk so the
 * key-space operator acts from the right (the remark after Eq. (1)); the zero start is
 * section 2.2 step 2.  The read-out is not on the pages; this is the standard GDN one.
 * Value head h reads query/key head h / (Hv / Hqk).  The bf16 path evaluates the
 * recurrence in 64-token chunks (WY form) with bf16 MFMA operands, fp32 accumulation
 * and an fp32 state; its results match the token recurrence to within rounding.
 *
 * Arguments
 *   q, k        [device] [T, Hqk, dk]  dtype `dt`, row-major (dk contiguous), 16-byte aligned
 *   v           [device] [T, Hv,  dv]  dtype `dt`
 *   g           [device] [T, Hv] fp32, log alpha (<= 0 for alpha in (0, 1])
 *   beta        [device] [T, Hv] fp32
 *   cu_seqlens_host [host]   [B+1] int32: cu[0] = 0, non-decreasing, cu[B] = T
 *   cu_seqlens_dev  [device] [B+1] int32: the same values
 *   B, T, Hqk, Hv, dk, dv   sizes; B >= 1, T >= 0, Hv % Hqk == 0
 *   dt          TR_BF16 or TR_F32
 *   q_scale     > 0, multiplies q in the read-out (1 when q is pre-scaled)
 *   state_in    [device] [B, Hv, dv, dk] fp32 (dk contiguous) or NULL for the zero state
 *   state_out   [device] [B, Hv, dv, dk] fp32; may equal state_in
 *   o           [device] [T, Hv, dv] dtype `dt`, or NULL to skip the per-token outputs
 *               (state-only mode)
 *   workspace   [device] scratch of at least tr_gdn_replay_workspace_size() bytes for this
 *               request, 16-byte aligned; may be NULL when that size is 0.  Contents on
 *               entry do not matter; the call overwrites them.
 *   workspace_bytes  its size
 *   stream      hipStream_t to enqueue on
 * Schedules (bf16): the fused schedule runs one workgroup per (sequence, value head) and
 * needs no workspace.  With few heads that leaves most of the chip idle, so the split
 * schedule (default for at most 256 / (dv / 32) heads in all) first runs every chunk's
 * state-free part in parallel -- gate cumsum, K K^T, (I + L)^{-1}, W, U0, Q K^T -- into the
 * workspace, then the state scan with each state split along dv across workgroups (rows of S
 * evolve independently, section 2.3).  Both schedules give the same bits.
 * Supported: dk, dv in {64, 128}.  Empty sequences copy state_in (or write zeros).
 * Errors: TR_ERR_INVALID_ARG (sizes, pointers, cu_seqlens), TR_ERR_UNSUPPORTED (head
 *   dims), TR_ERR_WORKSPACE (workspace NULL or smaller than needed), TR_ERR_HIP.
 * Numerics: keys with beta |k|^2 <= 2 keep the operator non-expanding (reading notes,
 *   section 2.3); far outside that the recurrence itself grows without bound.
 * ------------------------------------------------------------------------------- */
tr_status tr_gdn_replay(const void* q, const void* k, const void* v,
                        const float* g, const float* beta,
                        const int32_t* cu_seqlens_host, const int32_t* cu_seqlens_dev,
                        int32_t B, int32_t T, int32_t Hqk, int32_t Hv, int32_t dk, int32_t dv,
                        tr_dtype dt, float q_scale,
                        const float* state_in, float* state_out, void* o,
                        void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------
 * tr_gdn_replay_noalloc -- tr_gdn_replay for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * Same arguments, layouts, results and errors as tr_gdn_replay, without the workspace: when
 * the schedule takes the split path, its records go to a device array of
 * TR_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on until the process
 * ends.  The call allocates nothing (no hipMalloc, no host or device allocating routine; its
 * first call on a device looks the array's address up once).  A request whose records exceed
 * TR_NOALLOC_SCRATCH_BYTES (tr_gdn_replay_workspace_size tells) returns TR_ERR_WORKSPACE before
 * anything is enqueued; the fused schedule needs no scratch at any size.  The records are
 * written in full before they are read, so nothing needs clearing between calls.
 * Every call on one GPU shares that GPU's array: calls that overlap in time on one GPU (on
 * different streams, or from different threads without ordering) race on it. */
#define TR_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
tr_status tr_gdn_replay_noalloc(const void* q, const void* k, const void* v,
                                const float* g, const float* beta,
                                const int32_t* cu_seqlens_host, const int32_t* cu_seqlens_dev,
                                int32_t B, int32_t T, int32_t Hqk, int32_t Hv, int32_t dk, int32_t dv,
                                tr_dtype dt, float q_scale,
                                const float* state_in, float* state_out, void* o, void* stream);

/* Bytes of workspace tr_gdn_replay needs for this request under the current schedule
 * (0 when it needs none).  Arguments as for tr_gdn_replay; T is cu_seqlens_host[B].
 * Returns 0 and sets tr_last_error() for invalid arguments. */
size_t tr_gdn_replay_workspace_size(const int32_t* cu_seqlens_host, int32_t B, int32_t Hqk, int32_t Hv,
                                    int32_t dk, int32_t dv, tr_dtype dt);

/* Process-wide schedule of tr_gdn_replay's bf16 path (TR_SCHEDULE_AUTO at load).  Query the
 * workspace size after changing it.  Returns TR_ERR_INVALID_ARG for an unknown value. */
tr_status tr_gdn_set_schedule(tr_schedule schedule);
tr_schedule tr_gdn_get_schedule(void);

/* ---------------------------------------------------------------------------------
 * tr_gdn_transition -- the product of the transition operators of a replayed span.
 *
 * For every sequence b and value head h, over the n tokens of sequence b, computes
 *     Phi[b, h] = T_1 T_2 ... T_n,   T_t = alpha_t (I - beta_t k_t k_t^T):
 * the recurrence of tr_gdn_replay started from S = I with all values zero.  By the linearity
 * of the recurrence in its start (reading notes, section 2.3: S_m splits into the start
 * carried through the operators plus the replayed part from zero), a state S_a before the
 * span continues as
 *     S_m = S_a Phi + S_hat_m,
 * where S_hat_m is tr_gdn_replay of the span from zero; so E_m = S_a Phi is exactly the
 * error of replaying from zero, and Phi composes checkpoints (tr_state_compose).
 *
 * The decays multiply to exp(sum g), which leaves the fp32 range after a few thousand
 * tokens at typical gates.  With log_scale_out non-NULL the decay is kept apart:
 *     phi_out = (I - beta_1 k_1 k_1^T) ... (I - beta_n k_n k_n^T),  log_scale_out = sum_t g_t,
 * and Phi = exp(log_scale_out) phi_out.  With log_scale_out NULL, phi_out = Phi directly.
 *
 * Arguments
 *   k, g, beta, cu_seqlens_host, cu_seqlens_dev, B, T, Hqk, Hv, dt
 *                 as for tr_gdn_replay (no q and no v: they do not enter Phi)
 *   d             dk = dv = d, in {64, 128}
 *   phi_out       [device] [B, Hv, d, d] fp32 (row-major)
 *   log_scale_out [device] [B, Hv] fp32, or NULL (see above)
 *   workspace     [device] scratch of at least tr_gdn_transition_workspace_size() bytes,
 *                 16-byte aligned; may be NULL when that size is 0.  Contents on entry do
 *                 not matter.
 *   workspace_bytes  its size
 *   stream        hipStream_t to enqueue on
 * Arithmetic is fp32 token by token for both input types (bf16 keys are converted
 * exactly): a long product of operators keeps every rounding it meets, so the chunked bf16
 * path is not used here.  The decays are scalars and are kept out of the matrix product;
 * with log_scale_out NULL, exp(sum g) is applied once at the end.  The product is
 * associative, so with few (sequence, head) pairs each span is cut into segments that run
 * side by side from I, and each head's segment products are then multiplied in order (fp32
 * MFMA); the cut depends only on the lengths, Hv and d.  An empty sequence gives phi_out = I
 * (and log scale 0).
 * Errors: as for tr_gdn_replay (TR_ERR_WORKSPACE for a missing or short workspace).
 * ------------------------------------------------------------------------------- */
tr_status tr_gdn_transition(const void* k, const float* g, const float* beta,
                            const int32_t* cu_seqlens_host, const int32_t* cu_seqlens_dev,
                            int32_t B, int32_t T, int32_t Hqk, int32_t Hv, int32_t d,
                            tr_dtype dt, float* phi_out, float* log_scale_out,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace tr_gdn_transition needs for this request (0 when it needs none).
 * Arguments as for tr_gdn_transition; T is cu_seqlens_host[B].  Returns 0 and sets
 * tr_last_error() for invalid arguments. */
size_t tr_gdn_transition_workspace_size(const int32_t* cu_seqlens_host, int32_t B, int32_t Hqk, int32_t Hv,
                                        int32_t d, tr_dtype dt);

/* ---------------------------------------------------------------------------------
 * tr_state_compose -- out[n] = exp(log_scale[n]) S_c[n] phi[n] + S_hat[n] for n < N.
 *
 * The composition of reading notes section 2.3 (start carried through the span plus the
 * replayed part): with S_c a state before a span, exp(log_scale) phi its transition product
 * (tr_gdn_transition) and S_hat its replay from zero (tr_gdn_replay), out is the state after
 * the span; with S_hat NULL, out is the carried start alone (the exact truncation error
 * E_m = S_a Phi).
 *
 * Arguments
 *   S_c       [device] [N, dv, dk] fp32
 *   phi       [device] [N, dk, dk] fp32
 *   log_scale [device] [N] fp32, or NULL for 0 (phi is then the whole product)
 *   S_hat     [device] [N, dv, dk] fp32, or NULL for zero
 *   out       [device] [N, dv, dk] fp32; may equal S_hat, must not overlap S_c or phi
 *   N         >= 1 matrices; dv, dk in {64, 128}
 *   stream    hipStream_t to enqueue on
 * fp32 arithmetic; a scale below the fp32 range makes the carried term zero.  Errors:
 * TR_ERR_INVALID_ARG (N < 1, null pointers, forbidden aliasing), TR_ERR_UNSUPPORTED (sizes),
 * TR_ERR_HIP.
 * ------------------------------------------------------------------------------- */
tr_status tr_state_compose(const float* S_c, const float* phi, const float* log_scale, const float* S_hat,
                           float* out, int32_t N, int32_t dv, int32_t dk, void* stream);

/* ---------------------------------------------------------------------------------
 * tr_gdn_decode -- one recurrence step per (sequence, value head) on resident states.
 *
 * For every b < B and value head h (query/key head h / (Hv / Hqk)), in place:
 *     S[b, h] <- alpha S[b, h] (I - beta k k^T) + beta v k^T,   alpha = exp(g[b, h]),
 *     o[b, h]  = S[b, h] (q_scale q)
 * Reading notes, section 2.3, Eq. (1) for one token; after a replay the suffix continues
 * from the rebuilt state (section 2.2, step 4), one token at a time when decoding.
 *
 * Arguments
 *   q, k    [device] [B, Hqk, dk] dtype dt
 *   v       [device] [B, Hv, dv]  dtype dt
 *   g, beta [device] [B, Hv] fp32
 *   B, Hqk, Hv, dk, dv   sizes; Hv % Hqk == 0; dk, dv in {64, 128}
 *   dt      TR_BF16 or TR_F32 (inputs and o; the state and the arithmetic are fp32)
 *   q_scale > 0
 *   state   [device] [B, Hv, dv, dk] fp32, read and overwritten
 *   o       [device] [B, Hv, dv] dtype dt, or NULL
 *   stream  hipStream_t to enqueue on
 * Errors: TR_ERR_INVALID_ARG, TR_ERR_UNSUPPORTED, TR_ERR_HIP.
 * ------------------------------------------------------------------------------- */
tr_status tr_gdn_decode(const void* q, const void* k, const void* v, const float* g, const float* beta,
                        int32_t B, int32_t Hqk, int32_t Hv, int32_t dk, int32_t dv, tr_dtype dt, float q_scale,
                        float* state, void* o, void* stream);

/* ---------------------------------------------------------------------------------
 * One LA layer's weights, all [device] bf16, row-major [out, in]:
 *   w_qk [2*Hqk*dk, d_model]   query heads first, then key heads
 *   w_v  [Hv*dv,    d_model]
 *   w_a  [Hv,       d_model]   gate logits:  g = log alpha = -softplus(y w_a^T)
 *   w_b  [Hv,       d_model]   write logits: beta = sigmoid(y w_b^T)
 *   w_o  [d_model,  Hv*dv]     output projection (unused for a group's last layer)
 *   rms_gain [d_model] or NULL (unit gain)
 * ------------------------------------------------------------------------------- */
typedef struct {
    const void* w_qk;
    const void* w_v;
    const void* w_a;
    const void* w_b;
    const void* w_o;
    const void* rms_gain;
} tr_la_weights;

/* ---------------------------------------------------------------------------------
 * tr_la_layer_inputs -- the projections in front of one LA layer's recurrence, for
 * G independent token blocks that each have their own weights.
 *
 * For each block g (n_tokens rows of x[g]):
 *   y    = bf16( x / sqrt(mean(x^2) + rms_eps) * gain )
 *   q_h  = bf16( (y Wq_h^T) / sqrt(|y Wq_h^T|^2 + 1e-6) * dk^-1/2 )   per q/k head h
 *   k_h  = bf16( (y Wk_h^T) / sqrt(|y Wk_h^T|^2 + 1e-6) )
 *   v    = bf16( y Wv^T ),  g = -softplus(y Wa^T),  beta = sigmoid(y Wb^T)   (fp32)
 * The pages only say k, v, alpha, beta are produced inside the group (reading notes,
 * section 2.1 symbol table); this is the plainest Gated DeltaNet layer front.
 *
 *   x        [device] [G, n_tokens, d_model] bf16
 *   w        [host]   array of G pointers-to-weights (w[g] is used for block g)
 *   q, k     [device] [G*n_tokens, Hqk, dk] bf16 (block g occupies rows g*n_tokens..)
 *   v        [device] [G*n_tokens, Hv, dv] bf16
 *   g_out, beta_out [device] [G*n_tokens, Hv] fp32
 *   workspace [device] >= tr_la_layer_inputs_workspace_size(...) bytes
 * Supported: dk = dv = 128, d_model % 64 == 0, Hv <= 64.
 * ------------------------------------------------------------------------------- */
size_t tr_la_layer_inputs_workspace_size(int32_t G, int32_t n_tokens, int32_t d_model);
tr_status tr_la_layer_inputs(const void* x, const tr_la_weights* const* w,
                             int32_t G, int32_t n_tokens, int32_t d_model,
                             int32_t Hqk, int32_t Hv, int32_t dk, int32_t dv, float rms_eps,
                             void* q, void* k, void* v, float* g_out, float* beta_out,
                             void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------
 * The two halves of tr_la_layer_inputs, each a single kernel:
 *
 * tr_rmsnorm: y = bf16( x / sqrt(mean(x^2) + rms_eps) * gain ) row by row for G blocks of
 *   n_tokens rows; gain[g] is block g's [d_model] bf16 gain or NULL (unit gain).
 *   x, y [device] [G, n_tokens, d_model] bf16 (may be the same buffer); gain [host] array
 *   of G device pointers.  Supported: d_model % 128 == 0.
 *
 * tr_la_project: q, k, v, g, beta from an already normalised y (the projection GEMM with
 *   the per-head L2 norm and gate epilogue of tr_la_layer_inputs).  Same arguments and
 *   layouts as tr_la_layer_inputs, without the workspace.
 * ------------------------------------------------------------------------------- */
tr_status tr_rmsnorm(const void* x, const void* const* gain, int32_t G, int32_t n_tokens, int32_t d_model,
                     float rms_eps, void* y, void* stream);
tr_status tr_la_project(const void* y, const tr_la_weights* const* w,
                        int32_t G, int32_t n_tokens, int32_t d_model,
                        int32_t Hqk, int32_t Hv, int32_t dk, int32_t dv,
                        void* q, void* k, void* v, float* g_out, float* beta_out, void* stream);

/* ---------------------------------------------------------------------------------
 * tr_la_output_residual -- x_out = bf16( x_in + o Wo^T ) for G blocks with their own
 * Wo (the LA layer's output projection and residual, in front of the next LA layer
 * of the group).
 *   x_in, x_out [device] [G, n_tokens, d_model] bf16 (may be the same buffer)
 *   o           [device] [G*n_tokens, Hv*dv] bf16
 *   w           [host]   array of G pointers-to-weights (w_o is used)
 * Supported: d_model % 128 == 0, (Hv*dv) % 64 == 0.
 * ------------------------------------------------------------------------------- */
tr_status tr_la_output_residual(const void* x_in, const void* o, const tr_la_weights* const* w,
                                int32_t G, int32_t n_tokens, int32_t d_model, int32_t Hv, int32_t dv,
                                void* x_out, void* stream);

/* ---------------------------------------------------------------------------------
 * tr_group_replay -- rebuild every LA state of G groups from their cached FA hiddens.
 *
 * Reading notes, section 2.2 steps 2-3 and section 2.4: for each group, the tail of
 * the cached FA output hidden vectors h_{m-k+1..m} runs through the group's L LA
 * layers in order, every layer starting from a zero state; groups are independent
 * (and run concurrently here).  Section 2.5: nothing after the last layer's
 * recurrence is needed (its FFN, and here also its output projection, per-token
 * outputs and residual, are skipped).  The layer body is tr_la_layer_inputs, then
 * tr_gdn_replay from zero with q_scale = 1, then (all but the last layer)
 * tr_la_output_residual.  No FFN is modelled between layers.
 *
 *   h_tail     [device] [G, n_tokens, d_model] bf16 (read-only)
 *   w          [host]   array [G*L] of weights, layer-major within a group:
 *                       w[g*L + l] is layer l of group g
 *   states_out [device] [G, L, Hv, dv, dk] fp32
 *   workspace  [device] >= tr_group_replay_workspace_size(...) bytes
 * Supported: dk = dv = 128, d_model % 128 == 0, Hv % Hqk == 0, Hv <= 64, L >= 1.
 * ------------------------------------------------------------------------------- */
size_t tr_group_replay_workspace_size(int32_t G, int32_t L, int32_t n_tokens, int32_t d_model,
                                      int32_t Hqk, int32_t Hv, int32_t dk, int32_t dv);
tr_status tr_group_replay(const void* h_tail, const tr_la_weights* w,
                          int32_t G, int32_t L, int32_t n_tokens, int32_t d_model,
                          int32_t Hqk, int32_t Hv, int32_t dk, int32_t dv, float rms_eps,
                          float* states_out, void* workspace, size_t workspace_bytes,
                          void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TAILREPLAY_H */
