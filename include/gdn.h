/*
 * gdn.h -- C ABI of the MI355X (gfx950) Gated DeltaNet state-replay library.
 *
 * Three operations, each an asynchronous, stream-ordered sequence of HIP
 * kernel launches on the caller's stream.  No call allocates or frees device
 * memory, synchronises the device, or keeps a pointer after it returns; every
 * buffer belongs to the caller and must stay alive until the stream work is
 * done.  All argument checks happen on the host before any launch; on an
 * error nothing is launched and a status other than GDN_OK is returned (a
 * longer message is available from gdn_last_error(), per calling thread).
 * Device-side data are not validated: cu_seqlens / cu_chunks must be
 * nondecreasing with first entry 0 and last entry n_tokens, and every gate
 * alpha must lie in [0, 1].  The kernels take log(alpha) with a floor of -60:
 * a gate below e^-60 (about 8.8e-27), 0 included, acts as e^-60, i.e. it
 * scales the carried state by that factor instead of erasing it exactly.
 *
 * Pointer arguments are DEVICE pointers unless stated otherwise, 16-byte
 * aligned (GDN_ERR_ALIGNMENT otherwise), row-major and contiguous.
 * Shapes below use T = n_tokens, H = n_heads.
 *
 * The recurrence (page "Tail-Replay: Escaping the Curse of Linear Attention
 * in Prefix Caching for Hybrid LLMs", section 2, Eq. (1)), per head, with
 * the state S a dv x dk matrix:
 *     S_t = S_{t-1} alpha_t (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *     o_t = S_t q_t.
 * (The page writes the transition on the left of S; with S stored dv x dk it
 * acts from the right.  The transition is symmetric, so this only fixes the
 * storage orientation.)
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 1: gdn_replay, gdn_chunk_operator, gdn_compose and their helpers.
 * 2: adds gdn_decode, gdn_front_end, gdn_scalar_chunk_operator and
 *    gdn_scalar_compose; the version 1 calls are unchanged.
 * 3: adds gdn_replay_segmented and gdn_replay_noalloc; gates alpha = 0
 *    are accepted (see above); the earlier calls are unchanged.
 * 4: adds gdn_replay_raw; the earlier calls are unchanged. */
#define GDN_ABI_VERSION 4

typedef enum gdn_status {
  GDN_OK = 0,
  GDN_ERR_NULL_POINTER = 1, /* a required pointer is NULL                        */
  GDN_ERR_BAD_SHAPE = 2,    /* negative / inconsistent sizes                     */
  GDN_ERR_UNSUPPORTED = 3,  /* a size or dtype the library has no kernel for    */
  GDN_ERR_ALIGNMENT = 4,    /* a pointer is not 16-byte aligned                  */
  GDN_ERR_WORKSPACE = 5,    /* workspace missing or smaller than required        */
  GDN_ERR_HIP = 6           /* one of this call's own kernel launches failed
                               (errors left by earlier calls are not
                               reported); see gdn_last_error()            */
} gdn_status;

typedef enum gdn_dtype {
  GDN_F32 = 0,  /* IEEE binary32                                    */
  GDN_BF16 = 1  /* bfloat16 (upper half of a binary32)              */
} gdn_dtype;

/* A hipStream_t passed as an opaque pointer; NULL is the default stream. */
typedef void *gdn_stream_t;

/*
 * gdn_replay -- replay packed token sequences through the recurrence.
 * Page: Tail-Replay, section 2 Eq. (1) (the update) and section 3 Eq. (2)
 * (tail replay from a zero state: pass S0 = NULL).
 *
 *   q      [T, H, dk]  in_dtype   may be NULL when o is NULL
 *   k      [T, H, dk]  in_dtype   keys (used as given: no normalisation, no scale)
 *   v      [T, H, dv]  in_dtype
 *   alpha  [T, H]      in_dtype   gates in [0, 1]
 *   beta   [T, H]      in_dtype
 *   S0     [n_seqs, H, dv, dk] fp32 starting states, or NULL for zero
 *   cu_seqlens [n_seqs + 1] int32 (device): sequence n is tokens
 *          cu_seqlens[n] .. cu_seqlens[n+1]-1; sequences may be empty
 *   o      [T, H, dv]  o_dtype    o_t = S_t q_t with the state after token t,
 *          or NULL for a state-only replay
 *   S_final [n_seqs, H, dv, dk] fp32 (may alias S0: read fully before written)
 *   workspace / workspace_bytes: device scratch of at least
 *          gdn_replay_workspace_bytes(...) bytes (may be NULL if that is 0)
 *
 * Supported: dk, dv in {64, 128}; in_dtype F32 or BF16 (q, k, v, alpha,
 * beta all of it); o_dtype F32 or BF16; n_seqs >= 1; 1 <= n_heads <= 65536.
 * Deterministic: equal inputs give bitwise-equal outputs.
 */
gdn_status gdn_replay(const void *q, const void *k, const void *v,
                      const void *alpha, const void *beta, const float *S0,
                      const int32_t *cu_seqlens, int32_t n_seqs,
                      int64_t n_tokens, int32_t n_heads, int32_t dk,
                      int32_t dv, gdn_dtype in_dtype, void *o,
                      gdn_dtype o_dtype, float *S_final, void *workspace,
                      size_t workspace_bytes, gdn_stream_t stream);

/* Workspace bytes for gdn_replay with these sizes (enough for a state-only
 * call and a call with outputs, either dtype).  The split of long bf16
 * replays into time segments, and so the size, depends on the compute-unit
 * count of the current device (read once per device); call it with the
 * device of the replay's stream current. */
size_t gdn_replay_workspace_bytes(int32_t n_seqs, int64_t n_tokens,
                                  int32_t n_heads, int32_t dk, int32_t dv);

/*
 * gdn_replay_segmented -- gdn_replay with the number of time segments per
 * sequence given by the caller instead of the library's cost model (tuning
 * and tests).  A bf16 sequence cut into `segments` pieces of whole 64-token
 * chunks runs as that many independent recurrences: the first from S0, the
 * others as affine chunk operators (page "LinearKV: One Cached State
 * Suffices for Position-Independent Caching in Hybrid LLMs", affine-operator
 * and composition paragraphs) composed back to back; with outputs each
 * segment then runs again from its composed start state.  The result equals
 * gdn_replay's up to rounding.
 *
 *   segments: 0 = the cost model (exactly gdn_replay), 1 = no split,
 *             2 .. 64 = that many segments (segments past a sequence's end
 *             are empty).  fp32 inputs never split (the value is ignored).
 *   Other arguments as gdn_replay; the workspace must hold
 *   gdn_replay_segmented_workspace_bytes(..., segments) bytes.
 *   Errors: GDN_ERR_BAD_SHAPE for segments outside 0 .. 64, otherwise as
 *   gdn_replay.
 */
gdn_status gdn_replay_segmented(const void *q, const void *k, const void *v,
                                const void *alpha, const void *beta,
                                const float *S0, const int32_t *cu_seqlens,
                                int32_t n_seqs, int64_t n_tokens,
                                int32_t n_heads, int32_t dk, int32_t dv,
                                gdn_dtype in_dtype, void *o, gdn_dtype o_dtype,
                                float *S_final, int32_t segments,
                                void *workspace, size_t workspace_bytes,
                                gdn_stream_t stream);

size_t gdn_replay_segmented_workspace_bytes(int32_t n_seqs, int64_t n_tokens,
                                            int32_t n_heads, int32_t dk,
                                            int32_t dv, int32_t segments);

/*
 * gdn_replay_raw -- gdn_front_end followed by gdn_replay in one call, from
 * the raw projections: the front end runs inside the replay's own kernels,
 * so the normalised queries and keys and the activated gates are never
 * written to memory or rounded to bf16.
 * Page: Tail-Replay, section 3 (the replayed hidden states produce the keys,
 * values, transitions and write strengths at each replay step) with
 * section 2 Eq. (1).  Per (token, head), in fp32:
 *     q = q_raw / |q_raw|,  k = k_raw / |k_raw|   (a zero row gives zeros)
 *     alpha = exp(g),       beta = 1 / (1 + exp(-b))
 * then the recurrence of gdn_replay with those inputs.  The log-gate has the
 * floor of gdn_replay (log alpha >= -60), taken on g directly.
 *
 *   q_raw, k_raw  [n_tokens, H, dk]  bf16 (q_raw only read when o is given)
 *   v             [n_tokens, H, dv]  bf16
 *   g, b          [n_tokens, H]      bf16 log-gates and write-strength logits
 *   S0, cu_seqlens, o, o_dtype, S_final: as gdn_replay.
 *   in_dtype must be GDN_BF16 (GDN_ERR_UNSUPPORTED otherwise).
 *   workspace: gdn_replay_raw_workspace_bytes(...) bytes (the replay's
 *   workspace and 256 bytes of reciprocal key norms per chunk slot and
 *   head; the query norms are formed where the outputs are).
 * Errors and everything else as gdn_replay.  The result equals
 * gdn_front_end + gdn_replay up to the rounding of the normalised inputs to
 * bf16, which this call skips.
 */
gdn_status gdn_replay_raw(const void *q_raw, const void *k_raw, const void *v,
                          const void *g, const void *b, const float *S0,
                          const int32_t *cu_seqlens, int32_t n_seqs,
                          int64_t n_tokens, int32_t n_heads, int32_t dk,
                          int32_t dv, gdn_dtype in_dtype, void *o,
                          gdn_dtype o_dtype, float *S_final, void *workspace,
                          size_t workspace_bytes, gdn_stream_t stream);

/* Workspace bytes for gdn_replay_raw (as gdn_replay_workspace_bytes, with
 * the norms). */
size_t gdn_replay_raw_workspace_bytes(int32_t n_seqs, int64_t n_tokens,
                                      int32_t n_heads, int32_t dk, int32_t dv);

/*
 * gdn_replay_noalloc -- gdn_replay for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same kernels, with their scratch (per-chunk records,
 * time-split segment operators and states, the longest-first sequence
 * order) in a built-in device array of GDN_NOALLOC_SCRATCH_BYTES instead of
 * a caller's workspace.  The call allocates nothing: no hipMalloc, no
 * hipFree, no allocating library routine.
 *
 *   Arguments as gdn_replay, without the workspace.
 *   Each GPU the library runs on holds its own copy of the array (64 MiB)
 *   from the library's load until the process ends; its device address is
 *   looked up on the first call on each device (with that device current).
 *   The array keeps the last call's contents; nothing in it needs to start
 *   at zero.  Calls that overlap on one GPU (on different streams, or from
 *   different threads without ordering) share the array and RACE: order
 *   them on one stream.
 *   Errors: GDN_ERR_WORKSPACE when the replay needs more scratch than the
 *   array holds (e.g. more than ~4,700 (chunk, head) records); GDN_ERR_HIP
 *   when the array's device address cannot be read; otherwise as gdn_replay.
 */
#define GDN_NOALLOC_SCRATCH_BYTES (64u << 20)

gdn_status gdn_replay_noalloc(const void *q, const void *k, const void *v,
                              const void *alpha, const void *beta,
                              const float *S0, const int32_t *cu_seqlens,
                              int32_t n_seqs, int64_t n_tokens,
                              int32_t n_heads, int32_t dk, int32_t dv,
                              gdn_dtype in_dtype, void *o, gdn_dtype o_dtype,
                              float *S_final, gdn_stream_t stream);

/*
 * gdn_chunk_operator -- the affine operator of each chunk.
 * Page: "LinearKV: One Cached State Suffices for Position-Independent
 * Caching in Hybrid LLMs", the paragraph on the affine chunk operator: a
 * chunk maps an incoming state S_in to S_in T_C + S_local, where T_C is the
 * product of the chunk's per-token transitions in token order and S_local
 * the state the chunk reaches from a zero start.
 *
 *   k      [T, H, dk], alpha, beta [T, H], v [T, H, dv]  in_dtype
 *   cu_chunks [n_chunks + 1] int32 (device): chunk c is tokens
 *          cu_chunks[c] .. cu_chunks[c+1]-1 (an empty chunk gives T_C = I)
 *   T_C     [n_chunks, H, dk, dk] fp32 out
 *   S_local [n_chunks, H, dv, dk] fp32 out
 *   v and S_local may both be NULL: only T_C is built (T_C needs only the
 *   key / gate stream).
 * Supported: dk, dv in {64, 128}; in_dtype F32 or BF16; 1 <= n_heads <= 65536.
 */
gdn_status gdn_chunk_operator(const void *k, const void *v, const void *alpha,
                              const void *beta, const int32_t *cu_chunks,
                              int32_t n_chunks, int64_t n_tokens,
                              int32_t n_heads, int32_t dk, int32_t dv,
                              gdn_dtype in_dtype, float *T_C, float *S_local,
                              void *workspace, size_t workspace_bytes,
                              gdn_stream_t stream);

size_t gdn_chunk_operator_workspace_bytes(int32_t n_chunks, int64_t n_tokens,
                                          int32_t n_heads, int32_t dk,
                                          int32_t dv);

/*
 * gdn_compose -- apply chunk operators back to back in context order.
 * Page: LinearKV, the composition paragraph (chunk c's output is chunk
 * c+1's input; the closed form adds no approximation of its own):
 *     S <- S_in (or zero);  for c = 0 .. n_chunks-1:  S <- S T_C[c] + S_local[c]
 *
 *   S_in    [H, dv, dk] fp32 or NULL (zero)
 *   T_C     [n_chunks, H, dk, dk] fp32,  S_local [n_chunks, H, dv, dk] fp32
 *   S_out   [H, dv, dk] fp32 (may alias S_in)
 *   workspace: gdn_compose_workspace_bytes(...) bytes (n_chunks * H * dk * dk
 *          * 4: the operators converted to the products' split-bf16 form),
 *          16-byte aligned; may be NULL when that is 0
 * n_chunks may be 0 (S_out = S_in, or zero).
 */
gdn_status gdn_compose(const float *S_in, const float *T_C,
                       const float *S_local, int32_t n_chunks, int32_t n_heads,
                       int32_t dk, int32_t dv, float *S_out, void *workspace,
                       size_t workspace_bytes, gdn_stream_t stream);

size_t gdn_compose_workspace_bytes(int32_t n_chunks, int32_t n_heads,
                                   int32_t dk, int32_t dv);

/* Human-readable name of a status code (static storage). */
const char *gdn_status_string(gdn_status status);

/* Detail of the last error on the calling thread ("" if none). */
const char *gdn_last_error(void);

/*
 * gdn_decode -- one token per sequence from a given state: the step after a
 * replay, when serving continues token by token.
 * Page: Tail-Replay, section 2 Eq. (1) (per-token update) and section 3
 * (serving continues from the reconstructed states).  Per (sequence, head):
 *     y = S k;  S <- alpha S + beta (v - alpha y) k^T;  o = S q
 * (o with the updated state), in fp32.
 *
 *   q, k   [n_seqs, H, dk], v [n_seqs, H, dv], alpha, beta [n_seqs, H]  in_dtype
 *          (q may be NULL when o is NULL)
 *   S_in   [n_seqs, H, dv, dk] fp32, or NULL (zero state)
 *   o      [n_seqs, H, dv] o_dtype, or NULL (state only)
 *   S_out  [n_seqs, H, dv, dk] fp32 (may alias S_in: updated in place)
 * Supported: dk, dv in {64, 128}; dtypes F32 or BF16; 1 <= n_heads <= 65536.
 * No workspace; stream-ordered, no synchronisation.
 */
gdn_status gdn_decode(const void *q, const void *k, const void *v,
                      const void *alpha, const void *beta, const float *S_in,
                      int32_t n_seqs, int32_t n_heads, int32_t dk, int32_t dv,
                      gdn_dtype in_dtype, void *o, gdn_dtype o_dtype,
                      float *S_out, gdn_stream_t stream);

/*
 * gdn_scalar_chunk_operator -- the affine chunk operator when the per-token
 * transition is a scalar decay (the Mamba-2 family): T_t = alpha_t I, so
 * the chunk's transition is the scalar gamma = prod_t alpha_t.
 * Page: LinearKV, the affine-operator paragraph (the two families differ
 * only in what the chunk's transition is), with the write term of
 * Tail-Replay section 2 Eq. (1):  S_t = alpha_t S_{t-1} + beta_t v_t k_t^T.
 * From a zero start over chunk c:
 *     gamma[c]   = prod_t alpha_t
 *     S_local[c] = sum_t beta_t (prod_{s > t} alpha_s) v_t k_t^T
 *
 *   k [T, H, dk], v [T, H, dv], alpha, beta [T, H]   in_dtype (alpha in [0, 1])
 *   cu_chunks [n_chunks + 1] int32 (device), as for gdn_chunk_operator
 *          (an empty chunk gives gamma = 1, S_local = 0)
 *   gamma   [n_chunks, H] fp32 out
 *   S_local [n_chunks, H, dv, dk] fp32 out, or NULL (then v may be NULL)
 * Supported: dk, dv in {64, 128}; in_dtype F32 or BF16; 1 <= n_heads <= 65536;
 * n_tokens < 2^31.  No workspace; stream-ordered, no synchronisation.
 */
gdn_status gdn_scalar_chunk_operator(const void *k, const void *v,
                                     const void *alpha, const void *beta,
                                     const int32_t *cu_chunks, int32_t n_chunks,
                                     int64_t n_tokens, int32_t n_heads,
                                     int32_t dk, int32_t dv, gdn_dtype in_dtype,
                                     float *gamma, float *S_local,
                                     gdn_stream_t stream);

/*
 * gdn_scalar_compose -- scalar-decay chunk operators back to back in context
 * order (LinearKV, the composition paragraph, with a scalar transition):
 *     S <- S_in (or zero);  for c = 0 .. n_chunks-1:  S <- gamma[c] S + S_local[c]
 *
 *   S_in  [H, dv, dk] fp32 or NULL (zero);  gamma [n_chunks, H] fp32;
 *   S_local [n_chunks, H, dv, dk] fp32;  S_out [H, dv, dk] fp32 (may alias S_in)
 * n_chunks may be 0 (S_out = S_in, or zero).  No workspace.
 * The LinearKV last-block initializer, S_init = S_local of the last matched
 * chunk, needs no call: it is S_local[n_chunks - 1] of either operator.
 */
gdn_status gdn_scalar_compose(const float *S_in, const float *gamma,
                              const float *S_local, int32_t n_chunks,
                              int32_t n_heads, int32_t dk, int32_t dv,
                              float *S_out, gdn_stream_t stream);

/*
 * gdn_front_end -- the step before the recurrence: queries and keys
 * L2-normalised per (token, head), the decay from its log-gate and the write
 * strength from its logit.
 * Page: Tail-Replay, section 3 (the replayed hidden states produce the keys,
 * values, transitions and write strengths) and section 2 Eq. (1) (alpha in
 * (0, 1]; an underflow to 0 is accepted by the calls above).  Per (token, head), in fp32, each result rounded once to dtype:
 *     q = q_raw / |q_raw|,  k = k_raw / |k_raw|   (a zero row gives zeros)
 *     alpha = exp(g),       beta = 1 / (1 + exp(-b))
 * The outputs are the q, k, alpha and beta that gdn_replay, gdn_chunk_operator
 * and gdn_decode take (values v pass through unchanged and are not touched).
 *
 *   q_raw, k_raw  [n_tokens, H, dk]  dtype   (q_raw may be NULL, then q is too)
 *   g, b          [n_tokens, H]      dtype   log-gate (g <= 0 keeps alpha in
 *                                            [0, 1]: exp(g) rounds to 0 below
 *                                            about -104 in fp32 and -92 in
 *                                            bf16, which the replay accepts;
 *                                            larger g is not rejected) and
 *                                            beta logit
 *   q, k          [n_tokens, H, dk]  dtype   outputs (may alias q_raw, k_raw)
 *   alpha, beta   [n_tokens, H]      dtype   outputs (may alias g, b)
 * Supported: dk in {64, 128}; dtypes F32 or BF16; 1 <= n_heads <= 65536;
 * n_tokens <= 2^40.  No workspace; stream-ordered, no synchronisation.
 */
gdn_status gdn_front_end(const void *q_raw, const void *k_raw, const void *g,
                         const void *b, int64_t n_tokens, int32_t n_heads,
                         int32_t dk, gdn_dtype dtype, void *q, void *k,
                         void *alpha, void *beta, gdn_stream_t stream);

/* GDN_ABI_VERSION of the loaded library. */
int gdn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
