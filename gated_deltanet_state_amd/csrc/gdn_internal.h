// gdn_internal.h -- host-side launch descriptors shared by the C ABI and the
// kernel translation units (not part of the public interface).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <tuple>
#include <utility>

namespace gdn {

// Launch `kernel` on `stream` and return the status of this launch alone.
// (A triple-chevron launch reports its error only through hipGetLastError,
// which also returns errors left by earlier, unrelated calls of the thread.)
template <typename... KArgs, size_t... I>
inline hipError_t launch_tuple(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t shmem, hipStream_t stream,
                               std::tuple<KArgs...> &args, std::index_sequence<I...>) {
  void *ptrs[] = {static_cast<void *>(&std::get<I>(args))...};
  return hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, ptrs, shmem, stream);
}
template <typename... KArgs, typename... Args>
inline hipError_t launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t shmem, hipStream_t stream,
                                Args &&...args) {
  static_assert(sizeof...(KArgs) > 0 && sizeof...(KArgs) == sizeof...(Args), "kernel arguments");
  std::tuple<KArgs...> a(std::forward<Args>(args)...);
  return launch_tuple(kernel, grid, block, shmem, stream, a, std::index_sequence_for<KArgs...>{});
}

// ---------------------------------------------------------------------------
// Chunk slots.  Sequence n (tokens cu[n] .. cu[n+1]-1) is cut into 64-token
// chunks; its chunk j lives in slot floor(cu[n] / 64) + n + j.  Slots of
// different sequences never collide and all lie below
// n_tokens / 64 + n_seqs + 1, so the host can size per-chunk storage
// without reading cu (which lives on the device).
// ---------------------------------------------------------------------------
constexpr int kChunk = 64;
// Per-chunk factor record, one per (slot, head), 12 KiB:
//   * fp32 inputs: Tau = (I + A)^{-1}, lower 16 x 16 block rows packed, block
//     row b holds 16 rows x 16 (b + 1) columns, row-major, at element offset
//     256 * b (b + 1) / 2 (2560 floats);
//   * bf16 inputs: Tau diag(beta) as the six A operands of the k = 32 MFMAs
//     that apply it to a 64 x 16 right-hand side given as C-layout tiles (see
//     kTauFrags), split bf16 planes [hi/lo][fragment][lane][8].
// (The recurrence forms the chunk's gates itself from alpha.)
constexpr int kRecFloats = 3072;
// Fragment f of Tau covers token block row bt and the pair of 16-column
// blocks (2m, 2m + 1): f = 0: (0,0), 1: (1,0), 2: (2,0), 3: (2,1), 4: (3,0),
// 5: (3,1).  Lane l holds row 16 bt + (l & 15), columns
// 32 m + 4 (l >> 4) + {0..3} then 32 m + 16 + 4 (l >> 4) + {0..3}.
constexpr int kTauFrags = 6;

// Raw inputs (gdn_replay_raw: the front end folded into the replay).  The
// gate arrays hold the log-gates g (alpha = e^g) and the write-strength
// logits (beta = 1 / (1 + e^-b)), and the keys and queries are raw
// projections.  The record builder stores, per (chunk slot, head), the
// reciprocal norms 1 / |k_t| of the chunk's keys (0 for a zero row); every
// product with a key row carries that factor.  The query norms are formed by
// the output recurrence from the queries it stages (outputs are linear in
// their token's query, so each output row is scaled when it is stored).
constexpr int kNormFloats = kChunk;

constexpr int kTauFragPlane = kTauFrags * 64 * 8;  // bf16 elements per plane

inline int64_t slot_count(int64_t n_tokens, int32_t n_seqs) { return n_tokens / kChunk + n_seqs + 1; }

inline size_t tau_workspace_bytes(int64_t n_tokens, int32_t n_seqs, int32_t n_heads) {
  return (size_t)slot_count(n_tokens, n_seqs) * (size_t)n_heads * kRecFloats * sizeof(float);
}
inline size_t norm_workspace_bytes(int64_t n_tokens, int32_t n_seqs, int32_t n_heads) {
  return (size_t)slot_count(n_tokens, n_seqs) * (size_t)n_heads * kNormFloats * sizeof(float);
}

// Longest-first order of the sequences of a packed replay that runs without
// a time split: order[r] is the sequence with the r-th most chunks (ties by
// index).  The recurrence then starts the longest (sequence, head) items
// first, which shortens the tail of the launch when the items outnumber the
// compute units.  Built by the bf16 prep kernel for 2 .. kMaxOrderedSeqs
// sequences (a quadratic rank count by one wave); above that, sequence order.
constexpr int32_t kMaxOrderedSeqs = 256;
inline size_t order_workspace_bytes(int32_t n_seqs) {
  return (n_seqs > 1 && n_seqs <= kMaxOrderedSeqs) ? ((size_t)n_seqs * 4 + 255) / 256 * 256 : 0;
}

// Per-chunk factor build: one workgroup per (slot, head).
struct PrepLaunch {
  const void *k, *alpha, *beta;
  const int32_t *cu;
  int32_t n_seqs, H, dk;
  int in_bf16;
  float *tau;        // [n_slots, H, kRecFloats] per-chunk factor records
  int64_t n_slots;
  int32_t *order;    // [n_seqs] longest-first sequence order to build, or null (bf16 only)
  // raw inputs (bf16 only, see kNormFloats): k raw keys, alpha log-gates,
  // beta logits
  int raw;
  float *norms;      // [n_slots, H, kNormFloats]
};

// One launch of the chunked recurrence kernel.  A work item is one tile of
// 16 rows of the state of one (sequence, head).  Row tiles come in two kinds:
//   * tiles_T "transition" tiles (chunk-operator mode): rows of a dk x dk
//     matrix that starts as the identity and receives no value input; after
//     the sequence they hold rows of the transition product T_C.
//   * tiles_S "state" tiles: rows of the dv x dk state, starting from S0 (or
//     zero) and receiving the value input; they end as S_final / S_local.
struct ChainLaunch {
  const void *q, *k, *v, *alpha, *beta;
  const float *S0;          // [n_seqs, H, dv, dk] or null
  const int32_t *cu;        // [n_seqs + 1] (device)
  const float *tau;         // per-chunk factors from the prep kernel
  int32_t n_seqs;
  int32_t H;
  int32_t dk, dv;
  int in_bf16;              // inputs are bf16 (else fp32)
  void *o;                  // [T, H, dv] or null
  int o_bf16;
  float *S_out;             // [n_seqs, n_segs, H, dv, dk] (state tiles) or null
  float *T_out;             // [n_seqs, n_segs, H, dk, dk] (transition tiles) or null
  int32_t tiles_T, tiles_S;
  // Time split: each sequence is cut into n_segs segments of whole chunks;
  // every segment runs independently (state tiles of segment 0 from S0, of
  // later segments from S0_seg or zero; transition tiles from the identity).
  int32_t n_segs;           // >= 1
  const float *S0_seg;      // [n_seqs, n_segs, H, dv, dk]: start of every segment (replaces S0), or null
  int skip_T0;              // segment 0 has no transition tiles
  // Time split with outputs ("lead" layout, n_segs >= 2): segments 1 ..
  // n_segs - 1 all have one length and segment 0 (the lead) takes the rest.
  // The segment launch (transition tiles) runs segments 0 .. n_segs - 2:
  // the lead from S0 with its outputs, into o, and the others with
  // transition rows, which also build the records of the last segment (the
  // lead does when there are no others); the output launch (no transition
  // tiles) runs segments 1 .. n_segs - 1 from S0_seg and writes the last
  // segment's end state to S_last.
  int lead;
  float *S_last;            // [n_seqs, H, dv, dk] or null
  // write each segment's T as composition fragments (kSegOpFragments)
  // instead of row-major fp32
  int T_frags;
  // bf16 inputs with transition tiles: every workgroup first builds the
  // per-chunk records of its own segment (no separate prep launch)
  int fuse_prep;
  // [n_seqs] longest-first sequence order (PrepLaunch::order), or null;
  // used by the bf16 recurrence when each (sequence, head) is one workgroup
  const int32_t *order;
  // bf16 chunk operators (fuse_prep, one workgroup per (sequence, head), no
  // time split): > 0 runs that many workgroups, each over a contiguous run
  // of the (sequence, head) items as one stream of chunks; 0: one
  // workgroup per item
  int multi_wgs;
  // raw inputs (kNormFloats): alpha holds log-gates, beta logits, k and q
  // raw projections; norms [n_slots, H, kNormFloats] come from the record
  // builder (written by the fused prologue, read by the recurrence)
  int raw;
  float *norms;
};


// Segment operator fragments (time-split replay): per (sequence, segment,
// head), dk * dk * 4 bytes holding T as split-bf16 MFMA operands of the
// composition S_new^T = T^T S^T + S_seg^T: fragment f = jb * (dk / 32) + ks
// (jb < dk / 16, ks < dk / 32), lane (q, g) = (l & 15, l >> 4) holds
// T[32 ks + 8 g + i][16 jb + q], i < 8; hi plane [f][lane][8] bf16, then
// the lo plane.
//
// Composition of time-split segments: for each (sequence, head),
//   S = S_seg[0];  S <- S T_seg[s] + S_seg[s] for s = 1 .. n_segs - 1.
struct SegComposeLaunch {
  const float *S_seg;       // [n_seqs, n_segs, H, dv, dk]
  const void *T_frag;       // [n_seqs, n_segs, H] operators as fragments (segment 0 unused)
  float *S_prefix;          // [n_seqs, n_segs, H, dv, dk]: state entering each segment, or null
  const float *S0;          // [n_seqs, H, dv, dk] start of segment 0 (copied to S_prefix), or null = zero
  int32_t n_seqs, n_segs, H, dk, dv;
  float *S_out;             // [n_seqs, H, dv, dk]
  // start from S0 and apply every operator, segment 0's included (else
  // S_seg[0] is the state after segment 0 and T_frag[0] is unused)
  int from_start;
  // lead layout of a time split with outputs (ChainLaunch::lead): the last
  // segment has no operator; the state entering it goes to S_prefix and
  // S_out is unused
  int lead;
};

// One token per sequence from a given state (gdn_decode).
struct DecodeLaunch {
  const void *q, *k, *v, *alpha, *beta;   // q, k [n_seqs, H, dk]; v [n_seqs, H, dv]; alpha, beta [n_seqs, H]
  const float *S_in;                      // [n_seqs, H, dv, dk] or null (zero)
  float *S_out;                           // [n_seqs, H, dv, dk] (may be S_in)
  void *o;                                // [n_seqs, H, dv] or null
  int32_t n_seqs, H, dk, dv;
  int in_bf16, o_bf16;
};

// Normalised queries and keys and activated gates (gdn_front_end).
struct FrontLaunch {
  const void *q_in, *k_in, *g, *b;   // q_in, k_in [n_tokens, H, dk] (q_in may be null); g, b [n_tokens, H]
  void *q_out, *k_out, *alpha, *beta; // same shapes (may alias the inputs)
  int64_t n_tokens;
  int32_t H, dk;
  int in_bf16;
};

// Scalar-decay chunk operators (gdn_scalar_chunk_operator) and their composition.
struct ScalarOpLaunch {
  const void *k, *v, *alpha, *beta;   // k [T, H, dk], v [T, H, dv], alpha, beta [T, H]
  const int32_t *cu;                  // chunk bounds [n_chunks + 1]
  float *gamma;                       // [n_chunks, H]
  float *S_local;                     // [n_chunks, H, dv, dk] or null
  int32_t n_chunks, H, dk, dv;
  int in_bf16;
  int64_t n_tokens;                   // rows of k, v, alpha, beta
};
struct ScalarComposeLaunch {
  const float *S_in;                  // [H, dv, dk] or null (zero)
  const float *gamma, *S_local;       // [n_chunks, H], [n_chunks, H, dv, dk]
  float *S_out;                       // [H, dv, dk] (may be S_in)
  int32_t n_chunks, H, dk, dv;
};
hipError_t launch_scalar_op(const ScalarOpLaunch &p, hipStream_t stream);
hipError_t launch_scalar_compose(const ScalarComposeLaunch &p, hipStream_t stream);

hipError_t launch_decode(const DecodeLaunch &p, hipStream_t stream);
hipError_t launch_front(const FrontLaunch &p, hipStream_t stream);
hipError_t launch_prep(const PrepLaunch &p, hipStream_t stream);        // dispatches bf16 inputs to launch_prep_bf16
hipError_t launch_prep_bf16(const PrepLaunch &p, hipStream_t stream);
hipError_t launch_chain(const ChainLaunch &p, hipStream_t stream);        // fp32 inputs
hipError_t launch_chain_bf16(const ChainLaunch &p, hipStream_t stream);   // bf16 inputs
// fp32 operators [n_ops, dk, dk] into composition fragments (n_ops * dk * dk * 4 bytes)
hipError_t launch_op_frags(const float *T, int64_t n_ops, int32_t dk, void *frag, hipStream_t stream);
hipError_t launch_seg_compose(const SegComposeLaunch &p, hipStream_t stream);

}  // namespace gdn
