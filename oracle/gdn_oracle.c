/*
 * gdn_oracle.c -- plain, slow, fp64 CPU oracle for Gated DeltaNet state replay,
 * the affine chunk operator and its composition.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header or constant with the
 * HIP library.
 *
 * Sources (cited by page title and passage):
 *  - "Tail-Replay: Escaping the Curse of Linear Attention in Prefix Caching
 *    for Hybrid LLMs", section 2 (Preliminary), Eq. (1): the per-token
 *    update of the recurrent state with the transition
 *    T_i = alpha_i (I - beta_i k_i k_i^T) and the write beta_i v_i k_i^T.
 *    Section 3 (Method), Eq. (2): tail replay from a zero state.
 *  - "LinearKV: One Cached State Suffices for Position-Independent Caching in
 *    Hybrid LLMs", the paragraph on the affine chunk operator: a chunk maps
 *    an incoming state through the product of its per-token transitions and
 *    adds the state it reaches from an empty start; chunks are applied back
 *    to back in context order.
 *
 * Orientation (a reading, the pages print the state update with the
 * transition on the left, which only type-checks when dk == dv): the state S
 * is dv x dk, row-major, and one token does
 *     S <- S * alpha (I - beta k k^T) + beta v k^T
 *  which, multiplied out, is
 *     y = S k;  S <- alpha S + beta (v - alpha y) k^T.
 * The output of a token is o = S q with the state after that token's update.
 * The chunk transition is the chronological product T_C = T_1 T_2 ... T_L so
 * that S_out = S_in T_C + S_local.
 *
 * Layouts (all row-major, contiguous, fp64):
 *   q, k  [n_tokens, H, dk]     v, o  [n_tokens, H, dv]
 *   alpha, beta [n_tokens, H]
 *   S0, S_final [n_seqs, H, dv, dk]
 *   T_C [n_chunks, H, dk, dk]   S_local [n_chunks, H, dv, dk]
 *   cu_seqlens / cu_chunks: int32 [n + 1], cu[0] = 0, nondecreasing.
 *
 * Work over (sequence, head) pairs is independent; it is spread over
 * n_threads OpenMP threads, nothing else is parallel or reordered.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* One token of the recurrence on one head: state S (dv x dk). */
static void token_update(double *S, int dk, int dv, const double *k,
                         const double *v, double alpha, double beta) {
  for (int i = 0; i < dv; ++i) {
    double *row = S + (size_t)i * dk;
    double y = 0.0;
    for (int j = 0; j < dk; ++j) y += row[j] * k[j];
    double delta = beta * (v[i] - alpha * y);
    for (int j = 0; j < dk; ++j) row[j] = alpha * row[j] + delta * k[j];
  }
}

/* o = S q for one head. */
static void state_times(const double *S, int dk, int dv, const double *q,
                        double *o) {
  for (int i = 0; i < dv; ++i) {
    const double *row = S + (size_t)i * dk;
    double acc = 0.0;
    for (int j = 0; j < dk; ++j) acc += row[j] * q[j];
    o[i] = acc;
  }
}

static int threads_or_default(int n_threads) {
  if (n_threads > 0) return n_threads;
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

int gdn_oracle_threads(void) { return threads_or_default(0); }

/*
 * Replay (Tail-Replay Eq. (1) applied over each packed sequence; Eq. (2) when
 * S0 is NULL, i.e. a zero starting state).
 *   q may be NULL when o is NULL.  S0 NULL means zero.  o NULL means
 *   state-only.  Returns 0, or -1 on a bad argument.
 */
int gdn_oracle_replay(const double *q, const double *k, const double *v,
                      const double *alpha, const double *beta,
                      const double *S0, const int32_t *cu_seqlens,
                      int n_seqs, int64_t n_tokens, int H, int dk, int dv,
                      double *o, double *S_final, int n_threads) {
  if (!k || !v || !alpha || !beta || !cu_seqlens || !S_final) return -1;
  if (o && !q) return -1;
  if (n_seqs < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
  if (cu_seqlens[0] != 0 || cu_seqlens[n_seqs] != n_tokens) return -1;
  for (int n = 0; n < n_seqs; ++n)
    if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
  const int64_t units = (int64_t)n_seqs * H;
  const size_t ss = (size_t)dv * dk;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(threads_or_default(n_threads)) reduction(| : bad)
  for (int64_t u = 0; u < units; ++u) {
    const int n = (int)(u / H), h = (int)(u % H);
    double *S = (double *)malloc(ss * sizeof(double));
    if (!S) { bad |= 1; continue; }
    if (S0)
      memcpy(S, S0 + (size_t)u * ss, ss * sizeof(double));
    else
      memset(S, 0, ss * sizeof(double));
    for (int64_t t = cu_seqlens[n]; t < cu_seqlens[n + 1]; ++t) {
      const size_t th = (size_t)t * H + h;
      token_update(S, dk, dv, k + th * dk, v + th * dv, alpha[th], beta[th]);
      if (o) state_times(S, dk, dv, q + th * dk, o + th * dv);
    }
    memcpy(S_final + (size_t)u * ss, S, ss * sizeof(double));
    free(S);
  }
  return bad ? -1 : 0;
}

/*
 * Chunk operator (LinearKV, the affine chunk operator paragraph).
 * For chunk c = tokens cu_chunks[c] .. cu_chunks[c+1]-1 and each head:
 *   T_C = product over the chunk, in token order, of alpha (I - beta k k^T),
 *         built as P <- I; per token: y = P k; P <- alpha (P - beta y k^T).
 *   S_local = the replay of the chunk from a zero state (needs v).
 * v and S_local may both be NULL (transition only).
 */
int gdn_oracle_chunk_operator(const double *k, const double *v,
                              const double *alpha, const double *beta,
                              const int32_t *cu_chunks, int n_chunks,
                              int64_t n_tokens, int H, int dk, int dv,
                              double *T_C, double *S_local, int n_threads) {
  if (!k || !alpha || !beta || !cu_chunks || !T_C) return -1;
  if ((v == NULL) != (S_local == NULL)) return -1;
  if (n_chunks < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
  if (cu_chunks[0] != 0 || cu_chunks[n_chunks] != n_tokens) return -1;
  for (int c = 0; c < n_chunks; ++c)
    if (cu_chunks[c + 1] < cu_chunks[c]) return -1;
  const int64_t units = (int64_t)n_chunks * H;
  const size_t tt = (size_t)dk * dk, ss = (size_t)dv * dk;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(threads_or_default(n_threads)) reduction(| : bad)
  for (int64_t u = 0; u < units; ++u) {
    const int c = (int)(u / H), h = (int)(u % H);
    double *P = T_C + (size_t)u * tt;
    double *y = (double *)malloc((size_t)dk * sizeof(double));
    if (!y) { bad |= 1; continue; }
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dk; ++j) P[(size_t)i * dk + j] = (i == j) ? 1.0 : 0.0;
    for (int64_t t = cu_chunks[c]; t < cu_chunks[c + 1]; ++t) {
      const size_t th = (size_t)t * H + h;
      const double *kt = k + th * dk;
      const double a = alpha[th], b = beta[th];
      for (int i = 0; i < dk; ++i) {
        double acc = 0.0;
        for (int j = 0; j < dk; ++j) acc += P[(size_t)i * dk + j] * kt[j];
        y[i] = acc;
      }
      for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dk; ++j)
          P[(size_t)i * dk + j] = a * (P[(size_t)i * dk + j] - b * y[i] * kt[j]);
    }
    free(y);
    if (S_local) {
      double *S = S_local + (size_t)u * ss;
      memset(S, 0, ss * sizeof(double));
      for (int64_t t = cu_chunks[c]; t < cu_chunks[c + 1]; ++t) {
        const size_t th = (size_t)t * H + h;
        token_update(S, dk, dv, k + th * dk, v + th * dv, alpha[th], beta[th]);
      }
    }
  }
  return bad ? -1 : 0;
}

/*
 * Composition (LinearKV, chunks applied back to back in context order):
 *   S <- S_in (or zero); for c = 0 .. n_chunks-1: S <- S T_C[c] + S_local[c].
 * S_out [H, dv, dk].  S_out may alias S_in.
 */
int gdn_oracle_compose(const double *S_in, const double *T_C,
                       const double *S_local, int n_chunks, int H, int dk,
                       int dv, double *S_out, int n_threads) {
  if (!T_C || !S_local || !S_out) return -1;
  if (n_chunks < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
  const size_t tt = (size_t)dk * dk, ss = (size_t)dv * dk;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(threads_or_default(n_threads)) reduction(| : bad)
  for (int h = 0; h < H; ++h) {
    double *S = (double *)malloc(ss * sizeof(double));
    double *N = (double *)malloc(ss * sizeof(double));
    if (!S || !N) { free(S); free(N); bad |= 1; continue; }
    if (S_in)
      memcpy(S, S_in + (size_t)h * ss, ss * sizeof(double));
    else
      memset(S, 0, ss * sizeof(double));
    for (int c = 0; c < n_chunks; ++c) {
      const double *T = T_C + ((size_t)c * H + h) * tt;
      const double *L = S_local + ((size_t)c * H + h) * ss;
      for (int i = 0; i < dv; ++i)
        for (int j = 0; j < dk; ++j) {
          double acc = L[(size_t)i * dk + j];
          for (int m = 0; m < dk; ++m) acc += S[(size_t)i * dk + m] * T[(size_t)m * dk + j];
          N[(size_t)i * dk + j] = acc;
        }
      double *tmp = S; S = N; N = tmp;
    }
    memcpy(S_out + (size_t)h * ss, S, ss * sizeof(double));
    free(S);
    free(N);
  }
  return bad ? -1 : 0;
}
