// gdn_api.cpp -- the C ABI declared in include/gdn.h: argument checks,
// workspace sizing and kernel launches on the caller's stream.
#include "gdn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdlib>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "gdn_internal.h"

namespace {

thread_local std::string g_last_error;

gdn_status fail(gdn_status s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
gdn_status fail(gdn_status s, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

gdn_status ok() {
  g_last_error.clear();
  return GDN_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool supported_dim(int32_t d) { return d == 64 || d == 128; }

bool valid_dtype(gdn_dtype t) { return t == GDN_F32 || t == GDN_BF16; }

// Largest token count whose (token, head) indexing stays within the 32-bit
// arithmetic of the chunk loop.
constexpr int64_t kMaxTokens = (int64_t(1) << 31) - 64;
// Largest head count whose in-chunk byte offsets (64 tokens x heads x 128
// bf16) fit the kernels' 32-bit offsets.
constexpr int32_t kMaxHeads = 65536;

gdn_status check_align(const char *name, const void *p) {
  if (p && !aligned16(p)) return fail(GDN_ERR_ALIGNMENT, "%s is not 16-byte aligned", name);
  return GDN_OK;
}

gdn_status launched(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(GDN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// Compute units of the current device, read once per device
// (hipDeviceAttributeMultiprocessorCount); 256 when no device answers.
constexpr int kMaxDevices = 64;
std::once_flag g_cu_once[kMaxDevices];
int g_cus[kMaxDevices];

int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  std::call_once(g_cu_once[dev], [dev] {
    int n = 0;
    g_cus[dev] = (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0) ? n
                                                                                                             : 256;
  });
  return g_cus[dev];
}

// Largest segment count a caller may force.
constexpr int32_t kMaxSegments = 64;

// Segments per sequence for a state-only replay with bf16 inputs.  A
// sequence cut into P segments of whole chunks runs as P independent
// recurrences (segment 0 from S0 with its state rows only, later segments as
// affine operators with dk transition rows as well), composed afterwards.
// Cost model, in units of one chunk step of an eight-wave state workgroup
// (one workgroup per compute unit):
//   P = 1:  (workgroups / CUs rounded up) x chunks per sequence
//   P > 1:  one workgroup of transition + state tiles per (sequence, head,
//           segment), each chunk step about 1.25 units, plus about 0.3 units
//           per composition step.
// P = 1 unless splitting pays.
int replay_segments(int32_t n_seqs, int64_t n_tokens, int32_t n_heads, int32_t dk, int32_t dv, int cus) {
  if ((dk + dv) / 16 > 16) return 1;
  const double chunks = std::ceil((double)n_tokens / gdn::kChunk / (n_seqs > 0 ? n_seqs : 1));
  int pmax = (int)chunks;
  if (pmax > 16) pmax = 16;
  if (pmax < 1) pmax = 1;
  const int64_t wg1 = (int64_t)n_seqs * n_heads * ((dv / 16 + 7) / 8);
  int best = 1;
  double best_t = (double)((wg1 + cus - 1) / cus) * chunks;
  for (int P = 2; P <= pmax; ++P) {
    const int64_t wg = (int64_t)n_seqs * n_heads * P;
    if (wg > (int64_t(1) << 28)) break;
    const double t = (double)((wg + cus - 1) / cus) * std::ceil(chunks / P) * 1.25 + 0.3 * (P - 1);
    if (t < best_t) {
      best = P;
      best_t = t;
    }
  }
  return best;
}

// Segments per sequence for a bf16 replay with outputs.  A split runs three
// passes: the segment launch (the lead segment 0 with its outputs from S0,
// beside the transition and state rows of the middle segments), the
// composition (every later segment's true start state), and the output
// launch (segments 1 .. P - 1 with outputs from those states).  Worth it
// when the (sequence, head) pairs alone leave compute units idle: the P - 1
// later segments fill the compute units with one workgroup per (sequence,
// head, segment), with at least 8 chunks per segment.
int replay_segments_o(int32_t n_seqs, int64_t n_tokens, int32_t n_heads, int32_t dk, int32_t dv, int cus) {
  if ((dk + dv) / 16 > 16) return 1;
  const int64_t chunks = (n_tokens / gdn::kChunk) / (n_seqs > 0 ? n_seqs : 1);
  const int64_t units = (int64_t)n_seqs * n_heads;
  int64_t Q = cus / (units > 0 ? units : 1);
  if (Q > chunks / 8) Q = chunks / 8;
  if (Q > 8) Q = 8;
  return Q < 2 ? 1 : (int)Q + 1;
}

// Segment count of one call: `forced` (>= 1, from gdn_replay_segmented) or
// the cost model; fp32 inputs never split.
int32_t segments_for(bool bf, bool with_o, int32_t forced, int32_t n_seqs, int64_t n_tokens, int32_t n_heads,
                     int32_t dk, int32_t dv) {
  if (!bf) return 1;
  if (forced >= 1) return forced < kMaxSegments ? forced : kMaxSegments;
  const int cus = device_cus();
  return with_o ? replay_segments_o(n_seqs, n_tokens, n_heads, dk, dv, cus)
                : replay_segments(n_seqs, n_tokens, n_heads, dk, dv, cus);
}

// Segment operators and states: [n_seqs, P, H] x (dk x dk + dv x dk) fp32;
// with outputs also the start states [n_seqs, P, H, dv, dk].
size_t seg_workspace_bytes(int32_t n_seqs, int32_t P, int32_t n_heads, int32_t dk, int32_t dv, bool prefix = false) {
  if (P <= 1) return 0;
  return (size_t)n_seqs * P * n_heads * ((size_t)dk * dk + (size_t)dv * dk * (prefix ? 2 : 1)) * sizeof(float);
}

// Workspace of one replay call (the records, then the segment operators and
// states of a time split, or the longest-first order of an unsplit bf16 call).
size_t replay_need(bool bf, bool with_o, int32_t P, int32_t n_seqs, int64_t n_tokens, int32_t n_heads, int32_t dk,
                   int32_t dv) {
  const bool ordered = bf && P == 1 && gdn::order_workspace_bytes(n_seqs) > 0;
  return gdn::tau_workspace_bytes(n_tokens, n_seqs, n_heads) +
         (P > 1 ? seg_workspace_bytes(n_seqs, P, n_heads, dk, dv, with_o)
                : (ordered ? gdn::order_workspace_bytes(n_seqs) : 0));
}

// Enough for any call with these sizes (state only or with outputs, bf16 or
// fp32 inputs).
size_t replay_workspace_max(int32_t n_seqs, int64_t n_tokens, int32_t n_heads, int32_t dk, int32_t dv,
                            int32_t forced) {
  if (n_seqs < 1 || n_tokens < 0 || n_heads < 1) return 0;
  if (!supported_dim(dk) || !supported_dim(dv)) return gdn::tau_workspace_bytes(n_tokens, n_seqs, n_heads);
  size_t best = 0;
  for (int with_o = 0; with_o < 2; ++with_o) {
    const int32_t P = segments_for(true, with_o != 0, forced, n_seqs, n_tokens, n_heads, dk, dv);
    const size_t b = replay_need(true, with_o != 0, P, n_seqs, n_tokens, n_heads, dk, dv);
    best = b > best ? b : best;
  }
  return best;
}

// raw: the inputs are raw projections (gdn_replay_raw; bf16 only): the
// record builder normalises keys and queries and activates the gates, and
// the workspace ends with their reciprocal norms.
gdn_status replay_impl(const void *q, const void *k, const void *v, const void *alpha, const void *beta,
                       const float *S0, const int32_t *cu_seqlens, int32_t n_seqs, int64_t n_tokens,
                       int32_t n_heads, int32_t dk, int32_t dv, gdn_dtype in_dtype, void *o, gdn_dtype o_dtype,
                       float *S_final, int32_t forced_segments, void *workspace, size_t workspace_bytes,
                       gdn_stream_t stream, const char *fn, bool raw = false) {
  if (!k || !v || !alpha || !beta || !cu_seqlens || !S_final)
    return fail(GDN_ERR_NULL_POINTER, "%s: k, v, alpha, beta, cu_seqlens and S_final are required", fn);
  if (o && !q) return fail(GDN_ERR_NULL_POINTER, "%s: o requested without q", fn);
  if (n_seqs < 1 || n_tokens < 0 || n_heads < 1 || dk < 1 || dv < 1)
    return fail(GDN_ERR_BAD_SHAPE, "%s: need n_seqs >= 1, n_tokens >= 0, n_heads >= 1 (got %d, %lld, %d)", fn,
                n_seqs, (long long)n_tokens, n_heads);
  if (!supported_dim(dk) || !supported_dim(dv))
    return fail(GDN_ERR_UNSUPPORTED, "%s: dk and dv must be 64 or 128 (got %d, %d)", fn, dk, dv);
  if (!valid_dtype(in_dtype) || (o && !valid_dtype(o_dtype)))
    return fail(GDN_ERR_UNSUPPORTED, "%s: dtypes must be GDN_F32 or GDN_BF16", fn);
  if (raw && in_dtype != GDN_BF16) return fail(GDN_ERR_UNSUPPORTED, "%s: raw inputs must be GDN_BF16", fn);
  if (n_tokens > kMaxTokens || n_heads > kMaxHeads || (int64_t)n_seqs * n_heads * (dv / 16) > (int64_t(1) << 30))
    return fail(GDN_ERR_UNSUPPORTED, "%s: problem too large for one call", fn);
  gdn_status s;
  if ((s = check_align("q", q)) || (s = check_align("k", k)) || (s = check_align("v", v)) ||
      (s = check_align("alpha", alpha)) || (s = check_align("beta", beta)) || (s = check_align("S0", S0)) ||
      (s = check_align("cu_seqlens", cu_seqlens)) || (s = check_align("o", o)) ||
      (s = check_align("S_final", S_final)))
    return s;
  const bool bf = in_dtype == GDN_BF16;
  const int32_t P = segments_for(bf, o != nullptr, forced_segments, n_seqs, n_tokens, n_heads, dk, dv);
  const size_t tau_bytes = gdn::tau_workspace_bytes(n_tokens, n_seqs, n_heads);
  // longest-first sequence order (bf16 replays without a time split, built by the prep kernel)
  const bool ordered = bf && P == 1 && gdn::order_workspace_bytes(n_seqs) > 0;
  const size_t base = replay_need(bf, o != nullptr, P, n_seqs, n_tokens, n_heads, dk, dv);
  const size_t need = base + (raw ? gdn::norm_workspace_bytes(n_tokens, n_seqs, n_heads) : 0);
  if (workspace_bytes < need || !workspace)
    return fail(GDN_ERR_WORKSPACE, "%s: workspace of %zu bytes required (got %zu)", fn, need, workspace_bytes);
  if ((s = check_align("workspace", workspace))) return s;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  float *norms = raw ? reinterpret_cast<float *>(static_cast<char *>(workspace) + base) : nullptr;
  gdn::PrepLaunch pp{};
  pp.raw = raw ? 1 : 0;
  pp.norms = norms;
  pp.k = k;
  pp.alpha = alpha;
  pp.beta = beta;
  pp.cu = cu_seqlens;
  pp.n_seqs = n_seqs;
  pp.H = n_heads;
  pp.dk = dk;
  pp.in_bf16 = in_dtype == GDN_BF16;
  pp.tau = static_cast<float *>(workspace);
  pp.n_slots = gdn::slot_count(n_tokens, n_seqs);
  int32_t *order = ordered ? reinterpret_cast<int32_t *>(static_cast<char *>(workspace) + tau_bytes) : nullptr;
  pp.order = order;
  // bf16 time-split replays build the per-chunk records inside the segment
  // kernel; everything else runs the stand-alone prep kernel first
  const bool fuse = bf && P > 1;   // (records built inside the segment launch)
  if (!fuse && (s = launched(gdn::launch_prep(pp, st), "gdn_replay prep launch"))) return s;
  gdn::ChainLaunch p{};
  p.tau = pp.tau;
  p.q = o ? q : nullptr;
  p.k = k;
  p.v = v;
  p.alpha = alpha;
  p.beta = beta;
  p.S0 = S0;
  p.cu = cu_seqlens;
  p.n_seqs = n_seqs;
  p.H = n_heads;
  p.dk = dk;
  p.dv = dv;
  p.in_bf16 = in_dtype == GDN_BF16;
  p.o = o;
  p.o_bf16 = o_dtype == GDN_BF16;
  p.raw = raw ? 1 : 0;
  p.norms = norms;
  p.n_segs = 1;
  if (P == 1) {
    p.order = order;
    p.S_out = S_final;
    p.T_out = nullptr;
    p.tiles_T = 0;
    p.tiles_S = dv / 16;
    return launched(bf ? gdn::launch_chain_bf16(p, st) : gdn::launch_chain(p, st), "gdn_replay launch");
  }
  // time split: segment operators, then their composition
  float *Tseg = reinterpret_cast<float *>(static_cast<char *>(workspace) + tau_bytes);
  float *Sseg = Tseg + (size_t)n_seqs * P * n_heads * dk * dk;
  float *Spre = Sseg + (size_t)n_seqs * P * n_heads * dv * dk;   // start states (with outputs)
  p.n_segs = P;
  p.lead = o ? 1 : 0;   // with outputs: segment 0 runs with them here
  p.fuse_prep = 1;
  p.skip_T0 = 1;
  p.T_frags = 1;
  p.tiles_T = dk / 16;
  p.tiles_S = dv / 16;
  p.T_out = Tseg;
  p.S_out = Sseg;
  if ((s = launched(gdn::launch_chain_bf16(p, st), "gdn_replay segment launch"))) return s;
  gdn::SegComposeLaunch c{};
  c.S_seg = Sseg;
  c.T_frag = Tseg;
  c.n_seqs = n_seqs;
  c.n_segs = P;
  c.H = n_heads;
  c.dk = dk;
  c.dv = dv;
  c.S_out = o ? nullptr : S_final;
  c.S_prefix = o ? Spre : nullptr;
  c.S0 = S0;
  c.lead = o ? 1 : 0;
  if ((s = launched(gdn::launch_seg_compose(c, st), "gdn_replay segment compose launch"))) return s;
  if (!o) return ok();
  // outputs: segments 1 .. P - 1 from their start states, with the records
  // the segment launch built; the last one ends in S_final
  gdn::ChainLaunch r = p;
  r.S0 = nullptr;
  r.S0_seg = Spre;
  r.S_out = nullptr;
  r.S_last = S_final;
  r.T_out = nullptr;
  r.tiles_T = 0;
  r.T_frags = 0;
  r.fuse_prep = 0;
  return launched(gdn::launch_chain_bf16(r, st), "gdn_replay segment output launch");
}


// ---------------------------------------------------------------------------
// Built-in scratch of gdn_replay_noalloc: a file-scope device array, one copy
// per GPU, held until the process ends.  Host code never passes the array's
// name to a kernel (on the host it only names a stand-in): the device address
// of this GPU's copy comes from hipGetSymbolAddress, taken once per device
// with that device current, and only that address is used.
// ---------------------------------------------------------------------------
__device__ __attribute__((aligned(256))) char scratch[GDN_NOALLOC_SCRATCH_BYTES];

std::once_flag g_scratch_once[kMaxDevices];
void *g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// This device's copy of the scratch array (nullptr and a failed status if
// the current device cannot be read or the symbol has no address).
void *device_scratch(hipError_t &err) {
  int dev = 0;
  err = hipGetDevice(&dev);
  if (err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::call_once(g_scratch_once[dev], [dev] {
    void *ptr = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? ptr : nullptr;
  });
  err = g_scratch_err[dev];
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

size_t gdn_replay_workspace_bytes(int32_t n_seqs, int64_t n_tokens, int32_t n_heads, int32_t dk, int32_t dv) {
  return replay_workspace_max(n_seqs, n_tokens, n_heads, dk, dv, 0);
}

size_t gdn_replay_segmented_workspace_bytes(int32_t n_seqs, int64_t n_tokens, int32_t n_heads, int32_t dk,
                                            int32_t dv, int32_t segments) {
  if (segments < 0) return 0;
  return replay_workspace_max(n_seqs, n_tokens, n_heads, dk, dv, segments);
}

size_t gdn_chunk_operator_workspace_bytes(int32_t n_chunks, int64_t n_tokens, int32_t n_heads, int32_t,
                                          int32_t) {
  if (n_chunks < 1 || n_tokens < 0 || n_heads < 1) return 0;
  return gdn::tau_workspace_bytes(n_tokens, n_chunks, n_heads);
}

size_t gdn_compose_workspace_bytes(int32_t n_chunks, int32_t n_heads, int32_t dk, int32_t) {
  // the operators as composition fragments: as many bytes as T_C
  if (n_chunks < 1 || n_heads < 1 || dk < 1) return 0;
  return (size_t)n_chunks * n_heads * dk * dk * sizeof(float);
}

gdn_status gdn_replay(const void *q, const void *k, const void *v, const void *alpha, const void *beta,
                      const float *S0, const int32_t *cu_seqlens, int32_t n_seqs, int64_t n_tokens,
                      int32_t n_heads, int32_t dk, int32_t dv, gdn_dtype in_dtype, void *o, gdn_dtype o_dtype,
                      float *S_final, void *workspace, size_t workspace_bytes, gdn_stream_t stream) {
  return replay_impl(q, k, v, alpha, beta, S0, cu_seqlens, n_seqs, n_tokens, n_heads, dk, dv, in_dtype, o, o_dtype,
                     S_final, 0, workspace, workspace_bytes, stream, "gdn_replay");
}

size_t gdn_replay_raw_workspace_bytes(int32_t n_seqs, int64_t n_tokens, int32_t n_heads, int32_t dk, int32_t dv) {
  const size_t b = replay_workspace_max(n_seqs, n_tokens, n_heads, dk, dv, 0);
  return b ? b + gdn::norm_workspace_bytes(n_tokens, n_seqs, n_heads) : 0;
}

gdn_status gdn_replay_raw(const void *q_raw, const void *k_raw, const void *v, const void *g, const void *b,
                          const float *S0, const int32_t *cu_seqlens, int32_t n_seqs, int64_t n_tokens,
                          int32_t n_heads, int32_t dk, int32_t dv, gdn_dtype in_dtype, void *o, gdn_dtype o_dtype,
                          float *S_final, void *workspace, size_t workspace_bytes, gdn_stream_t stream) {
  return replay_impl(q_raw, k_raw, v, g, b, S0, cu_seqlens, n_seqs, n_tokens, n_heads, dk, dv, in_dtype, o, o_dtype,
                     S_final, 0, workspace, workspace_bytes, stream, "gdn_replay_raw", true);
}

gdn_status gdn_replay_segmented(const void *q, const void *k, const void *v, const void *alpha, const void *beta,
                                const float *S0, const int32_t *cu_seqlens, int32_t n_seqs, int64_t n_tokens,
                                int32_t n_heads, int32_t dk, int32_t dv, gdn_dtype in_dtype, void *o,
                                gdn_dtype o_dtype, float *S_final, int32_t segments, void *workspace,
                                size_t workspace_bytes, gdn_stream_t stream) {
  if (segments < 0 || segments > kMaxSegments)
    return fail(GDN_ERR_BAD_SHAPE, "gdn_replay_segmented: segments must be 0 .. %d (got %d)", kMaxSegments, segments);
  return replay_impl(q, k, v, alpha, beta, S0, cu_seqlens, n_seqs, n_tokens, n_heads, dk, dv, in_dtype, o, o_dtype,
                     S_final, segments, workspace, workspace_bytes, stream, "gdn_replay_segmented");
}

gdn_status gdn_replay_noalloc(const void *q, const void *k, const void *v, const void *alpha, const void *beta,
                              const float *S0, const int32_t *cu_seqlens, int32_t n_seqs, int64_t n_tokens,
                              int32_t n_heads, int32_t dk, int32_t dv, gdn_dtype in_dtype, void *o,
                              gdn_dtype o_dtype, float *S_final, gdn_stream_t stream) {
  // the sizes are checked first (host only), so an oversized call fails
  // before the device is touched
  if (n_seqs >= 1 && n_tokens >= 0 && n_heads >= 1 && supported_dim(dk) && supported_dim(dv) &&
      valid_dtype(in_dtype) && n_tokens <= kMaxTokens && n_heads <= kMaxHeads) {
    const bool bf = in_dtype == GDN_BF16;
    const int32_t P = segments_for(bf, o != nullptr, 0, n_seqs, n_tokens, n_heads, dk, dv);
    const size_t need = replay_need(bf, o != nullptr, P, n_seqs, n_tokens, n_heads, dk, dv);
    if (need > (size_t)GDN_NOALLOC_SCRATCH_BYTES)
      return fail(GDN_ERR_WORKSPACE,
                  "gdn_replay_noalloc: this replay needs %zu bytes of scratch, more than the built-in %zu; "
                  "call gdn_replay with a workspace",
                  need, (size_t)GDN_NOALLOC_SCRATCH_BYTES);
  }
  hipError_t e = hipSuccess;
  void *ws = nullptr;
  if (k && v && alpha && beta && cu_seqlens && S_final) {
    ws = device_scratch(e);
    if (!ws) return fail(GDN_ERR_HIP, "gdn_replay_noalloc: no device address for the scratch: %s", hipGetErrorString(e));
  }
  return replay_impl(q, k, v, alpha, beta, S0, cu_seqlens, n_seqs, n_tokens, n_heads, dk, dv, in_dtype, o, o_dtype,
                     S_final, 0, ws, GDN_NOALLOC_SCRATCH_BYTES, stream, "gdn_replay_noalloc");
}

gdn_status gdn_chunk_operator(const void *k, const void *v, const void *alpha, const void *beta,
                              const int32_t *cu_chunks, int32_t n_chunks, int64_t n_tokens, int32_t n_heads,
                              int32_t dk, int32_t dv, gdn_dtype in_dtype, float *T_C, float *S_local,
                              void *workspace, size_t workspace_bytes, gdn_stream_t stream) {
  if (!k || !alpha || !beta || !cu_chunks || !T_C)
    return fail(GDN_ERR_NULL_POINTER, "gdn_chunk_operator: k, alpha, beta, cu_chunks and T_C are required");
  if ((v == nullptr) != (S_local == nullptr))
    return fail(GDN_ERR_NULL_POINTER, "gdn_chunk_operator: v and S_local must be given together");
  if (n_chunks < 0 || n_tokens < 0 || n_heads < 1 || dk < 1 || dv < 1)
    return fail(GDN_ERR_BAD_SHAPE, "gdn_chunk_operator: bad sizes (n_chunks %d, n_tokens %lld, n_heads %d)",
                n_chunks, (long long)n_tokens, n_heads);
  if (!supported_dim(dk) || !supported_dim(dv))
    return fail(GDN_ERR_UNSUPPORTED, "gdn_chunk_operator: dk and dv must be 64 or 128 (got %d, %d)", dk, dv);
  if (!valid_dtype(in_dtype)) return fail(GDN_ERR_UNSUPPORTED, "gdn_chunk_operator: bad dtype");
  if (n_tokens > kMaxTokens || n_heads > kMaxHeads || (int64_t)n_chunks * n_heads * ((dk + dv) / 16) > (int64_t(1) << 30))
    return fail(GDN_ERR_UNSUPPORTED, "gdn_chunk_operator: problem too large for one call");
  gdn_status s;
  if ((s = check_align("k", k)) || (s = check_align("v", v)) || (s = check_align("alpha", alpha)) ||
      (s = check_align("beta", beta)) || (s = check_align("cu_chunks", cu_chunks)) ||
      (s = check_align("T_C", T_C)) || (s = check_align("S_local", S_local)))
    return s;
  if (n_chunks == 0) return ok();
  const size_t need = gdn_chunk_operator_workspace_bytes(n_chunks, n_tokens, n_heads, dk, dv);
  if (workspace_bytes < need || !workspace)
    return fail(GDN_ERR_WORKSPACE, "gdn_chunk_operator: workspace of %zu bytes required (got %zu)", need,
                workspace_bytes);
  if ((s = check_align("workspace", workspace))) return s;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  gdn::PrepLaunch pp{};
  pp.k = k;
  pp.alpha = alpha;
  pp.beta = beta;
  pp.cu = cu_chunks;
  pp.n_seqs = n_chunks;
  pp.H = n_heads;
  pp.dk = dk;
  pp.in_bf16 = in_dtype == GDN_BF16;
  pp.tau = static_cast<float *>(workspace);
  pp.n_slots = gdn::slot_count(n_tokens, n_chunks);
  // bf16: each chunk's workgroup builds the records of its own 64-token
  // sub-chunks first (no separate prep launch)
  const bool fuse = in_dtype == GDN_BF16;
  if (!fuse && (s = launched(gdn::launch_prep(pp, st), "gdn_chunk_operator prep launch"))) return s;
  gdn::ChainLaunch p{};
  p.tau = pp.tau;
  p.k = k;
  p.v = v;
  p.alpha = alpha;
  p.beta = beta;
  p.cu = cu_chunks;
  p.n_seqs = n_chunks;
  p.H = n_heads;
  p.dk = dk;
  p.dv = dv;
  p.in_bf16 = in_dtype == GDN_BF16;
  p.S_out = S_local;
  p.T_out = T_C;
  p.n_segs = 1;
  p.tiles_T = dk / 16;
  p.tiles_S = v ? dv / 16 : 0;
  p.fuse_prep = fuse ? 1 : 0;
  // bf16 with transition and state rows in one workgroup per (chunk, head),
  // more of them than two per compute unit: one workgroup per compute unit,
  // each running its run of (chunk, head) items as one stream of chunks
  // (records of all of them built first, an item's first copies issued
  // during the previous item's last chunk)
  const int cus = device_cus();
  if (fuse && (dk + (v ? dv : 0)) / 16 > 8 && (int64_t)n_chunks * n_heads > 2 * (int64_t)cus) p.multi_wgs = cus;
  return launched(p.in_bf16 ? gdn::launch_chain_bf16(p, st) : gdn::launch_chain(p, st),
                  "gdn_chunk_operator launch");
}

gdn_status gdn_compose(const float *S_in, const float *T_C, const float *S_local, int32_t n_chunks,
                       int32_t n_heads, int32_t dk, int32_t dv, float *S_out, void *workspace,
                       size_t workspace_bytes, gdn_stream_t stream) {
  if (!S_out || (n_chunks > 0 && (!T_C || !S_local)))
    return fail(GDN_ERR_NULL_POINTER, "gdn_compose: T_C, S_local and S_out are required");
  if (n_chunks < 0 || n_heads < 1 || dk < 1 || dv < 1)
    return fail(GDN_ERR_BAD_SHAPE, "gdn_compose: bad sizes (n_chunks %d, n_heads %d)", n_chunks, n_heads);
  if (!supported_dim(dk) || !supported_dim(dv))
    return fail(GDN_ERR_UNSUPPORTED, "gdn_compose: dk and dv must be 64 or 128 (got %d, %d)", dk, dv);
  if ((int64_t)n_chunks * n_heads * (dk / 32) > INT32_MAX)
    return fail(GDN_ERR_UNSUPPORTED, "gdn_compose: too many operators for one call (%d chunks x %d heads)", n_chunks,
                n_heads);
  gdn_status s;
  if ((s = check_align("S_in", S_in)) || (s = check_align("T_C", T_C)) || (s = check_align("S_local", S_local)) ||
      (s = check_align("S_out", S_out)))
    return s;
  const size_t need = gdn_compose_workspace_bytes(n_chunks, n_heads, dk, dv);
  if (workspace_bytes < need || (need > 0 && !workspace))
    return fail(GDN_ERR_WORKSPACE, "gdn_compose: workspace of %zu bytes required (got %zu)", need, workspace_bytes);
  if ((s = check_align("workspace", workspace))) return s;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  // operators into fragments (all at once), then the chain per (head, 32 rows)
  if (n_chunks > 0 && (s = launched(gdn::launch_op_frags(T_C, (int64_t)n_chunks * n_heads, dk, workspace, st),
                                    "gdn_compose operator launch")))
    return s;
  gdn::SegComposeLaunch c{};
  c.S_seg = S_local;
  c.T_frag = workspace;
  c.S_prefix = nullptr;
  c.S0 = S_in;
  c.n_seqs = 1;
  c.n_segs = n_chunks;
  c.H = n_heads;
  c.dk = dk;
  c.dv = dv;
  c.S_out = S_out;
  c.from_start = 1;
  return launched(gdn::launch_seg_compose(c, st), "gdn_compose launch");
}

gdn_status gdn_decode(const void *q, const void *k, const void *v, const void *alpha, const void *beta,
                      const float *S_in, int32_t n_seqs, int32_t n_heads, int32_t dk, int32_t dv,
                      gdn_dtype in_dtype, void *o, gdn_dtype o_dtype, float *S_out, gdn_stream_t stream) {
  if (!k || !v || !alpha || !beta || !S_out)
    return fail(GDN_ERR_NULL_POINTER, "gdn_decode: k, v, alpha, beta and S_out are required");
  if (o && !q) return fail(GDN_ERR_NULL_POINTER, "gdn_decode: o requested without q");
  if (n_seqs < 0 || n_heads < 1 || dk < 1 || dv < 1)
    return fail(GDN_ERR_BAD_SHAPE, "gdn_decode: need n_seqs >= 0 and n_heads >= 1 (got %d, %d)", n_seqs, n_heads);
  if (!supported_dim(dk) || !supported_dim(dv))
    return fail(GDN_ERR_UNSUPPORTED, "gdn_decode: dk and dv must be 64 or 128 (got %d, %d)", dk, dv);
  if (!valid_dtype(in_dtype) || (o && !valid_dtype(o_dtype)))
    return fail(GDN_ERR_UNSUPPORTED, "gdn_decode: dtypes must be GDN_F32 or GDN_BF16");
  if (n_heads > kMaxHeads || (int64_t)n_seqs * n_heads > INT32_MAX)
    return fail(GDN_ERR_UNSUPPORTED, "gdn_decode: problem too large for one call");
  gdn_status s;
  if ((s = check_align("q", q)) || (s = check_align("k", k)) || (s = check_align("v", v)) ||
      (s = check_align("alpha", alpha)) || (s = check_align("beta", beta)) || (s = check_align("S_in", S_in)) ||
      (s = check_align("o", o)) || (s = check_align("S_out", S_out)))
    return s;
  gdn::DecodeLaunch p{};
  p.q = o ? q : nullptr;
  p.k = k;
  p.v = v;
  p.alpha = alpha;
  p.beta = beta;
  p.S_in = S_in;
  p.S_out = S_out;
  p.o = o;
  p.n_seqs = n_seqs;
  p.H = n_heads;
  p.dk = dk;
  p.dv = dv;
  p.in_bf16 = in_dtype == GDN_BF16;
  p.o_bf16 = o_dtype == GDN_BF16;
  return launched(gdn::launch_decode(p, reinterpret_cast<hipStream_t>(stream)), "gdn_decode launch");
}

gdn_status gdn_front_end(const void *q_raw, const void *k_raw, const void *g, const void *b, int64_t n_tokens,
                         int32_t n_heads, int32_t dk, gdn_dtype dtype, void *q, void *k, void *alpha, void *beta,
                         gdn_stream_t stream) {
  if (!k_raw || !g || !b || !k || !alpha || !beta)
    return fail(GDN_ERR_NULL_POINTER, "gdn_front_end: k_raw, g, b, k, alpha and beta are required");
  if (!q_raw != !q) return fail(GDN_ERR_NULL_POINTER, "gdn_front_end: q_raw and q must both be given or both NULL");
  if (n_tokens < 0 || n_heads < 1)
    return fail(GDN_ERR_BAD_SHAPE, "gdn_front_end: need n_tokens >= 0 and n_heads >= 1 (got %lld, %d)",
                (long long)n_tokens, n_heads);
  if (!supported_dim(dk)) return fail(GDN_ERR_UNSUPPORTED, "gdn_front_end: dk must be 64 or 128 (got %d)", dk);
  if (!valid_dtype(dtype)) return fail(GDN_ERR_UNSUPPORTED, "gdn_front_end: dtype must be GDN_F32 or GDN_BF16");
  if (n_heads > kMaxHeads || n_tokens > (int64_t)1 << 40)
    return fail(GDN_ERR_UNSUPPORTED, "gdn_front_end: problem too large for one call");
  gdn_status s;
  if ((s = check_align("q_raw", q_raw)) || (s = check_align("k_raw", k_raw)) || (s = check_align("g", g)) ||
      (s = check_align("b", b)) || (s = check_align("q", q)) || (s = check_align("k", k)) ||
      (s = check_align("alpha", alpha)) || (s = check_align("beta", beta)))
    return s;
  gdn::FrontLaunch p{};
  p.q_in = q_raw;
  p.k_in = k_raw;
  p.g = g;
  p.b = b;
  p.q_out = q;
  p.k_out = k;
  p.alpha = alpha;
  p.beta = beta;
  p.n_tokens = n_tokens;
  p.H = n_heads;
  p.dk = dk;
  p.in_bf16 = dtype == GDN_BF16;
  return launched(gdn::launch_front(p, reinterpret_cast<hipStream_t>(stream)), "gdn_front_end launch");
}

gdn_status gdn_scalar_chunk_operator(const void *k, const void *v, const void *alpha, const void *beta,
                                     const int32_t *cu_chunks, int32_t n_chunks, int64_t n_tokens, int32_t n_heads,
                                     int32_t dk, int32_t dv, gdn_dtype in_dtype, float *gamma, float *S_local,
                                     gdn_stream_t stream) {
  if (!k || !alpha || !beta || !cu_chunks || !gamma)
    return fail(GDN_ERR_NULL_POINTER, "gdn_scalar_chunk_operator: k, alpha, beta, cu_chunks and gamma are required");
  if (S_local && !v) return fail(GDN_ERR_NULL_POINTER, "gdn_scalar_chunk_operator: S_local requested without v");
  if (n_chunks < 0 || n_tokens < 0 || n_heads < 1)
    return fail(GDN_ERR_BAD_SHAPE, "gdn_scalar_chunk_operator: need n_chunks >= 0, n_tokens >= 0, n_heads >= 1");
  if (!supported_dim(dk) || !supported_dim(dv))
    return fail(GDN_ERR_UNSUPPORTED, "gdn_scalar_chunk_operator: dk and dv must be 64 or 128 (got %d, %d)", dk, dv);
  if (!valid_dtype(in_dtype)) return fail(GDN_ERR_UNSUPPORTED, "gdn_scalar_chunk_operator: dtype must be F32 or BF16");
  if (n_heads > kMaxHeads || (int64_t)n_chunks * n_heads > INT32_MAX || n_tokens > INT32_MAX)
    return fail(GDN_ERR_UNSUPPORTED, "gdn_scalar_chunk_operator: problem too large for one call");
  gdn_status s;
  if ((s = check_align("k", k)) || (s = check_align("v", v)) || (s = check_align("alpha", alpha)) ||
      (s = check_align("beta", beta)) || (s = check_align("cu_chunks", cu_chunks)) ||
      (s = check_align("gamma", gamma)) || (s = check_align("S_local", S_local)))
    return s;
  gdn::ScalarOpLaunch p{};
  p.k = k;
  p.v = v;
  p.alpha = alpha;
  p.beta = beta;
  p.cu = cu_chunks;
  p.gamma = gamma;
  p.S_local = S_local;
  p.n_chunks = n_chunks;
  p.H = n_heads;
  p.dk = dk;
  p.dv = dv;
  p.in_bf16 = in_dtype == GDN_BF16;
  p.n_tokens = n_tokens;
  return launched(gdn::launch_scalar_op(p, reinterpret_cast<hipStream_t>(stream)), "gdn_scalar_chunk_operator launch");
}

gdn_status gdn_scalar_compose(const float *S_in, const float *gamma, const float *S_local, int32_t n_chunks,
                              int32_t n_heads, int32_t dk, int32_t dv, float *S_out, gdn_stream_t stream) {
  if (!S_out || (n_chunks > 0 && (!gamma || !S_local)))
    return fail(GDN_ERR_NULL_POINTER, "gdn_scalar_compose: S_out, and gamma and S_local when n_chunks > 0, are required");
  if (n_chunks < 0 || n_heads < 1) return fail(GDN_ERR_BAD_SHAPE, "gdn_scalar_compose: need n_chunks >= 0, n_heads >= 1");
  if (!supported_dim(dk) || !supported_dim(dv))
    return fail(GDN_ERR_UNSUPPORTED, "gdn_scalar_compose: dk and dv must be 64 or 128 (got %d, %d)", dk, dv);
  if (n_heads > kMaxHeads) return fail(GDN_ERR_UNSUPPORTED, "gdn_scalar_compose: too many heads");
  gdn_status s;
  if ((s = check_align("S_in", S_in)) || (s = check_align("gamma", gamma)) || (s = check_align("S_local", S_local)) ||
      (s = check_align("S_out", S_out)))
    return s;
  gdn::ScalarComposeLaunch p{};
  p.S_in = S_in;
  p.gamma = gamma;
  p.S_local = S_local;
  p.S_out = S_out;
  p.n_chunks = n_chunks;
  p.H = n_heads;
  p.dk = dk;
  p.dv = dv;
  return launched(gdn::launch_scalar_compose(p, reinterpret_cast<hipStream_t>(stream)), "gdn_scalar_compose launch");
}

const char *gdn_status_string(gdn_status status) {
  switch (status) {
    case GDN_OK: return "GDN_OK";
    case GDN_ERR_NULL_POINTER: return "GDN_ERR_NULL_POINTER";
    case GDN_ERR_BAD_SHAPE: return "GDN_ERR_BAD_SHAPE";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED";
    case GDN_ERR_ALIGNMENT: return "GDN_ERR_ALIGNMENT";
    case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE";
    case GDN_ERR_HIP: return "GDN_ERR_HIP";
  }
  return "GDN_ERR_UNKNOWN";
}

const char *gdn_last_error(void) { return g_last_error.c_str(); }

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

}  // extern "C"
