// gdn_prep_bf16.hip -- per-chunk UT transform for bf16 inputs on gfx950:
// one wave per (chunk slot, head) running prep_chunk_wave (gdn_prep_wave.h),
// each in a workgroup of its own with its LDS scratch (no barriers), so that
// the scratch and register use alone set how many waves share a compute
// unit.  The factor
// Tau = (I + A)^{-1} follows from the page "Tail-Replay: Escaping the Curse
// of Linear Attention in Prefix Caching for Hybrid LLMs", section 2
// Eq. (1), unrolled over a chunk.
#include "gdn_prep_wave.h"

namespace gdn {

namespace {

constexpr int PW = 1;   // waves per workgroup

// Largest n in [0, n_seqs) whose first chunk slot floor(cu[n]/64) + n is <= slot.
__device__ __forceinline__ int find_seq_b(const int32_t *cu, int n_seqs, int64_t slot) {
  int lo = 0, hi = n_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int64_t)(cu[mid] / kChunk) + mid <= slot)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// Longest-first order of the sequences by chunk count (ties by index): each
// lane ranks its sequences against all others (the inner loop is uniform, so
// cu comes through scalar loads); ranks are distinct, so order is a
// permutation.
__device__ __forceinline__ void rank_sequences(const int32_t *cu, int n_seqs, int32_t *order) {
  for (int i = lane_id(); i < n_seqs; i += 64) {
    const int ci = (cu[i + 1] - cu[i] + kChunk - 1) / kChunk;
    int r = 0;
    for (int j = 0; j < n_seqs; ++j) {
      const int cj = (cu[j + 1] - cu[j] + kChunk - 1) / kChunk;
      r += (cj > ci || (cj == ci && j < i)) ? 1 : 0;
    }
    order[r] = i;
  }
}

template <int DK, bool RAW>
__global__ void __launch_bounds__(PW * 64) prep_bf16_kernel(PrepLaunch p) {
  __shared__ __attribute__((aligned(16))) float scratch[PW][kPrepWaveLds / 4];
  const int w = __builtin_amdgcn_readfirstlane(wave_id());
  if (p.order && blockIdx.x == 0 && blockIdx.y == 0 && w == 0) rank_sequences(p.cu, p.n_seqs, p.order);
  const int64_t slot = (int64_t)blockIdx.x * PW + w;
  if (slot >= p.n_slots) return;
  const int h = blockIdx.y, H = p.H;
  const int n = find_seq_b(p.cu, p.n_seqs, slot);
  const int tbeg = p.cu[n], len = p.cu[n + 1] - tbeg;
  const int64_t j = slot - ((int64_t)(tbeg / kChunk) + n);
  if (j < 0 || j * kChunk >= len) return;  // slot past the end of its sequence
  const int t0 = tbeg + (int)j * kChunk;
  const int Lc = min(kChunk, len - (int)j * kChunk);
  char *rec = reinterpret_cast<char *>(p.tau + (slot * H + h) * (int64_t)kRecFloats);
  prep_chunk_wave<DK, RAW>(reinterpret_cast<const bf16 *>(p.k), reinterpret_cast<const bf16 *>(p.alpha),
                           reinterpret_cast<const bf16 *>(p.beta), H, h, t0, Lc, rec, scratch[w], nullptr,
                           RAW ? p.norms + (slot * H + h) * kNormFloats : nullptr);
}

template <int DK>
hipError_t launch_pb(const PrepLaunch &p, hipStream_t stream) {
  if (p.n_slots <= 0) return hipSuccess;
  if (p.raw && !p.norms) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((p.n_slots + PW - 1) / PW), (unsigned)p.H);
  return p.raw ? launch_kernel(prep_bf16_kernel<DK, true>, grid, dim3(PW * 64), 0, stream, p)
               : launch_kernel(prep_bf16_kernel<DK, false>, grid, dim3(PW * 64), 0, stream, p);
}

}  // namespace

hipError_t launch_prep_bf16(const PrepLaunch &p, hipStream_t stream) {
  if (p.dk == 64) return launch_pb<64>(p, stream);
  if (p.dk == 128) return launch_pb<128>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace gdn
