// gdn_prep.hip -- per-chunk UT transform for the chunkwise GDN recurrence.
//
// For a chunk of L <= 64 tokens (page "Tail-Replay: Escaping the Curse of
// Linear Attention in Prefix Caching for Hybrid LLMs", section 2 Eq. (1),
// unrolled over the chunk) the per-token delta-rule corrections D satisfy
//     (I + A) D = diag(beta) (V - diag(e^g) K S^T),
//     A = strictly lower part of  beta_r exp(g_r - g_s) (k_r . k_s),
// with g the cumulative log-gate.  A depends only on keys and gates, so its
// inverse Tau = (I + A)^{-1} (unit lower triangular) is built here once per
// (chunk, head), fully in parallel, and consumed by every row tile of the
// recurrence kernel.
//
// One workgroup (4 waves) per (chunk slot, head):
//   1. keys of the chunk to LDS; cumulative log-gates by a wave-wide scan
//   2. A = scaled K K^T on fp32 MFMA, 10 lower 16 x 16 blocks
//   3. inverses of the four diagonal 16 x 16 blocks by forward substitution
//      (one lane per column)
//   4. off-diagonal blocks Tau_ij = -Tau_ii sum_{m=j}^{i-1} A_im Tau_mj; a
//      block column depends only on the diagonal blocks and the blocks above
//      it, so one wave per block column (fp32 MFMA)
// The result is written packed (lower block rows only) in fp32.  This
// kernel serves fp32 inputs; bf16 inputs have their own (gdn_prep_bf16.hip).
#include "gdn_device.h"
#include "gdn_internal.h"

#include <type_traits>

namespace gdn {

namespace {

constexpr int PNW = 4;
constexpr int PNT = PNW * 64;

template <class Tin, int DK>
struct PCfg {
  static constexpr bool BF = std::is_same<Tin, bf16>::value;
  static constexpr int LDK = BF ? DK + 8 : DK + 1;  // sK [64][LDK] Tin
  static constexpr int LDC = BF ? 68 : 65;          // sA, sTau [64][LDC] fp32
  static constexpr int LDX = 17;
  static constexpr size_t al(size_t x) { return (x + 15) & ~size_t(15); }
  static constexpr size_t oK = 0;
  static constexpr size_t oA = oK + al(sizeof(Tin) * 64 * LDK);
  static constexpr size_t oTau = oA + al(4 * 64 * LDC);
  static constexpr size_t oX = oTau + al(4 * 64 * LDC);
  static constexpr size_t oGate = oX + (BF ? 0 : al(4 * 3 * 16 * LDX));
  static constexpr size_t TOTAL = oGate + al(4 * 2 * 64);
  static constexpr int VEC = 16 / sizeof(Tin);
  static constexpr int KSEG = DK / VEC;
  static constexpr int NKP = (64 * KSEG + PNT - 1) / PNT;
};



// Largest n in [0, n_seqs) whose first chunk slot floor(cu[n]/64) + n is <= slot.
__device__ __forceinline__ int find_seq(const int32_t *cu, int n_seqs, int64_t slot) {
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

template <class Tin, int DK>
__global__ void __launch_bounds__(PNT) prep_kernel(PrepLaunch p) {
  using C = PCfg<Tin, DK>;
  constexpr bool BF = C::BF;
  __shared__ __attribute__((aligned(16))) char smem[C::TOTAL];
  Tin *sK = reinterpret_cast<Tin *>(smem + C::oK);
  float *sA = reinterpret_cast<float *>(smem + C::oA);
  float *sTau = reinterpret_cast<float *>(smem + C::oTau);
  float *sX = reinterpret_cast<float *>(smem + C::oX);
  float *sG = reinterpret_cast<float *>(smem + C::oGate);
  float *sBeta = sG + 64;

  const int64_t slot = blockIdx.x;
  const int h = blockIdx.y, H = p.H;
  const int n = find_seq(p.cu, p.n_seqs, slot);
  const int tbeg = p.cu[n], len = p.cu[n + 1] - tbeg;
  const int64_t j = slot - ((int64_t)(tbeg / kChunk) + n);
  if (j < 0 || j * kChunk >= len) return;  // slot past the end of its sequence
  const int t0 = tbeg + (int)j * kChunk;
  const int Lc = min(kChunk, len - (int)j * kChunk);
  const int tid = threadIdx.x, w = wave_id(), l = lane_id();
  // output: fp32 packed Tau
  float *out = p.tau + (slot * H + h) * (int64_t)kRecFloats;
  auto put = [&](int idx, float x) {
    if constexpr (!BF) out[idx] = x;
  };

  // ---- 1. keys and gates ----
  const Tin *gk = reinterpret_cast<const Tin *>(p.k);
#pragma unroll
  for (int i = 0; i < C::NKP; ++i) {
    const int s = tid + i * PNT;
    if (s < 64 * C::KSEG) {
      const int r = s / C::KSEG, seg = s % C::KSEG;
      f32x4 x = zero4();
      if (r < Lc) x = *reinterpret_cast<const f32x4 *>(gk + ((int64_t)(t0 + r) * H + h) * DK + seg * C::VEC);
#pragma unroll
      for (int e = 0; e < 4; ++e) sK[r * C::LDK + seg * 4 + e] = x[e];
    }
  }
  if (w == 0) {
    float g = 0.f, b = 0.f;
    if (l < Lc) {
      const int64_t gi = (int64_t)(t0 + l) * H + h;
      g = log_gate(ld_in(reinterpret_cast<const Tin *>(p.alpha), gi));
      b = ld_in(reinterpret_cast<const Tin *>(p.beta), gi);
    }
    g = wave_inclusive_scan(g);
    sG[l] = g;
    sBeta[l] = b;
  }
  lds_barrier();

  // ---- 2. A = strictly-lower beta_r e^{g_r - g_s} K K^T ----
  for (int t = w; t < 10; t += PNW) {
    const int bi = t < 1 ? 0 : (t < 3 ? 1 : (t < 6 ? 2 : 3));
    const int bj = t - (bi * (bi + 1)) / 2;
    f32x4 c = zero4();
    mma_f32(c, RowMajor<float>{sK, C::LDK}, RowMajor<float>{sK, C::LDK}, 16 * bi, 16 * bj, 0, DK);
    const int col = 16 * bj + (l & 15);
    const float gc = sG[col];
    const int row0 = 16 * bi + 4 * (l >> 4);
    const f32x4 gr = *reinterpret_cast<const f32x4 *>(sG + row0);
    const f32x4 br = *reinterpret_cast<const f32x4 *>(sBeta + row0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      sA[(row0 + i) * C::LDC + col] = (col < row0 + i) ? br[i] * __expf(gr[i] - gc) * c[i] : 0.f;
  }
  lds_barrier();

  // ---- 3. diagonal blocks: lane (b, jj) solves column jj of block b ----
  if (w == 0) {
    const int b = l >> 4, jj = l & 15;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float *arow = sA + (16 * b + r) * C::LDC + 16 * b;
      float acc0 = (r == jj) ? 1.f : 0.f, acc1 = 0.f;
#pragma unroll
      for (int s = 0; s < r; ++s) {
        if (s & 1)
          acc1 -= arow[s] * x[s];
        else
          acc0 -= arow[s] * x[s];
      }
      x[r] = acc0 + acc1;
    }
    const int ob = tau_off(b) + 16 * b + jj;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sTau[(16 * b + r) * C::LDC + 16 * b + jj] = x[r];
      put(ob + r * 16 * (b + 1), x[r]);
    }
  }
  lds_barrier();

  // ---- 4. off-diagonal blocks, one block column per wave ----
  if (w < 3) {
    const int jc = w;
    {
      float *xs = sX + w * 16 * C::LDX;
      for (int i = jc + 1; i < 4; ++i) {
        f32x4 X = zero4();
        mma_f32(X, RowMajor<float>{sA + 16 * i * C::LDC, C::LDC}, ColMajor<float>{sTau + 16 * jc, C::LDC}, 0, 0,
                16 * jc, 16 * i);
        store_tile(xs, C::LDX, 0, 0, X);
        wave_lds_fence();
        f32x4 Y = zero4();
        mma_f32(Y, RowMajor<float>{sTau + 16 * i * C::LDC + 16 * i, C::LDC}, ColMajor<float>{xs, C::LDX}, 0, 0, 0,
                16);
#pragma unroll
        for (int q = 0; q < 4; ++q) Y[q] = -Y[q];
        store_tile(sTau, C::LDC, 16 * i, 16 * jc, Y);
        const int ob = tau_off(i) + 16 * jc + (l & 15);
#pragma unroll
        for (int q = 0; q < 4; ++q) put(ob + (4 * (l >> 4) + q) * 16 * (i + 1), Y[q]);
        wave_lds_fence();
      }
    }
  }

}

template <class Tin, int DK>
hipError_t launch_p(const PrepLaunch &p, hipStream_t stream) {
  if (p.n_slots <= 0) return hipSuccess;
  return launch_kernel(prep_kernel<Tin, DK>, dim3((unsigned)p.n_slots, (unsigned)p.H), dim3(PNT), 0, stream, p);
}

}  // namespace

hipError_t launch_prep(const PrepLaunch &p, hipStream_t stream) {
  if (p.in_bf16) {
    return launch_prep_bf16(p, stream);
  } else {
    if (p.dk == 64) return launch_p<float, 64>(p, stream);
    if (p.dk == 128) return launch_p<float, 128>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
