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
//   2. A = scaled K K^T on bf16 (or fp32) MFMA, 10 lower 16 x 16 blocks
//   3. inverses of the four diagonal 16 x 16 blocks by forward substitution
//      (one lane per column)
//   4. off-diagonal blocks Tau_ij = -Tau_ii sum_{m=j}^{i-1} A_im Tau_mj; a
//      block column depends only on the diagonal blocks and the blocks above
//      it, so one wave per block column, in registers (split-bf16 products)
// The result is written packed (lower block rows only) in fp32 for fp32
// inputs.  For bf16 inputs the record holds what the recurrence kernel feeds
// its k = 32 MFMAs, in their lane order (layout in gdn_internal.h), so that
// it can copy the record straight into LDS: Tau diag(beta) as split-bf16 A
// fragments, and K^T as the A fragments of its state update.
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
  // output: fp32 packed Tau (fp32 inputs); bf16 inputs: fragments, below
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
      if constexpr (BF) {
        *reinterpret_cast<f32x4 *>(sK + r * C::LDK + seg * C::VEC) = x;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) sK[r * C::LDK + seg * 4 + e] = x[e];
      }
    }
  }
  if (w == 0) {
    float g = 0.f, b = 0.f;
    if (l < Lc) {
      const int64_t gi = (int64_t)(t0 + l) * H + h;
      g = logf(ld_in(reinterpret_cast<const Tin *>(p.alpha), gi));
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
    if constexpr (BF)
      mma_bf16<1, 1>(c, RowMajor<bf16>{sK, C::LDK}, RowMajor<bf16>{sK, C::LDK}, 16 * bi, 16 * bj, 0, DK);
    else
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
    if constexpr (BF) {
      // a C-layout tile is its own B operand for the k = 16 MFMA
      const int rA = l & 15, kq = 4 * (l >> 4);
      f32x4 T[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) T[m] = zero4();
#pragma unroll
      for (int m = 0; m < 3; ++m)
        if (m == jc) {
#pragma unroll
          for (int i = 0; i < 4; ++i) T[m][i] = sTau[(16 * m + kq + i) * C::LDC + 16 * m + rA];
        }
#pragma unroll
      for (int i = 1; i < 4; ++i) {
        if (i <= jc) continue;
        f32x4 X = zero4();
#pragma unroll
        for (int m = 0; m < 3; ++m) {
          if (m < jc || m >= i) continue;
          const f32x4 a = *reinterpret_cast<const f32x4 *>(sA + (16 * i + rA) * C::LDC + 16 * m + kq);
          X = mma16_split3(a, T[m], X);
        }
        const f32x4 d = *reinterpret_cast<const f32x4 *>(sTau + (16 * i + rA) * C::LDC + 16 * i + kq);
        f32x4 Y = mma16_split3(d, X, zero4());
#pragma unroll
        for (int q = 0; q < 4; ++q) Y[q] = -Y[q];
        T[i] = Y;
#pragma unroll
        for (int q = 0; q < 4; ++q) sTau[(16 * i + kq + q) * C::LDC + 16 * jc + rA] = Y[q];
      }
    } else {
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

  // ---- 5. (bf16 inputs) Tau as split-bf16 MFMA A fragments ----
  if constexpr (BF) {
    lds_barrier();
    bf16 *outh = reinterpret_cast<bf16 *>(out), *outl = outh + kTauFragPlane;
    for (int s = tid; s < kTauFrags * 64; s += PNT) {
      const int f = s >> 6, ln = s & 63;
      const int bt = f < 2 ? f : (f - 2) / 2 + 2;
      const int m = f < 2 ? 0 : (f - 2) % 2;
      const int row = 16 * bt + (ln & 15);
      float x[8];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int c0 = 32 * m + 16 * half + 4 * (ln >> 4);
        const bool live = (c0 >> 4) <= bt;  // blocks right of the diagonal are zero
        const f32x4 v = live ? *reinterpret_cast<const f32x4 *>(sTau + row * C::LDC + c0) : zero4();
#pragma unroll
        for (int e = 0; e < 4; ++e) x[4 * half + e] = v[e];
      }
      // fold beta into the columns: Tau R = (Tau diag(beta)) (V - e^g Y)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const f32x4 bc = *reinterpret_cast<const f32x4 *>(sBeta + 32 * m + 16 * half + 4 * (ln >> 4));
#pragma unroll
        for (int e = 0; e < 4; ++e) x[4 * half + e] *= bc[e];
      }
      bf16x8 hi, lo;
      split8(x, hi, lo);
      *reinterpret_cast<bf16x8 *>(outh + 8 * s) = hi;
      *reinterpret_cast<bf16x8 *>(outl + 8 * s) = lo;
    }
    // K^T fragments of the state update S^T += K^T D': fragment (d, mm), lane
    // (q, g) holds K[32 mm + 4 g + e (+16)][32 (d >> 1) + 8 (q >> 2) + 4 (d & 1) + (q & 3)],
    // e < 4: the row order of the recurrence kernel's S^T blocks and the
    // token order of its paired C-layout right-hand sides
    bf16 *kt = reinterpret_cast<bf16 *>(reinterpret_cast<char *>(out) + kRecKtOffsetBytes);
    for (int s = tid; s < 2 * (DK / 16) * 64; s += PNT) {
      const int j = s >> 6, ln = s & 63;
      const int d = j >> 1, mm = j & 1, q = ln & 15, g = ln >> 4;
      const int col = 32 * (d >> 1) + 8 * (q >> 2) + 4 * (d & 1) + (q & 3);
      bf16x8 v;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = sK[(32 * mm + 4 * g + (e & 3) + 16 * (e >> 2)) * C::LDK + col];
      *reinterpret_cast<bf16x8 *>(kt + 8 * s) = v;
    }
  }
}

template <class Tin, int DK>
hipError_t launch_p(const PrepLaunch &p, hipStream_t stream) {
  if (p.n_slots <= 0) return hipSuccess;
  hipLaunchKernelGGL((prep_kernel<Tin, DK>), dim3((unsigned)p.n_slots, (unsigned)p.H), dim3(PNT), 0, stream, p);
  return hipGetLastError();
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
