// gdn_prep_bf16.hip -- per-chunk UT transform for bf16 inputs on gfx950.
//
// For a chunk of L <= 64 tokens (page "Tail-Replay: Escaping the Curse of
// Linear Attention in Prefix Caching for Hybrid LLMs", section 2 Eq. (1),
// unrolled over the chunk) the per-token delta-rule corrections D satisfy
//     (I + A) D = diag(beta) (V - diag(e^g) K S^T),
//     A = strictly lower part of  beta_r exp(g_r - g_s) (k_r . k_s),
// with g the cumulative log-gate.  A depends only on keys and gates, so
// Tau = (I + A)^{-1} is built here once per (chunk, head), fully in
// parallel, for every row tile of the recurrence kernel.
//
// One wave per (chunk slot, head), no workgroup barriers (a workgroup is a
// single wave with its own LDS):
//   1. keys to LDS by load-to-LDS DMA, in MFMA A-fragment order; cumulative
//      log-gates by a wave-wide scan
//   2. the 10 lower 16 x 16 blocks of A on bf16 MFMA (keys are exact in
//      bf16), ten independent accumulators
//   3. the four diagonal blocks inverted at once by forward substitution:
//      lane (b, c) = (l >> 4, l & 15) computes column c of (I + A_bb)^{-1}
//   4. off-diagonal blocks Tau_ij = -Tau_ii sum_{m=j}^{i-1} A_im Tau_mj on
//      split-bf16 k = 16 MFMAs, in three dependency levels
//   5. Tau diag(beta) as split-bf16 A fragments of the recurrence kernel's
//      k = 32 products (record layout of gdn_internal.h).
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

__device__ __forceinline__ int blk(int i, int j) { return i * (i + 1) / 2 + j; }  // i >= j

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

// x (4 fp32 in A layout) times y (4 fp32 in B layout), k = 16, as split bf16
// with the three partial products in separate accumulators (no product
// waits on the one before it).
struct Acc3 {
  f32x4 a, b, c;
};
__device__ __forceinline__ void acc_split3(Acc3 &acc, const f32x4 &x, const f32x4 &y) {
  bf16x4 xh, xl, yh, yl;
  split4(x, xh, xl);
  split4(y, yh, yl);
  acc.a = mfma_bf16_k16(xh, yh, acc.a);
  acc.b = mfma_bf16_k16(xh, yl, acc.b);
  acc.c = mfma_bf16_k16(xl, yh, acc.c);
}
__device__ __forceinline__ Acc3 acc3_zero() { return Acc3{zero4(), zero4(), zero4()}; }
__device__ __forceinline__ f32x4 acc3_sum(const Acc3 &a) { return a.a + a.b + a.c; }

template <int DK>
__global__ void __launch_bounds__(64) prep_bf16_kernel(PrepLaunch p) {
  constexpr int NKS = DK / 32;
  constexpr int NKA = 4 * NKS;                     // 1 KiB key fragments (bt, m)
  // sK: keys, then (once the keys are no longer read) the row-major Tau
  // blocks (10 KiB) and the transposed diagonal blocks (4 KiB)
  __shared__ __attribute__((aligned(16))) char sK[NKA * 1024 > 14336 ? NKA * 1024 : 14336];
  __shared__ __attribute__((aligned(16))) float sA[10 * 256];  // A blocks, 16 x 16 row-major
  __shared__ __attribute__((aligned(16))) float sG[64], sB[64];
  float *sT = reinterpret_cast<float *>(sK);       // Tau blocks, row-major, block blk(i, j)
  float *sTT = sT + 10 * 256;                      // Tau_bb transposed, block b

  const int64_t slot = blockIdx.x;
  const int h = blockIdx.y, H = p.H;
  const int n = find_seq_b(p.cu, p.n_seqs, slot);
  const int tbeg = p.cu[n], len = p.cu[n + 1] - tbeg;
  const int64_t j = slot - ((int64_t)(tbeg / kChunk) + n);
  if (j < 0 || j * kChunk >= len) return;  // slot past the end of its sequence
  const int t0 = tbeg + (int)j * kChunk;
  const int Lc = min(kChunk, len - (int)j * kChunk);
  const int l = lane_id(), g4 = l >> 4, jl = l & 15;
  char *rec = reinterpret_cast<char *>(p.tau + (slot * H + h) * (int64_t)kRecFloats);

  // ---- 1. keys (rows past the chunk: copies of its last row; they meet
  // beta = 0 below) and gates ----
  const bf16 *gk = reinterpret_cast<const bf16 *>(p.k);
#pragma unroll
  for (int f = 0; f < NKA; ++f) {
    const int bt = f / NKS, m = f % NKS;
    const int r = min(16 * bt + jl, Lc - 1);
    dma16_global(gk + ((int64_t)(t0 + r) * H + h) * DK + 32 * m + 8 * g4, (lds_void *)(sK + f * 1024));
  }
  {
    float g = 0.f, b = 0.f;
    if (l < Lc) {
      const int64_t gi = (int64_t)(t0 + l) * H + h;
      g = logf((float)reinterpret_cast<const bf16 *>(p.alpha)[gi]);
      b = (float)reinterpret_cast<const bf16 *>(p.beta)[gi];
    }
    sG[l] = wave_inclusive_scan(g);
    sB[l] = b;
  }
  wait_vmem();
  wave_lds_fence();

  // ---- 2. A = strictly-lower beta_r e^{g_r - g_s} K K^T, 10 blocks ----
  {
    f32x4 acc[10];
#pragma unroll
    for (int t = 0; t < 10; ++t) acc[t] = zero4();
#pragma unroll
    for (int m = 0; m < NKS; ++m) {
      bf16x8 kf[4];
#pragma unroll
      for (int bt = 0; bt < 4; ++bt) kf[bt] = *reinterpret_cast<const bf16x8 *>(sK + (bt * NKS + m) * 1024 + 16 * l);
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
#pragma unroll
        for (int bj = 0; bj <= bi; ++bj) acc[blk(bi, bj)] = mfma_bf16(kf[bi], kf[bj], acc[blk(bi, bj)]);
    }
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
      for (int bj = 0; bj <= bi; ++bj) {
        const int col = 16 * bj + jl, row0 = 16 * bi + 4 * g4;
        const float gc = sG[col];
        const f32x4 gr = *reinterpret_cast<const f32x4 *>(sG + row0);
        const f32x4 br = *reinterpret_cast<const f32x4 *>(sB + row0);
        float *dst = sA + blk(bi, bj) * 256 + 4 * g4 * 16 + jl;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          dst[e * 16] = (col < row0 + e) ? br[e] * __expf(gr[e] - gc) * acc[blk(bi, bj)][e] : 0.f;
      }
  }
  // the key buffer is reused for Tau from here on (this wave's key reads
  // above were consumed by the products before these writes)
  wave_lds_fence();

  // ---- 3. diagonal blocks: lane (b, c) solves (I + A_bb) x = e_c ----
  {
    const int b = g4, c = jl;
    const float *ab = sA + blk(b, b) * 256;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float acc0 = (r == c) ? 1.f : 0.f, acc1 = 0.f;
#pragma unroll
      for (int s4 = 0; s4 < (r + 3) / 4; ++s4) {
        const f32x4 ar = *reinterpret_cast<const f32x4 *>(ab + r * 16 + 4 * s4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int s = 4 * s4 + e;
          if (s < r) {
            if (e & 1)
              acc1 -= ar[e] * x[s];
            else
              acc0 -= ar[e] * x[s];
          }
        }
      }
      x[r] = acc0 + acc1;
    }
    float *tr = sT + blk(b, b) * 256 + c;           // row-major: Tau_bb[r][c]
#pragma unroll
    for (int r = 0; r < 16; ++r) tr[r * 16] = x[r];
    float *tt = sTT + b * 256 + c * 16;             // transposed: row c holds column c
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) *reinterpret_cast<f32x4 *>(tt + 4 * r4) = f32x4{x[4 * r4], x[4 * r4 + 1], x[4 * r4 + 2], x[4 * r4 + 3]};
  }
  wave_lds_fence();

  // ---- 4. off-diagonal blocks (C layout: lane column jl, rows 4 g4 + e) ----
  {
    // operands: A_im and Tau_ii in A layout (row jl, columns 4 g4 ..), Tau_jj
    // in B layout (column jl, rows 4 g4 ..) from the transposed copy
    auto Aop = [&](int i, int m) { return *reinterpret_cast<const f32x4 *>(sA + blk(i, m) * 256 + jl * 16 + 4 * g4); };
    auto Tii = [&](int i) { return *reinterpret_cast<const f32x4 *>(sT + blk(i, i) * 256 + jl * 16 + 4 * g4); };
    auto Tjj = [&](int i) { return *reinterpret_cast<const f32x4 *>(sTT + i * 256 + jl * 16 + 4 * g4); };
    auto neg_tau = [&](int i, const Acc3 &x) {       // -Tau_ii X
      Acc3 y = acc3_zero();
      acc_split3(y, Tii(i), acc3_sum(x));
      return -acc3_sum(y);
    };
    const f32x4 T00 = Tjj(0), T11 = Tjj(1), T22 = Tjj(2);
    // level 1: Tau_10, Tau_21, Tau_32
    Acc3 x10 = acc3_zero(), x21 = acc3_zero(), x32 = acc3_zero();
    acc_split3(x10, Aop(1, 0), T00);
    acc_split3(x21, Aop(2, 1), T11);
    acc_split3(x32, Aop(3, 2), T22);
    const f32x4 T10 = neg_tau(1, x10), T21 = neg_tau(2, x21), T32 = neg_tau(3, x32);
    // level 2: Tau_20, Tau_31
    Acc3 x20 = acc3_zero(), x31 = acc3_zero();
    acc_split3(x20, Aop(2, 0), T00);
    acc_split3(x31, Aop(3, 1), T11);
    acc_split3(x20, Aop(2, 1), T10);
    acc_split3(x31, Aop(3, 2), T21);
    const f32x4 T20 = neg_tau(2, x20), T31 = neg_tau(3, x31);
    // level 3: Tau_30
    Acc3 x30 = acc3_zero();
    acc_split3(x30, Aop(3, 0), T00);
    acc_split3(x30, Aop(3, 1), T10);
    acc_split3(x30, Aop(3, 2), T20);
    const f32x4 T30 = neg_tau(3, x30);
    auto put = [&](int i, int jb, const f32x4 &t) {
      float *dst = sT + blk(i, jb) * 256 + 4 * g4 * 16 + jl;
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[e * 16] = t[e];
    };
    put(1, 0, T10);
    put(2, 1, T21);
    put(3, 2, T32);
    put(2, 0, T20);
    put(3, 1, T31);
    put(3, 0, T30);
  }
  wave_lds_fence();

  // ---- 5. Tau diag(beta) as split-bf16 A fragments: fragment f = (bt, m),
  // lane (r, g) = (l & 15, l >> 4) holds row 16 bt + r, columns
  // 32 m + 4 g + {0..3} then 32 m + 16 + 4 g + {0..3} ----
  bf16 *outh = reinterpret_cast<bf16 *>(rec), *outl = outh + kTauFragPlane;
#pragma unroll
  for (int f = 0; f < kTauFrags; ++f) {
    const int bt = f < 2 ? f : (f - 2) / 2 + 2;
    const int m = f < 2 ? 0 : (f - 2) % 2;
    float x[8];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int cb = 2 * m + half, c0 = 16 * cb + 4 * g4;
      f32x4 v = zero4();
      if (cb <= bt) v = *reinterpret_cast<const f32x4 *>(sT + blk(bt, cb) * 256 + jl * 16 + 4 * g4);
      const f32x4 bc = *reinterpret_cast<const f32x4 *>(sB + c0);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * half + e] = v[e] * bc[e];
    }
    bf16x8 hi, lo;
    split8(x, hi, lo);
    *reinterpret_cast<bf16x8 *>(outh + 8 * (f * 64 + l)) = hi;
    *reinterpret_cast<bf16x8 *>(outl + 8 * (f * 64 + l)) = lo;
  }
}

template <int DK>
hipError_t launch_pb(const PrepLaunch &p, hipStream_t stream) {
  if (p.n_slots <= 0) return hipSuccess;
  hipLaunchKernelGGL((prep_bf16_kernel<DK>), dim3((unsigned)p.n_slots, (unsigned)p.H), dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prep_bf16(const PrepLaunch &p, hipStream_t stream) {
  if (p.dk == 64) return launch_pb<64>(p, stream);
  if (p.dk == 128) return launch_pb<128>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace gdn
