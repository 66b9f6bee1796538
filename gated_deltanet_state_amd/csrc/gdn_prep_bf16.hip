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
// One workgroup (4 waves) per (chunk slot, head):
//   1. keys to LDS by load-to-LDS DMA, in MFMA A-fragment order; cumulative
//      log-gates by a wave-wide scan
//   2. the 10 lower 16 x 16 blocks of A on bf16 MFMA (keys are exact in bf16)
//   3. wave b inverts diagonal block b by forward substitution, one lane per
//      column, from registers
//   4. off-diagonal blocks Tau_ij = -Tau_ii sum_{m=j}^{i-1} A_im Tau_mj, one
//      block column per wave, on split-bf16 k = 16 MFMAs in registers
//   5. the record of gdn_internal.h: Tau diag(beta) as split-bf16 A fragments
//      of the recurrence kernel's k = 32 products, and K^T as the A fragments
//      of its state update (zero past the chunk), read from the staged keys
//      with the transposing LDS read.
// A and Tau live in LDS as packed 16 x 16 blocks (row pitch 20 floats), which
// keeps the workgroup at about 36 KiB (four per compute unit).
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int PW = 4;
constexpr int PT = PW * 64;
constexpr int LDB = 20;            // row pitch of a packed 16 x 16 block (floats)
constexpr int BLK = 16 * LDB;      // floats per packed block

__device__ __forceinline__ int blk(int i, int j) { return i * (i + 1) / 2 + j; }  // i >= j

template <int DK>
struct PB {
  static constexpr int NKS = DK / 32;
  static constexpr int NKA = 4 * NKS;               // 1 KiB key fragments (bt, m)
  static constexpr size_t oK = 0;
  static constexpr size_t oA = oK + NKA * 1024;
  static constexpr size_t oT = oA + 10 * BLK * 4;
  static constexpr size_t oG = oT + 10 * BLK * 4;
  static constexpr size_t TOTAL = oG + 2 * 64 * 4;
};

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

// Byte offset of key row r, columns c .. c + 3 (c a multiple of 4) in the
// fragment-ordered key buffer: fragment (r >> 4, c >> 5), lane
// (r & 15) + 16 ((c >> 3) & 3), half (c >> 2) & 1.
template <int DK>
__device__ __forceinline__ int kfrag_off(int r, int c) {
  return (((r >> 4) * PB<DK>::NKS + (c >> 5)) * 64 + (r & 15) + 16 * ((c >> 3) & 3)) * 16 + 8 * ((c >> 2) & 1);
}

template <int DK>
__global__ void __launch_bounds__(PT) prep_bf16_kernel(PrepLaunch p) {
  using C = PB<DK>;
  __shared__ __attribute__((aligned(16))) char smem[C::TOTAL];
  char *sK = smem + C::oK;
  float *sA = reinterpret_cast<float *>(smem + C::oA);
  float *sT = reinterpret_cast<float *>(smem + C::oT);
  float *sG = reinterpret_cast<float *>(smem + C::oG);
  float *sB = sG + 64;

  const int64_t slot = blockIdx.x;
  const int h = blockIdx.y, H = p.H;
  const int n = find_seq_b(p.cu, p.n_seqs, slot);
  const int tbeg = p.cu[n], len = p.cu[n + 1] - tbeg;
  const int64_t j = slot - ((int64_t)(tbeg / kChunk) + n);
  if (j < 0 || j * kChunk >= len) return;  // slot past the end of its sequence
  const int t0 = tbeg + (int)j * kChunk;
  const int Lc = min(kChunk, len - (int)j * kChunk);
  const int tid = threadIdx.x, w = wave_id(), l = lane_id();
  const int g4 = l >> 4, jl = l & 15;
  char *rec = reinterpret_cast<char *>(p.tau + (slot * H + h) * (int64_t)kRecFloats);

  // ---- 1. keys (rows past the chunk: copies of its last row; they only meet
  // beta = 0 below) and gates ----
  const bf16 *gk = reinterpret_cast<const bf16 *>(p.k);
  for (int f = w; f < C::NKA; f += PW) {
    const int bt = f / C::NKS, m = f % C::NKS;
    const int r = min(16 * bt + jl, Lc - 1);
    dma16_global(gk + ((int64_t)(t0 + r) * H + h) * DK + 32 * m + 8 * g4, (lds_void *)(sK + f * 1024));
  }
  if (w == 0) {
    float g = 0.f, b = 0.f;
    if (l < Lc) {
      const int64_t gi = (int64_t)(t0 + l) * H + h;
      g = logf((float)reinterpret_cast<const bf16 *>(p.alpha)[gi]);
      b = (float)reinterpret_cast<const bf16 *>(p.beta)[gi];
    }
    g = wave_inclusive_scan(g);
    sG[l] = g;
    sB[l] = b;
  }
  wait_vmem();
  lds_barrier();

  // ---- 2. A = strictly-lower beta_r e^{g_r - g_s} K K^T, packed blocks ----
  for (int t = w; t < 10; t += PW) {
    const int bi = t < 1 ? 0 : (t < 3 ? 1 : (t < 6 ? 2 : 3));
    const int bj = t - (bi * (bi + 1)) / 2;
    bf16x8 a[C::NKS], bb[C::NKS];
#pragma unroll
    for (int m = 0; m < C::NKS; ++m) {
      a[m] = *reinterpret_cast<const bf16x8 *>(sK + (bi * C::NKS + m) * 1024 + 16 * l);
      bb[m] = *reinterpret_cast<const bf16x8 *>(sK + (bj * C::NKS + m) * 1024 + 16 * l);
    }
    f32x4 c = zero4();
#pragma unroll
    for (int m = 0; m < C::NKS; ++m) c = mfma_bf16(a[m], bb[m], c);
    const int col = 16 * bj + jl;
    const float gc = sG[col];
    const int row0 = 16 * bi + 4 * g4;
    const f32x4 gr = *reinterpret_cast<const f32x4 *>(sG + row0);
    const f32x4 br = *reinterpret_cast<const f32x4 *>(sB + row0);
    float *dst = sA + blk(bi, bj) * BLK + 4 * g4 * LDB + jl;
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[e * LDB] = (col < row0 + e) ? br[e] * __expf(gr[e] - gc) * c[e] : 0.f;
  }
  lds_barrier();

  // ---- 3. diagonal blocks: wave b solves (I + A_bb) x = e_jj, lane jj ----
  {
    const int b = w;
    const float *ab = sA + blk(b, b) * BLK;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float acc0 = (r == jl) ? 1.f : 0.f, acc1 = 0.f;
#pragma unroll
      for (int s4 = 0; s4 < (r + 3) / 4; ++s4) {
        const f32x4 ar = *reinterpret_cast<const f32x4 *>(ab + r * LDB + 4 * s4);
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
    if (l < 16) {
      float *tb = sT + blk(b, b) * BLK + jl;
#pragma unroll
      for (int r = 0; r < 16; ++r) tb[r * LDB] = x[r];
    }
  }
  lds_barrier();

  // ---- 4. off-diagonal blocks, block column jc = w (a C-layout 16 x 16 tile
  // is its own B operand for the k = 16 MFMA; A operands read by rows) ----
  if (w < 3) {
    const int jc = w;
    f32x4 T[4], AL[4][3], TD[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      T[i] = zero4();
      TD[i] = zero4();
#pragma unroll
      for (int m = 0; m < 3; ++m) AL[i][m] = zero4();
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) T[jc][e] = sT[blk(jc, jc) * BLK + (4 * g4 + e) * LDB + jl];
#pragma unroll
    for (int i = 1; i < 4; ++i) {
      if (i <= jc) continue;
      TD[i] = *reinterpret_cast<const f32x4 *>(sT + blk(i, i) * BLK + jl * LDB + 4 * g4);
#pragma unroll
      for (int m = 0; m < 3; ++m)
        if (m >= jc && m < i) AL[i][m] = *reinterpret_cast<const f32x4 *>(sA + blk(i, m) * BLK + jl * LDB + 4 * g4);
    }
#pragma unroll
    for (int i = 1; i < 4; ++i) {
      if (i <= jc) continue;
      f32x4 X = zero4();
#pragma unroll
      for (int m = 0; m < 3; ++m)
        if (m >= jc && m < i) X = mma16_split3(AL[i][m], T[m], X);
      f32x4 Y = mma16_split3(TD[i], X, zero4());
#pragma unroll
      for (int e = 0; e < 4; ++e) Y[e] = -Y[e];
      T[i] = Y;
#pragma unroll
      for (int e = 0; e < 4; ++e) sT[blk(i, jc) * BLK + (4 * g4 + e) * LDB + jl] = Y[e];
    }
  }
  lds_barrier();

  // ---- 5a. Tau diag(beta) as split-bf16 A fragments ----
  bf16 *outh = reinterpret_cast<bf16 *>(rec), *outl = outh + kTauFragPlane;
  for (int s = tid; s < kTauFrags * 64; s += PT) {
    const int f = s >> 6, ln = s & 63;
    const int bt = f < 2 ? f : (f - 2) / 2 + 2;
    const int m = f < 2 ? 0 : (f - 2) % 2;
    const int r = ln & 15;
    float x[8];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int c0 = 32 * m + 16 * half + 4 * (ln >> 4);
      const int cb = c0 >> 4;
      f32x4 v = zero4();
      if (cb <= bt) v = *reinterpret_cast<const f32x4 *>(sT + blk(bt, cb) * BLK + r * LDB + (c0 & 15));
      const f32x4 bc = *reinterpret_cast<const f32x4 *>(sB + c0);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * half + e] = v[e] * bc[e];
    }
    bf16x8 hi, lo;
    split8(x, hi, lo);
    *reinterpret_cast<bf16x8 *>(outh + 8 * s) = hi;
    *reinterpret_cast<bf16x8 *>(outl + 8 * s) = lo;
  }

  // ---- 5b. K^T fragments of the state update S^T += K^T D': fragment (d, mm),
  // lane (q, g) holds K[32 mm + 4 g + e (+16)][32 (d >> 1) + 8 (q >> 2) + 4 (d & 1) + (q & 3)]
  // for e < 4, zero past the chunk; each wave handles whole fragments, so the
  // transposing read sees the lanes of one fragment ----
  uint4 *kt = reinterpret_cast<uint4 *>(rec + kRecKtOffsetBytes);
  for (int jf = w; jf < 2 * (DK / 16); jf += PW) {
    const int d = jf >> 1, mm = jf & 1;
    const int row = 32 * mm + 4 * g4 + (jl >> 2);
    const int col = 32 * (d >> 1) + 8 * (jl & 3) + 4 * (d & 1);
    uint2 lo4 = ds_read_tr16(reinterpret_cast<const bf16 *>(sK + kfrag_off<DK>(row, col)));
    uint2 hi4 = ds_read_tr16(reinterpret_cast<const bf16 *>(sK + kfrag_off<DK>(row + 16, col)));
    const int tk = 32 * mm + 4 * g4;  // tokens tk + e and tk + 16 + e
    unsigned m0 = 0, m1 = 0;          // keep masks for the packed bf16 pairs
    auto keep = [&](int t) { return t < Lc ? 0xffffu : 0u; };
    m0 = keep(tk) | (keep(tk + 1) << 16);
    m1 = keep(tk + 2) | (keep(tk + 3) << 16);
    lo4.x &= m0;
    lo4.y &= m1;
    m0 = keep(tk + 16) | (keep(tk + 17) << 16);
    m1 = keep(tk + 18) | (keep(tk + 19) << 16);
    hi4.x &= m0;
    hi4.y &= m1;
    kt[jf * 64 + l] = uint4{lo4.x, lo4.y, hi4.x, hi4.y};
  }
}

template <int DK>
hipError_t launch_pb(const PrepLaunch &p, hipStream_t stream) {
  if (p.n_slots <= 0) return hipSuccess;
  hipLaunchKernelGGL((prep_bf16_kernel<DK>), dim3((unsigned)p.n_slots, (unsigned)p.H), dim3(PT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prep_bf16(const PrepLaunch &p, hipStream_t stream) {
  if (p.dk == 64) return launch_pb<64>(p, stream);
  if (p.dk == 128) return launch_pb<128>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace gdn
