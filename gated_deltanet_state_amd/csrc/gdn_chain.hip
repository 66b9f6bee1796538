// gdn_chain.hip -- chunkwise-parallel Gated DeltaNet recurrence for gfx950.
//
// The recurrence (page "Tail-Replay: Escaping the Curse of Linear Attention
// in Prefix Caching for Hybrid LLMs", section 2 Eq. (1); state S dv x dk):
//     S_t = S_{t-1} alpha_t (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,  o_t = S_t q_t.
// Unrolled over a chunk of L <= 64 tokens with cumulative log-gates
// g_r = sum_{s<=r} log alpha_s it becomes (derivation: substitute the state
// before each token into the delta-rule correction of the next one):
//     A    = strictly lower part of  beta_r exp(g_r - g_s) (k_r . k_s)
//     Tau  = (I + A)^{-1}                         (unit lower triangular)
//     W    = Tau diag(beta e^g) K,   U = Tau diag(beta) V
//     D    = U - W S^T                            (per-token corrections)
//     O    = diag(e^g) Q S^T + (M o Q K^T) D,     M_rs = e^{g_r - g_s}, s <= r
//     S   <- e^{g_L} S + (diag(e^{g_L - g}) D)^T K
// Rows of S evolve independently, so a workgroup owns 16 rows of one
// (sequence, head) state and walks its chunks in order; the dv-independent
// factors (A, Tau, W, P = M o QK^T) are rebuilt by every row tile.
//
// The same kernel builds the affine chunk operator of the page "LinearKV:
// One Cached State Suffices for Position-Independent Caching in Hybrid
// LLMs" (affine chunk operator paragraph): rows of the transition product
// T_C are the rows of a "state" that starts as the identity and receives no
// value input (T_C = e^{g_L} I - W^T diag(e^{g_L-g}) K per 64-token step).
//
// Precision (bf16 inputs, fp32 state): every MFMA operand that is an input
// (K, Q, V) is exact in bf16; fp32-derived operands are split into bf16
// hi + lo where their rounding would show in the result (see mma_bf16).
// fp32 inputs use the fp32 MFMA throughout.
#include "gdn_device.h"
#include "gdn_internal.h"

#include <type_traits>

namespace gdn {

namespace {

constexpr int CH = 64;      // tokens per chunk
constexpr int RT = 16;      // state rows per workgroup
constexpr int NW = 8;       // waves per workgroup
constexpr int NT = NW * 64; // threads per workgroup

template <class Tin, int DK>
struct Smem {
  static constexpr bool BF = std::is_same<Tin, bf16>::value;
  // leading dimensions (elements); bf16 paths need 16-byte aligned rows,
  // fp32 paths read single elements and use odd strides against bank conflicts
  static constexpr int LDK = BF ? DK + 8 : DK + 1;   // sK, sQ  [CH][LDK]   Tin
  static constexpr int LDKT = CH + 8;                // sKt     [DK][LDKT]  bf16 only
  static constexpr int LDVT = BF ? CH + 8 : CH + 1;  // sVt     [RT][LDVT]  Tin
  static constexpr int LDC = BF ? CH + 4 : CH + 1;   // sA(=sP), sTau [CH][LDC] fp32
  static constexpr int LDW = BF ? DK + 4 : DK + 1;   // sW [CH][LDW], sS [RT][LDW] fp32
  static constexpr int LDD = LDC;                    // sD, sDd [RT][LDD] fp32
  static constexpr int LDX = 17;                     // solve scratch [3][16][LDX]

  static constexpr size_t al(size_t x) { return (x + 15) & ~size_t(15); }
  static constexpr size_t oK = 0;
  static constexpr size_t oQ = oK + al(sizeof(Tin) * CH * LDK);
  static constexpr size_t oKt = oQ + al(sizeof(Tin) * CH * LDK);
  static constexpr size_t oVt = oKt + (BF ? al(sizeof(bf16) * DK * LDKT) : 0);
  static constexpr size_t oA = oVt + al(sizeof(Tin) * RT * LDVT);
  static constexpr size_t oTau = oA + al(4 * CH * LDC);
  static constexpr size_t oW = oTau + al(4 * CH * LDC);
  static constexpr size_t oS = oW + al(4 * CH * LDW);
  static constexpr size_t oD = oS + al(4 * RT * LDW);
  static constexpr size_t oDd = oD + al(4 * RT * LDD);
  static constexpr size_t oGate = oDd + al(4 * RT * LDD);  // 8 arrays of CH floats
  static constexpr size_t TOTAL = oGate + al(4 * 8 * CH);
  static_assert(3 * 16 * LDX * 4 <= 2 * 4 * RT * LDD, "solve scratch must fit in sD/sDd");
  static_assert(TOTAL <= 160 * 1024, "LDS budget");
};

__device__ __forceinline__ float ld_in(const float *p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ld_in(const bf16 *p, int64_t i) { return (float)p[i]; }

// C += A * B over k in [k0, k1); fp32 policy ignores the pass counts.
template <bool BF, int PA, int PB, class OA, class OB>
__device__ __forceinline__ void mma(f32x4 &c, const OA &a, const OB &b, int m0, int n0, int k0, int k1) {
  if constexpr (BF)
    mma_bf16<PA, PB>(c, a, b, m0, n0, k0, k1);
  else
    mma_f32(c, a, b, m0, n0, k0, k1);
}

// k range [0, kend) covering the lower-triangular blocks up to block b
// (inclusive): 16 (b + 1) rounded up to the MFMA k step.
template <bool BF>
__device__ __forceinline__ int tri_kend(int b) {
  return BF ? 32 * ((b + 2) >> 1) : 16 * (b + 1);
}

template <class Tin, int DK, bool WANT_O, bool PRECISE_S>
__global__ void __launch_bounds__(NT) chain_kernel(ChainLaunch p, int n_items) {
  using L = Smem<Tin, DK>;
  constexpr bool BF = L::BF;
  __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
  Tin *sK = reinterpret_cast<Tin *>(smem + L::oK);
  Tin *sQ = reinterpret_cast<Tin *>(smem + L::oQ);
  bf16 *sKt = reinterpret_cast<bf16 *>(smem + L::oKt);
  Tin *sVt = reinterpret_cast<Tin *>(smem + L::oVt);
  float *sA = reinterpret_cast<float *>(smem + L::oA);  // A, later P
  float *sTau = reinterpret_cast<float *>(smem + L::oTau);
  float *sW = reinterpret_cast<float *>(smem + L::oW);
  float *sS = reinterpret_cast<float *>(smem + L::oS);
  float *sD = reinterpret_cast<float *>(smem + L::oD);
  float *sDd = reinterpret_cast<float *>(smem + L::oDd);
  float *sX = sD;  // solve scratch (sD / sDd are idle during the solve)
  float *sGate = reinterpret_cast<float *>(smem + L::oGate);
  float *sG = sGate;               // g_r
  float *sBeta = sGate + CH;       // beta_r (0 past the chunk end)
  float *sBG = sGate + 2 * CH;     // beta_r e^{g_r}
  float *sDec = sGate + 3 * CH;    // e^{g_L - g_r} (0 past the end)
  float *sGam = sGate + 4 * CH;    // e^{g_r}
  float *sRawA = sGate + 5 * CH;   // alpha as loaded
  float *sRawB = sGate + 6 * CH;   // beta as loaded
  float *sScal = sGate + 7 * CH;   // [0] = e^{g_L}

  // ---- work item: XCD-aware order (block b runs on XCD b % 8; each XCD
  // takes a contiguous range of items so the row tiles of one head share
  // that XCD's L2) ----
  const int per = (int)(gridDim.x >> 3);
  const int item = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
  if (item >= n_items) return;
  const int tiles = p.tiles_T + p.tiles_S;
  const int unit = item / tiles, tile = item % tiles;
  const int n = unit / p.H, h = unit % p.H;
  const bool is_T = tile < p.tiles_T;
  const int row0 = is_T ? 16 * tile : 16 * (tile - p.tiles_T);
  const int H = p.H, DV = p.dv;

  const int tid = threadIdx.x, w = wave_id(), l = lane_id();
  const Tin *gq = reinterpret_cast<const Tin *>(p.q);
  const Tin *gk = reinterpret_cast<const Tin *>(p.k);
  const Tin *gv = reinterpret_cast<const Tin *>(p.v);
  const Tin *ga = reinterpret_cast<const Tin *>(p.alpha);
  const Tin *gb = reinterpret_cast<const Tin *>(p.beta);

  // ---- state tile in registers: wave w owns columns [16w, 16w + 16) ----
  constexpr int NST = DK / 16;  // state column tiles (4 or 8 <= NW)
  const bool owns = w < NST;
  f32x4 sacc = zero4();
  if (owns) {
    const int col = 16 * w + (l & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = row0 + 4 * (l >> 4) + i;
      if (is_T) {
        sacc[i] = (r == col) ? 1.f : 0.f;
      } else if (p.S0) {
        sacc[i] = p.S0[(((int64_t)n * H + h) * DV + r) * DK + col];
      }
    }
  }

  const int tbeg = p.cu[n], tend = p.cu[n + 1];
  for (int t0 = tbeg; t0 < tend; t0 += CH) {
    const int Lc = min(CH, tend - t0);

    // ---------------- phase 1: loads, state to LDS ----------------
    if (owns) store_tile(sS, L::LDW, 0, 16 * w, sacc);
    {
      constexpr int VEC = 16 / sizeof(Tin);  // elements per 16-byte load
      constexpr int SEGS = DK / VEC;
      for (int s = tid; s < CH * SEGS; s += NT) {
        const int r = s / SEGS, seg = s % SEGS;
        const int64_t goff = ((int64_t)(t0 + r) * H + h) * DK + seg * VEC;
        f32x4 kraw = zero4(), qraw = zero4();
        if (r < Lc) {
          kraw = *reinterpret_cast<const f32x4 *>(gk + goff);
          if (WANT_O) qraw = *reinterpret_cast<const f32x4 *>(gq + goff);
        }
        const Tin *kv = reinterpret_cast<const Tin *>(&kraw);
        const Tin *qv = reinterpret_cast<const Tin *>(&qraw);
        if constexpr (BF) {
          *reinterpret_cast<f32x4 *>(sK + r * L::LDK + seg * VEC) = kraw;
          if (WANT_O) *reinterpret_cast<f32x4 *>(sQ + r * L::LDK + seg * VEC) = qraw;
#pragma unroll
          for (int e = 0; e < VEC; ++e) sKt[(seg * VEC + e) * L::LDKT + r] = kv[e];
        } else {
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            sK[r * L::LDK + seg * VEC + e] = kv[e];
            if (WANT_O) sQ[r * L::LDK + seg * VEC + e] = qv[e];
          }
        }
      }
      if (!is_T) {
        constexpr int VSEGS = RT / VEC;
        for (int s = tid; s < CH * VSEGS; s += NT) {
          const int r = s / VSEGS, seg = s % VSEGS;
          f32x4 vraw = zero4();
          if (r < Lc)
            vraw = *reinterpret_cast<const f32x4 *>(gv + ((int64_t)(t0 + r) * H + h) * DV + row0 + seg * VEC);
          const Tin *vv = reinterpret_cast<const Tin *>(&vraw);
#pragma unroll
          for (int e = 0; e < VEC; ++e) sVt[(seg * VEC + e) * L::LDVT + r] = vv[e];
        }
      }
      if (tid < CH) {
        float a = 1.f, b = 0.f;
        if (tid < Lc) {
          const int64_t gi = (int64_t)(t0 + tid) * H + h;
          a = ld_in(ga, gi);
          b = ld_in(gb, gi);
        }
        sRawA[tid] = a;
        sRawB[tid] = b;
      }
    }
    __syncthreads();

    // ---------------- phase 2: gates; clear Tau's upper blocks ----------------
    if (w == 0) {
      const int r = l;
      float g = (r < Lc) ? logf(sRawA[r]) : 0.f;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(g, off);
        if (r >= off) g += y;
      }
      const float gL = __shfl(g, Lc - 1);
      const float bet = sRawB[r];
      const float gam = expf(g);
      sG[r] = g;
      sBeta[r] = bet;
      sBG[r] = bet * gam;
      sGam[r] = gam;
      sDec[r] = (r < Lc) ? expf(gL - g) : 0.f;
      if (r == 0) sScal[0] = expf(gL);
    } else {
      // upper blocks (bi < bj) of Tau are read as zeros by the k-steps
      for (int e = tid - 64; e < 6 * 256; e += NT - 64) {
        const int blk = e >> 8, rr = (e >> 4) & 15, cc = e & 15;
        const int bi = blk < 3 ? 0 : (blk < 5 ? 1 : 2);
        const int bj = blk < 3 ? blk + 1 : (blk < 5 ? blk - 1 : 3);
        sTau[(16 * bi + rr) * L::LDC + 16 * bj + cc] = 0.f;
      }
    }
    __syncthreads();

    // ---------------- phase 3: A = strictly-lower beta_r e^{g_r-g_s} K K^T ----------------
    for (int t = w; t < 10; t += NW) {
      const int bi = t < 1 ? 0 : (t < 3 ? 1 : (t < 6 ? 2 : 3));
      const int bj = t - (bi * (bi + 1)) / 2;
      f32x4 c = zero4();
      if constexpr (BF)
        mma<BF, 1, 1>(c, RowMajor<bf16>{(const bf16 *)sK, L::LDK}, RowMajor<bf16>{(const bf16 *)sK, L::LDK},
                      16 * bi, 16 * bj, 0, DK);
      else
        mma<BF, 1, 1>(c, RowMajor<float>{(const float *)sK, L::LDK}, RowMajor<float>{(const float *)sK, L::LDK},
                      16 * bi, 16 * bj, 0, DK);
      const int col = 16 * bj + (l & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * bi + 4 * (l >> 4) + i;
        sA[row * L::LDC + col] = (col < row) ? sBeta[row] * expf(sG[row] - sG[col]) * c[i] : 0.f;
      }
    }
    __syncthreads();

    // ---------------- phase 4: Tau = (I + A)^{-1} ----------------
    // diagonal 16x16 blocks by forward substitution, one column per lane
    if (w == 0) {
      const int b = l >> 4, j = l & 15;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float acc = (r == j) ? 1.f : 0.f;
        const float *arow = sA + (16 * b + r) * L::LDC + 16 * b;
#pragma unroll
        for (int s = 0; s < r; ++s) acc -= arow[s] * x[s];
        x[r] = acc;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sTau[(16 * b + r) * L::LDC + 16 * b + j] = x[r];
    }
    __syncthreads();
    // off-diagonal blocks, by distance from the diagonal:
    //   Tau_ij = -Tau_ii * sum_{m=j}^{i-1} A_im Tau_mj
    for (int d = 1; d < 4; ++d) {
      const int nb = 4 - d;
      if (w < nb) {
        const int i = d + w, j = w;
        f32x4 c = zero4();
        mma_f32(c, RowMajor<float>{sA + 16 * i * L::LDC, L::LDC}, ColMajor<float>{sTau + 16 * j, L::LDC}, 0, 0,
                16 * j, 16 * i);
        store_tile(sX + w * 16 * L::LDX, L::LDX, 0, 0, c);
      }
      __syncthreads();
      if (w < nb) {
        const int i = d + w, j = w;
        f32x4 c = zero4();
        mma_f32(c, RowMajor<float>{sTau + 16 * i * L::LDC + 16 * i, L::LDC},
                ColMajor<float>{sX + w * 16 * L::LDX, L::LDX}, 0, 0, 0, 16);
        const int col = 16 * j + (l & 15);
#pragma unroll
        for (int q = 0; q < 4; ++q) sTau[(16 * i + 4 * (l >> 4) + q) * L::LDC + col] = -c[q];
      }
      __syncthreads();
    }

    // ---------------- phase 5: W = Tau diag(beta e^g) K ; P = M o Q K^T ----------------
    {
      constexpr int NWT = 4 * (DK / 16);
      constexpr int NPT = WANT_O ? 10 : 0;
      for (int t = w; t < NWT + NPT; t += NW) {
        f32x4 c = zero4();
        if (t < NWT) {
          const int rb = t / (DK / 16), cb = t % (DK / 16);
          const RowScaled ta{sTau + 16 * rb * L::LDC, L::LDC, sBG};
          if constexpr (BF)
            mma<BF, 2, 1>(c, ta, RowMajor<bf16>{sKt, L::LDKT}, 0, 16 * cb, 0, tri_kend<BF>(rb));
          else
            mma<BF, 2, 1>(c, ta, ColMajor<float>{(const float *)sK, L::LDK}, 0, 16 * cb, 0, tri_kend<BF>(rb));
          store_tile(sW, L::LDW, 16 * rb, 16 * cb, c);
        } else {
          const int tt = t - NWT;
          const int bi = tt < 1 ? 0 : (tt < 3 ? 1 : (tt < 6 ? 2 : 3));
          const int bj = tt - (bi * (bi + 1)) / 2;
          mma<BF, 1, 1>(c, RowMajor<Tin>{sQ, L::LDK}, RowMajor<Tin>{sK, L::LDK}, 16 * bi, 16 * bj, 0, DK);
          const int col = 16 * bj + (l & 15);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = 16 * bi + 4 * (l >> 4) + i;
            sA[row * L::LDC + col] = (col <= row) ? expf(sG[row] - sG[col]) * c[i] : 0.f;
          }
        }
      }
      if (WANT_O) {
        // upper blocks of P are read as zeros by the PD product
        for (int e = tid; e < 6 * 256; e += NT) {
          const int blk = e >> 8, rr = (e >> 4) & 15, cc = e & 15;
          const int bi = blk < 3 ? 0 : (blk < 5 ? 1 : 2);
          const int bj = blk < 3 ? blk + 1 : (blk < 5 ? blk - 1 : 3);
          sA[(16 * bi + rr) * L::LDC + 16 * bj + cc] = 0.f;
        }
      }
    }
    __syncthreads();

    // ---------------- phase 6: D^T = U^T - S W^T ; first half of O^T ----------------
    f32x4 oacc = zero4();
    if (w < 4) {
      const int cb = w;
      f32x4 c = zero4();
      if (!is_T) {
        const RowScaled tb{sTau, L::LDC, sBeta};
        mma<BF, 1, 2>(c, RowMajor<Tin>{sVt, L::LDVT}, tb, 0, 16 * cb, 0, tri_kend<BF>(cb));
      }
      mma<BF, PRECISE_S ? 2 : 1, PRECISE_S ? 2 : 1>(c, RowNeg{sS, L::LDW}, RowMajor<float>{sW, L::LDW}, 0,
                                                    16 * cb, 0, DK);
      store_tile(sD, L::LDD, 0, 16 * cb, c);
      const float dec = sDec[16 * cb + (l & 15)];
      f32x4 cd;
#pragma unroll
      for (int i = 0; i < 4; ++i) cd[i] = c[i] * dec;
      store_tile(sDd, L::LDD, 0, 16 * cb, cd);
    } else if (WANT_O) {
      const int cb = w - 4;
      mma<BF, 1, 1>(oacc, RowMajor<float>{sS, L::LDW}, RowMajor<Tin>{sQ, L::LDK}, 0, 16 * cb, 0, DK);
      const float gam = sGam[16 * cb + (l & 15)];
#pragma unroll
      for (int i = 0; i < 4; ++i) oacc[i] *= gam;
    }
    __syncthreads();

    // ---------------- phase 7: O^T += D^T P^T, store o ; S update ----------------
    if (WANT_O && w >= 4) {
      const int cb = w - 4;
      mma<BF, 2, 2>(oacc, RowMajor<float>{sD, L::LDD}, RowMajor<float>{sA, L::LDC}, 0, 16 * cb, 0,
                    tri_kend<BF>(cb));
      const int r = 16 * cb + (l & 15);
      if (r < Lc) {
        const int64_t base = ((int64_t)(t0 + r) * H + h) * DV + row0 + 4 * (l >> 4);
        if (p.o_bf16) {
          bf16x4 ov;
#pragma unroll
          for (int i = 0; i < 4; ++i) ov[i] = (bf16)oacc[i];
          *reinterpret_cast<bf16x4 *>(reinterpret_cast<bf16 *>(p.o) + base) = ov;
        } else {
          *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(p.o) + base) = oacc;
        }
      }
    }
    if (owns) {
      const float gl = sScal[0];
#pragma unroll
      for (int i = 0; i < 4; ++i) sacc[i] *= gl;
      if constexpr (BF)
        mma<BF, 2, 1>(sacc, RowMajor<float>{sDd, L::LDD}, RowMajor<bf16>{sKt, L::LDKT}, 0, 16 * w, 0, CH);
      else
        mma<BF, 2, 1>(sacc, RowMajor<float>{sDd, L::LDD}, ColMajor<float>{(const float *)sK, L::LDK}, 0, 16 * w,
                      0, CH);
    }
    __syncthreads();
  }

  // ---------------- epilogue: final rows ----------------
  if (owns) {
    float *out = is_T ? p.T_out : p.S_out;
    const int nrows = is_T ? DK : DV;
    const int col = 16 * w + (l & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = row0 + 4 * (l >> 4) + i;
      out[(((int64_t)n * H + h) * nrows + r) * DK + col] = sacc[i];
    }
  }
}

template <class Tin, int DK, bool WANT_O, bool PRECISE_S>
hipError_t launch_t(const ChainLaunch &p, hipStream_t stream) {
  const int64_t items = (int64_t)p.n_seqs * p.H * (p.tiles_T + p.tiles_S);
  if (items <= 0) return hipSuccess;
  const int64_t grid = (items + 7) / 8 * 8;
  hipLaunchKernelGGL((chain_kernel<Tin, DK, WANT_O, PRECISE_S>), dim3((unsigned)grid), dim3(NT), 0, stream, p,
                     (int)items);
  return hipGetLastError();
}

template <class Tin, int DK>
hipError_t launch_dk(const ChainLaunch &p, hipStream_t stream) {
  const bool want_o = p.o != nullptr;
  if (p.precise_state) {
    return want_o ? launch_t<Tin, DK, true, true>(p, stream) : launch_t<Tin, DK, false, true>(p, stream);
  }
  return want_o ? launch_t<Tin, DK, true, false>(p, stream) : launch_t<Tin, DK, false, false>(p, stream);
}

}  // namespace

hipError_t launch_chain(const ChainLaunch &p, hipStream_t stream) {
  if (p.in_bf16) {
    if (p.dk == 64) return launch_dk<bf16, 64>(p, stream);
    if (p.dk == 128) return launch_dk<bf16, 128>(p, stream);
  } else {
    if (p.dk == 64) return launch_dk<float, 64>(p, stream);
    if (p.dk == 128) return launch_dk<float, 128>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
