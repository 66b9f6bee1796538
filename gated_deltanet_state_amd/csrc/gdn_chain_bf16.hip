// gdn_chain_bf16.hip -- chunkwise Gated DeltaNet recurrence for bf16 inputs
// on gfx950, one wave per 16 state rows.
//
// The recurrence (page "Tail-Replay: Escaping the Curse of Linear Attention
// in Prefix Caching for Hybrid LLMs", section 2 Eq. (1); state S dv x dk):
//     S_t = S_{t-1} alpha_t (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,  o_t = S_t q_t.
// Over a chunk of L <= 64 tokens with cumulative log-gates g and the
// per-chunk factor Tau = (I + A)^{-1} (built by gdn_prep.hip), for the 16
// state rows j owned by a wave (everything transposed: tokens x rows):
//     Y = K S^T                        (64 x 16)
//     R = diag(beta) (V - diag(e^g) Y)
//     D = Tau R                        (per-token delta-rule corrections)
//     O = diag(e^g) Q S^T + (M o Q K^T) D,   M_rs = e^{g_r - g_s}, s <= r
//     S^T <- e^{g_L} S^T + K^T diag(e^{g_L - g}) D
// A wave keeps S^T (dk x 16) in registers in MFMA C layout.  Each product's
// result is the B operand of the next one (paired C-layout tiles with a
// permuted k order, gdn_device.h), so the whole chain of a chunk runs in the
// wave's registers; only K, K^T, Q, Tau, M o QK^T and the gates are read
// from LDS, shared by the waves of the workgroup (one 16-row tile each).
//
// The same kernel builds the affine chunk operator of the page "LinearKV:
// One Cached State Suffices for Position-Independent Caching in Hybrid
// LLMs" (affine chunk operator paragraph): rows of the transition product
// T_C are rows of a "state" that starts as the identity and gets no value.
//
// Precision: K, Q, V are exact in bf16; S, R, D, Tau and M o QK^T are split
// into bf16 hi + lo where they enter a product (split-bfloat16), which keeps
// every product within a few fp32 ulps.
//
// Per chunk: each wave runs its chain on LDS buffer set (c & 1) while the
// workgroup stages chunk c + 1 into the other set and issues the global
// loads of chunk c + 2; one LDS-only barrier per chunk (two with outputs:
// M o QK^T of the next chunk is built after its keys and queries land).
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int CH = kChunk;
// packed lower block-row matrix (Tau or M o QK^T) as split bf16 planes:
// hi at [0, kPlane), lo at [kPlane, 2 kPlane)
constexpr int kPlane = kTauFloats;

template <int DK, int NWV, bool WANT_O>
struct BCfg {
  static constexpr int NT = NWV * 64;
  static constexpr int LDK = DK + 8;                  // sK, sQ [CH][LDK] bf16
  static constexpr size_t al(size_t x) { return (x + 15) & ~size_t(15); }
  static constexpr size_t KBYTES = al(2 * CH * LDK);
  static constexpr size_t TBYTES = al(2 * kPlane * sizeof(bf16));    // hi + lo planes
  static constexpr size_t GBYTES = al(4 * 5 * CH);
  static constexpr size_t oK = 0;                                    // [2]
  static constexpr size_t oQ = oK + 2 * KBYTES;                      // [2] (o)
  static constexpr size_t oT = oQ + (WANT_O ? 2 * KBYTES : 0);       // [2] Tau planes
  static constexpr size_t oP = oT + 2 * TBYTES;                      // [1] P planes (o)
  static constexpr size_t oG = oP + (WANT_O ? TBYTES : 0);           // [2] gates
  static constexpr size_t TOTAL = oG + 2 * GBYTES;
  static_assert(TOTAL <= 160 * 1024, "LDS budget");
  static constexpr int NSB = DK / 16;   // 16-row blocks of S^T
  static constexpr int NKS = DK / 32;   // k = 32 steps over dk
  // staging: 16-byte segments
  static constexpr int KSEG = DK / 8;
  static constexpr int NKP = (CH * KSEG + NT - 1) / NT;
  static constexpr int TSEG = (int)(2 * kPlane * sizeof(bf16) / 16);  // 16-byte segments of both planes
  static constexpr int NTP = (TSEG + NT - 1) / NT;
};

template <int DK, int NWV, bool WANT_O>
__global__ void __launch_bounds__(NWV * 64) chain_bf16_kernel(ChainLaunch p, int n_items) {
  using C = BCfg<DK, NWV, WANT_O>;
  __shared__ __attribute__((aligned(16))) char smem[C::TOTAL];
  bf16 *sK0 = reinterpret_cast<bf16 *>(smem + C::oK);
  bf16 *sQ0 = reinterpret_cast<bf16 *>(smem + C::oQ);
  bf16 *sT0 = reinterpret_cast<bf16 *>(smem + C::oT);
  bf16 *sP = reinterpret_cast<bf16 *>(smem + C::oP);
  float *sG0 = reinterpret_cast<float *>(smem + C::oG);
  constexpr int KE = C::KBYTES / 2, TE = C::TBYTES / 2, GE = C::GBYTES / 4;

  // ---- work item: XCD-aware order; an item is NWV row tiles of one
  // (sequence, head) ----
  const int per = (int)(gridDim.x >> 3);
  const int item = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
  if (item >= n_items) return;
  const int tiles = p.tiles_T + p.tiles_S;
  const int groups = (tiles + NWV - 1) / NWV;
  const int unit = item / groups, grp = item % groups;
  const int n = unit / p.H, h = unit % p.H;
  const int H = p.H, DV = p.dv;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id();
  const int g4 = l >> 4, jl = l & 15;
  const int tile = grp * NWV + w;
  const bool active = tile < tiles;
  const bool is_T = active && tile < p.tiles_T;
  const int row0 = is_T ? 16 * tile : 16 * (tile - p.tiles_T);

  const bf16 *gq = reinterpret_cast<const bf16 *>(p.q);
  const bf16 *gk = reinterpret_cast<const bf16 *>(p.k);
  const bf16 *gv = reinterpret_cast<const bf16 *>(p.v);
  const bf16 *ga = reinterpret_cast<const bf16 *>(p.alpha);
  const bf16 *gb = reinterpret_cast<const bf16 *>(p.beta);
  const bf16 *gtau = reinterpret_cast<const bf16 *>(p.tau);

  // ---- S^T in C layout: block d holds S[row0 + jl][16 d + 4 g4 + i] ----
  f32x4 st[C::NSB];
#pragma unroll
  for (int d = 0; d < C::NSB; ++d) {
    st[d] = zero4();
    if (active) {
      if (is_T) {
#pragma unroll
        for (int i = 0; i < 4; ++i) st[d][i] = (row0 + jl == 16 * d + 4 * g4 + i) ? 1.f : 0.f;
      } else if (p.S0) {
        st[d] = *reinterpret_cast<const f32x4 *>(p.S0 + (((int64_t)n * H + h) * DV + row0 + jl) * DK + 16 * d + 4 * g4);
      }
    }
  }

  // ---- prefetch registers ----
  f32x4 pk[C::NKP], pq[C::NKP], pt[C::NTP];
  unsigned short pv[16], cv[16];  // V[t0 + 16 b + 4 g4 + i][row0 + jl], b = idx >> 2, i = idx & 3
  bf16 pa = bf16(1.f), pb = bf16(0.f);
  const int tbeg = p.cu[n], tend = p.cu[n + 1];
  const int64_t slot0 = (int64_t)(tbeg / CH) + n;

  auto prefetch = [&](int t0, int Lc, int64_t slot) {
#pragma unroll
    for (int i = 0; i < C::NKP; ++i) {
      const int s = tid + i * C::NT;
      const int r = s / C::KSEG, seg = s % C::KSEG;
      pk[i] = zero4();
      pq[i] = zero4();
      if (s < CH * C::KSEG && r < Lc) {
        const int64_t goff = ((int64_t)(t0 + r) * H + h) * DK + seg * 8;
        pk[i] = *reinterpret_cast<const f32x4 *>(gk + goff);
        if (WANT_O) pq[i] = *reinterpret_cast<const f32x4 *>(gq + goff);
      }
    }
    const bf16 *tsrc = gtau + (slot * H + h) * (int64_t)(2 * kPlane);
#pragma unroll
    for (int i = 0; i < C::NTP; ++i) {
      const int s = tid + i * C::NT;
      if (s < C::TSEG) pt[i] = *reinterpret_cast<const f32x4 *>(tsrc + 8 * s);
    }
#pragma unroll
    for (int idx = 0; idx < 16; ++idx) {
      const int r = 16 * (idx >> 2) + 4 * g4 + (idx & 3);
      pv[idx] = 0;
      if (active && !is_T && r < Lc)
        pv[idx] = *reinterpret_cast<const unsigned short *>(gv + ((int64_t)(t0 + r) * H + h) * DV + row0 + jl);
    }
    if (w == 0) {
      pa = bf16(1.f);
      pb = bf16(0.f);
      if (l < Lc) {
        const int64_t gi = (int64_t)(t0 + l) * H + h;
        pa = ga[gi];
        pb = gb[gi];
      }
    }
  };

  // stage the prefetched chunk into buffer set `b`
  auto stage = [&](int b, int Lc) {
    bf16 *sK = sK0 + b * KE;
    bf16 *sQ = sQ0 + b * KE;
    bf16 *sT = sT0 + b * TE;
#pragma unroll
    for (int i = 0; i < C::NKP; ++i) {
      const int s = tid + i * C::NT;
      if (s < CH * C::KSEG) {
        const int r = s / C::KSEG, seg = s % C::KSEG;
        *reinterpret_cast<f32x4 *>(sK + r * C::LDK + seg * 8) = pk[i];
        if (WANT_O) *reinterpret_cast<f32x4 *>(sQ + r * C::LDK + seg * 8) = pq[i];
      }
    }
#pragma unroll
    for (int i = 0; i < C::NTP; ++i) {
      const int s = tid + i * C::NT;
      if (s < C::TSEG) *reinterpret_cast<f32x4 *>(sT + 8 * s) = pt[i];
    }
    if (w == 0) {
      float *sG = sG0 + b * GE;
      const float g = wave_inclusive_scan((l < Lc) ? logf((float)pa) : 0.f);
      const float gL = lane_value(g, Lc - 1);
      sG[l] = g;
      sG[CH + l] = (l < Lc) ? (float)pb : 0.f;
      sG[2 * CH + l] = __expf(g);
      sG[3 * CH + l] = (l < Lc) ? __expf(gL - g) : 0.f;
      if (l == 0) sG[4 * CH] = __expf(gL);
    }
#pragma unroll
    for (int idx = 0; idx < 16; ++idx) cv[idx] = pv[idx];
  };

  // P = M o Q K^T of the chunk in buffer set `b`, packed lower block rows,
  // split planes (upper blocks are never read)
  auto build_p = [&](int b) {
    const bf16 *sK = sK0 + b * KE;
    const bf16 *sQ = sQ0 + b * KE;
    const float *sG = sG0 + b * GE;
    for (int t = w; t < 10; t += NWV) {
      const int bi = t < 1 ? 0 : (t < 3 ? 1 : (t < 6 ? 2 : 3));
      const int bj = t - (bi * (bi + 1)) / 2;
      f32x4 c = zero4();
      mma_bf16<1, 1>(c, RowMajor<bf16>{sQ, C::LDK}, RowMajor<bf16>{sK, C::LDK}, 16 * bi, 16 * bj, 0, DK);
      const int col = 16 * bj + jl;
      const float gc = sG[col];
      const int rb = 16 * bi + 4 * g4;
      const f32x4 gr = *reinterpret_cast<const f32x4 *>(sG + rb);
      bf16 *dst = sP + tau_off(bi) + 4 * g4 * 16 * (bi + 1) + col;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = (col <= rb + i) ? __expf(gr[i] - gc) * c[i] : 0.f;
        const bf16 hi = (bf16)x;
        dst[i * 16 * (bi + 1)] = hi;
        dst[i * 16 * (bi + 1) + kPlane] = (bf16)(x - (float)hi);
      }
    }
  };

  // A fragment of a packed lower block-row matrix (planes at M, M + kPlane)
  // for token block bt, permuted step m; columns past the stored block row
  // are zero.
  auto a_frag_packed = [&](const bf16 *M, int bt, int m, bf16x8 &hi, bf16x8 &lo) {
    const int ncol = 16 * (bt + 1);
    const bf16 *row = M + tau_off(bt) + jl * ncol;
    const int c0 = 32 * m + 4 * g4, c1 = c0 + 16;
    const uint2 z = uint2{0u, 0u};
    const uint2 h0 = *reinterpret_cast<const uint2 *>(row + c0);
    const uint2 l0 = *reinterpret_cast<const uint2 *>(row + kPlane + c0);
    const bool has1 = c1 < ncol;
    const uint2 h1 = has1 ? *reinterpret_cast<const uint2 *>(row + c1) : z;
    const uint2 l1 = has1 ? *reinterpret_cast<const uint2 *>(row + kPlane + c1) : z;
    hi = cat_bf16x8(h0, h1);
    lo = cat_bf16x8(l0, l1);
  };

  if (tbeg < tend) {
    prefetch(tbeg, min(CH, tend - tbeg), slot0);
    stage(0, min(CH, tend - tbeg));
    if (tbeg + CH < tend) prefetch(tbeg + CH, min(CH, tend - tbeg - CH), slot0 + 1);
  }
  lds_barrier();
  if (WANT_O && tbeg < tend) {
    build_p(0);
    lds_barrier();
  }

  int64_t slot = slot0;
  int b = 0;
  for (int t0 = tbeg; t0 < tend; t0 += CH, ++slot, b ^= 1) {
    const int Lc = min(CH, tend - t0);
    const bf16 *sK = sK0 + b * KE;
    const bf16 *sQ = sQ0 + b * KE;
    const bf16 *sT = sT0 + b * TE;
    const float *sG = sG0 + b * GE;

    if (active) {
      // S^T as k = 32 B fragments
      bf16x8 sh[C::NKS], sl[C::NKS];
#pragma unroll
      for (int m = 0; m < C::NKS; ++m) b_frag_split(st[2 * m], st[2 * m + 1], sh[m], sl[m]);

      // ---- Y = K S^T, R = beta (V - e^g Y) ----
      f32x4 rr[4];
#pragma unroll
      for (int bt = 0; bt < 4; ++bt) {
        f32x4 y = zero4();
        const bf16 *krow = sK + (16 * bt + jl) * C::LDK;
#pragma unroll
        for (int m = 0; m < C::NKS; ++m) {
          const bf16x8 a = a_frag_perm(krow, 32 * m, g4);
          y = mfma_bf16(a, sh[m], y);
          y = mfma_bf16(a, sl[m], y);
        }
        const f32x4 bet = *reinterpret_cast<const f32x4 *>(sG + CH + 16 * bt + 4 * g4);
        const f32x4 gam = *reinterpret_cast<const f32x4 *>(sG + 2 * CH + 16 * bt + 4 * g4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          union { unsigned u; float f; } vv;
          vv.u = (unsigned)cv[4 * bt + i] << 16;
          rr[bt][i] = bet[i] * (vv.f - gam[i] * y[i]);
        }
      }

      // ---- D = Tau R ----
      bf16x8 rh[2], rl[2];
      b_frag_split(rr[0], rr[1], rh[0], rl[0]);
      b_frag_split(rr[2], rr[3], rh[1], rl[1]);
      f32x4 dd[4];
#pragma unroll
      for (int bt = 0; bt < 4; ++bt) {
        f32x4 c = zero4();
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          if (m > (bt >> 1)) continue;
          bf16x8 ah, alo;
          a_frag_packed(sT, bt, m, ah, alo);
          c = mfma_bf16(ah, rh[m], c);
          c = mfma_bf16(ah, rl[m], c);
          c = mfma_bf16(alo, rh[m], c);
        }
        dd[bt] = c;
      }

      // ---- O = e^g Q S^T + P D ----
      if (WANT_O) {
        bf16x8 dh[2], dl[2];
        b_frag_split(dd[0], dd[1], dh[0], dl[0]);
        b_frag_split(dd[2], dd[3], dh[1], dl[1]);
#pragma unroll
        for (int bt = 0; bt < 4; ++bt) {
          f32x4 z = zero4();
          const bf16 *qrow = sQ + (16 * bt + jl) * C::LDK;
#pragma unroll
          for (int m = 0; m < C::NKS; ++m) {
            const bf16x8 a = a_frag_perm(qrow, 32 * m, g4);
            z = mfma_bf16(a, sh[m], z);
            z = mfma_bf16(a, sl[m], z);
          }
          const f32x4 gam = *reinterpret_cast<const f32x4 *>(sG + 2 * CH + 16 * bt + 4 * g4);
#pragma unroll
          for (int i = 0; i < 4; ++i) z[i] *= gam[i];
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            if (m > (bt >> 1)) continue;
            bf16x8 ah, alo;
            a_frag_packed(sP, bt, m, ah, alo);
            z = mfma_bf16(ah, dh[m], z);
            z = mfma_bf16(ah, dl[m], z);
            z = mfma_bf16(alo, dh[m], z);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 16 * bt + 4 * g4 + i;
            if (r < Lc) {
              const int64_t oi = ((int64_t)(t0 + r) * H + h) * DV + row0 + jl;
              if (p.o_bf16)
                reinterpret_cast<bf16 *>(p.o)[oi] = (bf16)z[i];
              else
                reinterpret_cast<float *>(p.o)[oi] = z[i];
            }
          }
        }
      }

      // ---- S^T <- e^{g_L} S^T + K^T diag(e^{g_L - g}) D ----
      bf16x8 eh[2], el[2];
      {
        f32x4 de[4];
#pragma unroll
        for (int bt = 0; bt < 4; ++bt) {
          const f32x4 dec = *reinterpret_cast<const f32x4 *>(sG + 3 * CH + 16 * bt + 4 * g4);
#pragma unroll
          for (int i = 0; i < 4; ++i) de[bt][i] = dd[bt][i] * dec[i];
        }
        b_frag_split(de[0], de[1], eh[0], el[0]);
        b_frag_split(de[2], de[3], eh[1], el[1]);
      }
      const float gl = sG[4 * CH];
#pragma unroll
      for (int d = 0; d < C::NSB; ++d) {
        f32x4 c = st[d];
#pragma unroll
        for (int i = 0; i < 4; ++i) c[i] *= gl;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const bf16x8 a = a_frag_trans_perm(sK, C::LDK, 32 * m, 16 * d, l);
          c = mfma_bf16(a, eh[m], c);
          c = mfma_bf16(a, el[m], c);
        }
        st[d] = c;
      }
    }

    // ---- stage the next chunk into the other buffer set ----
    if (t0 + CH < tend) {
      stage(b ^ 1, min(CH, tend - t0 - CH));
      if (t0 + 2 * CH < tend) prefetch(t0 + 2 * CH, min(CH, tend - t0 - 2 * CH), slot + 2);
    }
    lds_barrier();
    if (WANT_O && t0 + CH < tend) {
      build_p(b ^ 1);
      lds_barrier();
    }
  }

  // ---------------- epilogue: final rows ----------------
  if (active) {
    float *out = is_T ? p.T_out : p.S_out;
    const int nrows = is_T ? DK : DV;
#pragma unroll
    for (int d = 0; d < C::NSB; ++d)
      *reinterpret_cast<f32x4 *>(out + (((int64_t)n * H + h) * nrows + row0 + jl) * DK + 16 * d + 4 * g4) = st[d];
  }
}

template <int DK, int NWV, bool WANT_O>
hipError_t launch_b(const ChainLaunch &p, hipStream_t stream) {
  const int tiles = p.tiles_T + p.tiles_S;
  const int64_t items = (int64_t)p.n_seqs * p.H * ((tiles + NWV - 1) / NWV);
  if (items <= 0) return hipSuccess;
  const int64_t grid = (items + 7) / 8 * 8;
  hipLaunchKernelGGL((chain_bf16_kernel<DK, NWV, WANT_O>), dim3((unsigned)grid), dim3(NWV * 64), 0, stream, p,
                     (int)items);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chain_bf16(const ChainLaunch &p, hipStream_t stream) {
  if (p.dk == 64) return p.o ? launch_b<64, 4, true>(p, stream) : launch_b<64, 4, false>(p, stream);
  if (p.dk == 128) return p.o ? launch_b<128, 4, true>(p, stream) : launch_b<128, 4, false>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace gdn
