// gdn_chain_bf16.hip -- chunkwise Gated DeltaNet recurrence for bf16 inputs
// on gfx950: one workgroup of four waves per 16 state rows.
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
// S^T (dk x 16) stays in registers in MFMA C layout, split by dk blocks
// over the four waves.  A C-layout result is used directly as the B operand
// of the next product (k = 16 tiles, or paired tiles with a permuted k
// order for k = 32, gdn_device.h).  Per chunk:
//   1. each wave forms the partial Y (and Z = Q S^T) over its dk blocks and
//      posts it to LDS                                         | barrier
//   2. every wave sums the partials, forms R; wave w forms token block w
//      of D = Tau R and posts D and diag(e^{g_L - g}) D          | barrier
//   3. wave w writes the outputs of token block w and updates its dk
//      blocks of S^T with K^T diag(e^{g_L - g}) D; the workgroup stages the
//      next chunk (keys, queries, values, Tau, gates)          | barrier
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
// Inputs are double-buffered in LDS by chunk parity; the global loads of a
// chunk are issued one chunk period before it is staged.  With outputs,
// M o QK^T of the next chunk is built after its keys and queries land (one
// more barrier).  All barriers are LDS-only.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int CH = kChunk;
// packed lower block-row matrix (Tau or M o QK^T) as split bf16 planes:
// hi at [0, kPlane), lo at [kPlane, 2 kPlane)
constexpr int kPlane = kTauFloats;

template <int DK, bool WANT_O>
struct BCfg {
  static constexpr int NWV = 4;                       // waves per workgroup (one 16-row tile)
  static constexpr int NT = NWV * 64;
  static constexpr int LDK = DK + 8;                  // sK, sQ [CH][LDK] bf16
  static constexpr int LDV = 16 + 8;                  // sV [CH][LDV] bf16 (the tile's 16 value columns)
  static constexpr int NSB = DK / 16;                 // 16-row blocks of S^T
  static constexpr int NOWN = NSB / NWV;              // blocks of S^T owned by a wave (1 or 2)
  static constexpr int NX = WANT_O ? 8 : 4;           // exchanged partial tiles per wave (Y, Z)
  static constexpr size_t al(size_t x) { return (x + 15) & ~size_t(15); }
  static constexpr size_t KBYTES = al(2 * CH * LDK);
  static constexpr size_t VBYTES = al(2 * CH * LDV);
  static constexpr size_t TBYTES = al(2 * kPlane * sizeof(bf16));    // hi + lo planes
  static constexpr size_t GBYTES = al(4 * 5 * CH);
  static constexpr size_t oK = 0;                                    // [2]
  static constexpr size_t oQ = oK + 2 * KBYTES;                      // [2] (o)
  static constexpr size_t oV = oQ + (WANT_O ? 2 * KBYTES : 0);       // [2]
  static constexpr size_t oT = oV + 2 * VBYTES;                      // [2] Tau planes
  static constexpr size_t oP = oT + 2 * TBYTES;                      // [1] P planes (o)
  static constexpr size_t oG = oP + (WANT_O ? TBYTES : 0);           // [2] gates
  static constexpr size_t oX = oG + 2 * GBYTES;                      // partial-sum exchange
  static constexpr size_t oE = oX + (size_t)NWV * NX * 64 * 16;      // D / D'' exchange
  static constexpr size_t TOTAL = oE + (size_t)NWV * 2 * 64 * 16;
  static_assert(TOTAL <= 160 * 1024, "LDS budget");
  // staging: 16-byte segments
  static constexpr int KSEG = DK / 8;
  static constexpr int NKP = (CH * KSEG + NT - 1) / NT;
  static constexpr int TSEG = (int)(2 * kPlane * sizeof(bf16) / 16);
  static constexpr int NTP = (TSEG + NT - 1) / NT;
};

__device__ __forceinline__ bf16x4 u2_bf16x4(uint2 u) {
  union { uint2 u; bf16x4 v; } x;
  x.u = u;
  return x.v;
}

template <int DK, bool WANT_O>
__global__ void __launch_bounds__(256) chain_bf16_kernel(ChainLaunch p, int n_items) {
  using C = BCfg<DK, WANT_O>;
  constexpr int NWV = C::NWV;
  __shared__ __attribute__((aligned(16))) char smem[C::TOTAL];
  bf16 *sK0 = reinterpret_cast<bf16 *>(smem + C::oK);
  bf16 *sQ0 = reinterpret_cast<bf16 *>(smem + C::oQ);
  bf16 *sV0 = reinterpret_cast<bf16 *>(smem + C::oV);
  bf16 *sT0 = reinterpret_cast<bf16 *>(smem + C::oT);
  bf16 *sP = reinterpret_cast<bf16 *>(smem + C::oP);
  float *sG0 = reinterpret_cast<float *>(smem + C::oG);
  f32x4 *sX = reinterpret_cast<f32x4 *>(smem + C::oX);
  f32x4 *sE = reinterpret_cast<f32x4 *>(smem + C::oE);
  constexpr int KE = C::KBYTES / 2, VE = C::VBYTES / 2, TE = C::TBYTES / 2, GE = C::GBYTES / 4;

  // ---- work item (XCD-aware order): one 16-row tile of one (sequence, head) ----
  const int per = (int)(gridDim.x >> 3);
  const int item = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
  if (item >= n_items) return;
  const int tiles = p.tiles_T + p.tiles_S;
  const int unit = item / tiles, tile = item % tiles;
  const int n = unit / p.H, h = unit % p.H;
  const int H = p.H, DV = p.dv;
  const bool is_T = tile < p.tiles_T;
  const int row0 = is_T ? 16 * tile : 16 * (tile - p.tiles_T);
  const int tid = threadIdx.x, w = wave_id(), l = lane_id();
  const int g4 = l >> 4, jl = l & 15;

  const bf16 *gq = reinterpret_cast<const bf16 *>(p.q);
  const bf16 *gk = reinterpret_cast<const bf16 *>(p.k);
  const bf16 *gv = reinterpret_cast<const bf16 *>(p.v);
  const bf16 *ga = reinterpret_cast<const bf16 *>(p.alpha);
  const bf16 *gb = reinterpret_cast<const bf16 *>(p.beta);
  const bf16 *gtau = reinterpret_cast<const bf16 *>(p.tau);

  // ---- owned blocks of S^T (C layout): st[u] holds S[row0 + jl][16 d + 4 g4 + i],
  // d = w NOWN + u ----
  f32x4 st[C::NOWN];
#pragma unroll
  for (int u = 0; u < C::NOWN; ++u) {
    const int d = w * C::NOWN + u;
    st[u] = zero4();
    if (is_T) {
#pragma unroll
      for (int i = 0; i < 4; ++i) st[u][i] = (row0 + jl == 16 * d + 4 * g4 + i) ? 1.f : 0.f;
    } else if (p.S0) {
      st[u] = *reinterpret_cast<const f32x4 *>(p.S0 + (((int64_t)n * H + h) * DV + row0 + jl) * DK + 16 * d + 4 * g4);
    }
  }
  // Let the start-state loads land here: otherwise the compiler's wait
  // bookkeeping keeps them pending into the chunk loop and waits for all
  // global loads (including the prefetch) at the top of every iteration.
  wait_vmem();

  // ---- prefetch registers (one chunk ahead of staging) ----
  f32x4 pk[C::NKP], pq[C::NKP], pt[C::NTP], pvv;
  bf16 pa = bf16(1.f), pb = bf16(0.f);
  const int tbeg = p.cu[n], tend = p.cu[n + 1];
  const int64_t slot0 = (int64_t)(tbeg / CH) + n;

  auto prefetch = [&](int t0, int Lc, int64_t slot) {
    const bool full = Lc == CH;
#pragma unroll
    for (int i = 0; i < C::NKP; ++i) {
      const int s = tid + i * C::NT;
      const int r = s / C::KSEG, seg = s % C::KSEG;
      const bool ok = (s < CH * C::KSEG) && (full || r < Lc);
      const int64_t goff = ((int64_t)(t0 + r) * H + h) * DK + seg * 8;
      pk[i] = ok ? *reinterpret_cast<const f32x4 *>(gk + goff) : zero4();
      if (WANT_O) pq[i] = ok ? *reinterpret_cast<const f32x4 *>(gq + goff) : zero4();
    }
    const bf16 *tsrc = gtau + (slot * H + h) * (int64_t)(2 * kPlane);
#pragma unroll
    for (int i = 0; i < C::NTP; ++i) {
      const int s = tid + i * C::NT;
      if (s < C::TSEG) pt[i] = *reinterpret_cast<const f32x4 *>(tsrc + 8 * s);
    }
    {
      // V rows t0 + r, columns row0 .. row0 + 15: 2 segments per token
      const int r = tid >> 1, seg = tid & 1;
      const bool ok = !is_T && tid < 2 * CH && (full || r < Lc);
      pvv = ok ? *reinterpret_cast<const f32x4 *>(gv + ((int64_t)(t0 + r) * H + h) * DV + row0 + 8 * seg) : zero4();
    }
    if (w == 0) {
      const bool ok = l < Lc;
      const int64_t gi = (int64_t)(t0 + l) * H + h;
      pa = ok ? ga[gi] : bf16(1.f);
      pb = ok ? gb[gi] : bf16(0.f);
    }
  };

  // stage the prefetched chunk into buffer set `b`
  auto stage = [&](int b, int Lc) {
    bf16 *sK = sK0 + b * KE;
    bf16 *sQ = sQ0 + b * KE;
    bf16 *sT = sT0 + b * TE;
    bf16 *sV = sV0 + b * VE;
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
    if (tid < 2 * CH) *reinterpret_cast<f32x4 *>(sV + (tid >> 1) * C::LDV + 8 * (tid & 1)) = pvv;
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
  };

  // P = M o Q K^T of the chunk in buffer set `b`: packed lower block rows,
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

  // A fragment (permuted k = 32 step m) of a packed lower block-row matrix,
  // token block bt; columns past the stored block row are zero.
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
    const bf16 *sV = sV0 + b * VE;
    const bf16 *sT = sT0 + b * TE;
    const float *sG = sG0 + b * GE;

    // ---- 1. partial Y = K S^T (and Z = Q S^T) over the owned dk blocks ----
    // (all fragment loads first, then the products on independent
    // accumulators, then the stores)
    {
      f32x4 y[4], z[4];
#pragma unroll
      for (int bt = 0; bt < 4; ++bt) {
        y[bt] = zero4();
        z[bt] = zero4();
      }
      if constexpr (C::NOWN == 2) {
        // the two owned blocks form one k = 32 step (permuted k order)
        bf16x8 sh, sl;
        b_frag_split(st[0], st[1], sh, sl);
        bf16x8 ka[4], qa[4];
#pragma unroll
        for (int bt = 0; bt < 4; ++bt) {
          ka[bt] = a_frag_perm(sK + (16 * bt + jl) * C::LDK, 32 * w, g4);
          if (WANT_O) qa[bt] = a_frag_perm(sQ + (16 * bt + jl) * C::LDK, 32 * w, g4);
        }
#pragma unroll
        for (int bt = 0; bt < 4; ++bt) y[bt] = mfma_bf16(ka[bt], sh, y[bt]);
#pragma unroll
        for (int bt = 0; bt < 4; ++bt) y[bt] = mfma_bf16(ka[bt], sl, y[bt]);
        if (WANT_O) {
#pragma unroll
          for (int bt = 0; bt < 4; ++bt) z[bt] = mfma_bf16(qa[bt], sh, z[bt]);
#pragma unroll
          for (int bt = 0; bt < 4; ++bt) z[bt] = mfma_bf16(qa[bt], sl, z[bt]);
        }
      } else {
        bf16x4 sh, sl;
        split4(st[0], sh, sl);
        uint2 ka[4], qa[4];
#pragma unroll
        for (int bt = 0; bt < 4; ++bt) {
          const int off = (16 * bt + jl) * C::LDK + 16 * w + 4 * g4;
          ka[bt] = *reinterpret_cast<const uint2 *>(sK + off);
          if (WANT_O) qa[bt] = *reinterpret_cast<const uint2 *>(sQ + off);
        }
#pragma unroll
        for (int bt = 0; bt < 4; ++bt) y[bt] = mfma_bf16_k16(u2_bf16x4(ka[bt]), sh, y[bt]);
#pragma unroll
        for (int bt = 0; bt < 4; ++bt) y[bt] = mfma_bf16_k16(u2_bf16x4(ka[bt]), sl, y[bt]);
        if (WANT_O) {
#pragma unroll
          for (int bt = 0; bt < 4; ++bt) z[bt] = mfma_bf16_k16(u2_bf16x4(qa[bt]), sh, z[bt]);
#pragma unroll
          for (int bt = 0; bt < 4; ++bt) z[bt] = mfma_bf16_k16(u2_bf16x4(qa[bt]), sl, z[bt]);
        }
      }
#pragma unroll
      for (int bt = 0; bt < 4; ++bt) {
        sX[(w * C::NX + bt) * 64 + l] = y[bt];
        if (WANT_O) sX[(w * C::NX + 4 + bt) * 64 + l] = z[bt];
      }
    }
    lds_barrier();

    // ---- 2. Y (summed), R = beta (V - e^g Y); D_w = (Tau R)_w ----
    {
      f32x4 part[NWV][4];
      uint2 vraw[4];
      f32x4 bet[4], gam[4];
#pragma unroll
      for (int bt = 0; bt < 4; ++bt) {
#pragma unroll
        for (int q = 0; q < NWV; ++q) part[q][bt] = sX[(q * C::NX + bt) * 64 + l];
        // V[16 bt + 4 g4 + e][jl] via the transposing read of the row-major tile
        vraw[bt] = ds_read_tr16(sV + (16 * bt + 4 * g4 + (jl >> 2)) * C::LDV + 4 * (jl & 3));
        bet[bt] = *reinterpret_cast<const f32x4 *>(sG + CH + 16 * bt + 4 * g4);
        gam[bt] = *reinterpret_cast<const f32x4 *>(sG + 2 * CH + 16 * bt + 4 * g4);
      }
      // Tau fragments of token block w (hi / lo planes, up to two k steps)
      bf16x8 th[2], tl[2];
#pragma unroll
      for (int m = 0; m < 2; ++m)
        if (m <= (w >> 1)) a_frag_packed(sT, w, m, th[m], tl[m]);
      const f32x4 dec = *reinterpret_cast<const f32x4 *>(sG + 3 * CH + 16 * w + 4 * g4);
      f32x4 rr[4];
#pragma unroll
      for (int bt = 0; bt < 4; ++bt) {
        const bf16x4 vv = u2_bf16x4(vraw[bt]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float y = part[0][bt][i];
#pragma unroll
          for (int q = 1; q < NWV; ++q) y += part[q][bt][i];
          rr[bt][i] = bet[bt][i] * ((float)vv[i] - gam[bt][i] * y);
        }
      }
      bf16x8 rh[2], rl[2];
      b_frag_split(rr[0], rr[1], rh[0], rl[0]);
      b_frag_split(rr[2], rr[3], rh[1], rl[1]);
      // three independent accumulators (one per split product), summed at the end
      f32x4 c0 = zero4(), c1 = zero4(), c2 = zero4();
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        if (m > (w >> 1)) continue;
        c0 = mfma_bf16(th[m], rh[m], c0);
        c1 = mfma_bf16(th[m], rl[m], c1);
        c2 = mfma_bf16(tl[m], rh[m], c2);
      }
      f32x4 c, cd;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c[i] = c0[i] + c1[i] + c2[i];
        cd[i] = c[i] * dec[i];
      }
      sE[(w * 2 + 0) * 64 + l] = cd;
      if (WANT_O) sE[(w * 2 + 1) * 64 + l] = c;
    }
    lds_barrier();

    // ---- 3. outputs of token block w; update of the owned S^T blocks ----
    {
      // K^T fragments of the owned dk blocks, and D'' for all token blocks
      bf16x8 kt[C::NOWN][2];
#pragma unroll
      for (int u = 0; u < C::NOWN; ++u)
#pragma unroll
        for (int m = 0; m < 2; ++m) kt[u][m] = a_frag_trans_perm(sK, C::LDK, 32 * m, 16 * (w * C::NOWN + u), l);
      f32x4 e4[4];
#pragma unroll
      for (int bt = 0; bt < 4; ++bt) e4[bt] = sE[(bt * 2) * 64 + l];
      const float gl = sG[4 * CH];

      if (WANT_O) {
        f32x4 zp[NWV], d4[4];
#pragma unroll
        for (int q = 0; q < NWV; ++q) zp[q] = sX[(q * C::NX + 4 + w) * 64 + l];
#pragma unroll
        for (int bt = 0; bt < 4; ++bt) d4[bt] = sE[(bt * 2 + 1) * 64 + l];
        bf16x8 ph[2], pl[2];
#pragma unroll
        for (int m = 0; m < 2; ++m)
          if (m <= (w >> 1)) a_frag_packed(sP, w, m, ph[m], pl[m]);
        const f32x4 gam = *reinterpret_cast<const f32x4 *>(sG + 2 * CH + 16 * w + 4 * g4);
        bf16x8 dh[2], dl[2];
        b_frag_split(d4[0], d4[1], dh[0], dl[0]);
        b_frag_split(d4[2], d4[3], dh[1], dl[1]);
        f32x4 o0 = zero4(), o1 = zero4(), o2 = zero4();
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          if (m > (w >> 1)) continue;
          o0 = mfma_bf16(ph[m], dh[m], o0);
          o1 = mfma_bf16(ph[m], dl[m], o1);
          o2 = mfma_bf16(pl[m], dh[m], o2);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float zz = zp[0][i];
#pragma unroll
          for (int q = 1; q < NWV; ++q) zz += zp[q][i];
          const float ov = gam[i] * zz + (o0[i] + o1[i] + o2[i]);
          const int r = 16 * w + 4 * g4 + i;
          if (r < Lc) {
            const int64_t oi = ((int64_t)(t0 + r) * H + h) * DV + row0 + jl;
            if (p.o_bf16)
              reinterpret_cast<bf16 *>(p.o)[oi] = (bf16)ov;
            else
              reinterpret_cast<float *>(p.o)[oi] = ov;
          }
        }
      }

      bf16x8 eh[2], el[2];
      b_frag_split(e4[0], e4[1], eh[0], el[0]);
      b_frag_split(e4[2], e4[3], eh[1], el[1]);
      f32x4 a0[C::NOWN], a1[C::NOWN];
#pragma unroll
      for (int u = 0; u < C::NOWN; ++u) {
        a0[u] = st[u];
#pragma unroll
        for (int i = 0; i < 4; ++i) a0[u][i] *= gl;
        a1[u] = zero4();
      }
#pragma unroll
      for (int m = 0; m < 2; ++m) {
#pragma unroll
        for (int u = 0; u < C::NOWN; ++u) a0[u] = mfma_bf16(kt[u][m], eh[m], a0[u]);
#pragma unroll
        for (int u = 0; u < C::NOWN; ++u) a1[u] = mfma_bf16(kt[u][m], el[m], a1[u]);
      }
#pragma unroll
      for (int u = 0; u < C::NOWN; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) st[u][i] = a0[u][i] + a1[u][i];
    }

    // ---- 4. stage the next chunk into the other buffer set ----
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

  // ---------------- epilogue: owned blocks of the final rows ----------------
  {
    float *out = is_T ? p.T_out : p.S_out;
    const int nrows = is_T ? DK : DV;
#pragma unroll
    for (int u = 0; u < C::NOWN; ++u) {
      const int d = w * C::NOWN + u;
      *reinterpret_cast<f32x4 *>(out + (((int64_t)n * H + h) * nrows + row0 + jl) * DK + 16 * d + 4 * g4) = st[u];
    }
  }
}

template <int DK, bool WANT_O>
hipError_t launch_b(const ChainLaunch &p, hipStream_t stream) {
  const int64_t items = (int64_t)p.n_seqs * p.H * (p.tiles_T + p.tiles_S);
  if (items <= 0) return hipSuccess;
  const int64_t grid = (items + 7) / 8 * 8;
  hipLaunchKernelGGL((chain_bf16_kernel<DK, WANT_O>), dim3((unsigned)grid), dim3(256), 0, stream, p, (int)items);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chain_bf16(const ChainLaunch &p, hipStream_t stream) {
  if (p.dk == 64) return p.o ? launch_b<64, true>(p, stream) : launch_b<64, false>(p, stream);
  if (p.dk == 128) return p.o ? launch_b<128, true>(p, stream) : launch_b<128, false>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace gdn
