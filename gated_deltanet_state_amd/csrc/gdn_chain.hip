// gdn_chain.hip -- chunkwise Gated DeltaNet recurrence for gfx950.
//
// The recurrence (page "Tail-Replay: Escaping the Curse of Linear Attention
// in Prefix Caching for Hybrid LLMs", section 2 Eq. (1); state S dv x dk):
//     S_t = S_{t-1} alpha_t (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,  o_t = S_t q_t.
// Unrolled over a chunk of L <= 64 tokens with cumulative log-gates
// g_r = sum_{s<=r} log alpha_s (substitute the state before each token into
// the delta-rule correction of the next one), with Tau = (I + A)^{-1} built
// per chunk by the prep kernel (gdn_prep.hip):
//     R    = diag(beta) (V - diag(e^g) K S^T)
//     D    = Tau R                                     (per-token corrections)
//     O    = diag(e^g) Q S^T + (M o Q K^T) D,          M_rs = e^{g_r - g_s}, s <= r
//     S   <- e^{g_L} S + (diag(e^{g_L - g}) D)^T K
// Rows of S evolve independently: a workgroup owns 16 rows of one
// (sequence, head) state and walks its chunks in order; all products are
// computed transposed (the 16 state rows are the MFMA M dimension).
//
// The same kernel builds the affine chunk operator of the page "LinearKV:
// One Cached State Suffices for Position-Independent Caching in Hybrid
// LLMs" (affine chunk operator paragraph): rows of the transition product
// T_C are rows of a "state" that starts as the identity and receives no
// value input.
//
// This kernel serves fp32 inputs (bf16 inputs have gdn_chain_bf16.hip): every
// product runs on the fp32 MFMA (v_mfma_f32_16x16x4_f32).
//
// Four waves; wave w owns token block w (16 tokens) of every 16 x 64 tile
// (Y, R, D, O) and state column tiles w, w + 4.  Per chunk, three phases
// separated by LDS-only barriers (each chunk's global loads are issued one
// chunk period before they are staged and stay in flight across the
// barriers); keys and gates are double-buffered in LDS:
//   P1  Y = S K^T -> R;  [o] Z = e^g S Q^T,  P = M o Q K^T
//   P2  D = R Tau^T (Tau rows straight from registers)
//   P3  [o] O = Z + D P^T -> o;  S = e^{g_L} S + (e^{g_L - g} D)^T K; then
//       state planes, the next chunk's keys / queries / gates to LDS, and
//       the loads of the chunk after it
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int CH = kChunk;  // tokens per chunk
constexpr int NW = 4;       // waves per workgroup
constexpr int NT = NW * 64; // threads per workgroup
constexpr int RT = 16;      // state rows per workgroup

template <int DK, bool WANT_O>
struct Cfg {
  // leading dimensions (elements): single-element reads, odd strides against
  // bank conflicts
  static constexpr int LDK = DK + 1;   // sK, sQ [CH][LDK]
  static constexpr int LDC = CH + 1;   // sP [CH][LDC]
  static constexpr int LDSP = DK + 1;  // state [RT][LDSP]
  static constexpr int LDRP = CH + 1;  // R, D, Dd [RT][LDRP]

  static constexpr size_t al(size_t x) { return (x + 15) & ~size_t(15); }
  static constexpr size_t KBYTES = al(4 * CH * LDK);
  static constexpr size_t oK = 0;                     // two buffers (chunk parity)
  static constexpr size_t oQ = oK + 2 * KBYTES;
  static constexpr size_t oP = oQ + (WANT_O ? al(4 * CH * LDK) : 0);
  static constexpr size_t oS = oP + (WANT_O ? al(4 * CH * LDC) : 0);
  static constexpr size_t oR = oS + al(4 * RT * LDSP);
  static constexpr size_t oD = oR + al(4 * RT * LDRP);
  static constexpr size_t oDd = oD + (WANT_O ? al(4 * RT * LDRP) : 0);
  static constexpr size_t oGate = oDd + al(4 * RT * LDRP);
  static constexpr size_t GBYTES = al(4 * 5 * CH);
  static constexpr size_t TOTAL = oGate + 2 * GBYTES;  // two gate buffers
  static_assert(TOTAL <= 160 * 1024, "LDS budget");

  static constexpr int NST = DK / 16;          // state column tiles
  static constexpr int SPW = (NST + NW - 1) / NW;
  static constexpr int VEC = 4;                // floats per 16-byte load
  static constexpr int KSEG = DK / VEC;        // 16-byte segments per key row
  static constexpr int NKP = (CH * KSEG + NT - 1) / NT;
  static constexpr int NTF = 4;                // Tau row: 16 single elements (k step 4)
};

template <int DK, bool WANT_O>
__global__ void __launch_bounds__(NT) chain_kernel(ChainLaunch p, int n_items) {
  using C = Cfg<DK, WANT_O>;
  using Tin = float;
  __shared__ __attribute__((aligned(16))) char smem[C::TOTAL];
  float *sK0 = reinterpret_cast<float *>(smem + C::oK);
  float *sQ = reinterpret_cast<float *>(smem + C::oQ);
  float *sP = reinterpret_cast<float *>(smem + C::oP);
  float *sSh = reinterpret_cast<float *>(smem + C::oS);
  float *sRh = reinterpret_cast<float *>(smem + C::oR);
  float *sDh = reinterpret_cast<float *>(smem + C::oD);
  float *sDdh = reinterpret_cast<float *>(smem + C::oDd);
  // gate buffer (per chunk parity): g_r | beta_r (0 past the chunk end) |
  // e^{g_r} | e^{g_L - g_r} (0 past the end) | [0] = e^{g_L}
  float *sGate0 = reinterpret_cast<float *>(smem + C::oGate);

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
  const int row0 = is_T ? RT * tile : RT * (tile - p.tiles_T);
  const int H = p.H, DV = p.dv;

  const int tid = threadIdx.x, w = wave_id(), l = lane_id();
  const int cb = w;  // token block of this wave
  const Tin *gq = reinterpret_cast<const Tin *>(p.q);
  const Tin *gk = reinterpret_cast<const Tin *>(p.k);
  const Tin *gv = reinterpret_cast<const Tin *>(p.v);
  const Tin *ga = reinterpret_cast<const Tin *>(p.alpha);
  const Tin *gb = reinterpret_cast<const Tin *>(p.beta);

  // ---- state column tiles ct = w + NW u in registers (C layout) ----
  f32x4 sacc[C::SPW];
#pragma unroll
  for (int u = 0; u < C::SPW; ++u) {
    sacc[u] = zero4();
    const int ct = w + u * NW;
    if (ct < C::NST) {
      const int col = 16 * ct + (l & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = row0 + 4 * (l >> 4) + i;
        if (is_T)
          sacc[u][i] = (r == col) ? 1.f : 0.f;
        else if (p.S0)
          sacc[u][i] = p.S0[(((int64_t)n * H + h) * DV + r) * DK + col];
      }
    }
  }

  wait_vmem();  // start-state loads land before the chunk loop (see the bf16 kernel)

  // ---- prefetch registers (next chunk) and current-chunk copies ----
  f32x4 pk[C::NKP], pq[C::NKP];
  f32x4 ptau[C::NTF], ctau[C::NTF];
  // V[t0 + 16 cb + (l & 15)][row0 + 4 (l >> 4) .. + 3]
  using VRaw = f32x4;
  VRaw pvv, cvv;
  // gates are carried as loaded (no conversion) so that issuing the next
  // chunk's loads never waits for them
  Tin pa = Tin(1.f), pb = Tin(0.f);
  const int tbeg = p.cu[n], tend = p.cu[n + 1];
  const int64_t slot0 = (int64_t)(tbeg / CH) + n;

  auto prefetch = [&](int t0, int Lc, int64_t slot) {
#pragma unroll
    for (int i = 0; i < C::NKP; ++i) {
      const int s = tid + i * NT;
      const int r = s / C::KSEG, seg = s % C::KSEG;
      pk[i] = zero4();
      pq[i] = zero4();
      if (s < CH * C::KSEG && r < Lc) {
        const int64_t goff = ((int64_t)(t0 + r) * H + h) * DK + seg * C::VEC;
        pk[i] = *reinterpret_cast<const f32x4 *>(gk + goff);
        if (WANT_O) pq[i] = *reinterpret_cast<const f32x4 *>(gq + goff);
      }
    }
    // Tau rows 16 cb + (l & 15) of this chunk
    const float *tau = p.tau + (slot * H + h) * (int64_t)kRecFloats + tau_off(cb) + (l & 15) * 16 * (cb + 1);
    const int ncol = 16 * (cb + 1);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int s = 4 * i + (l >> 4);
      ptau[i >> 2][i & 3] = (s < ncol) ? tau[s] : 0.f;
    }
    pvv = VRaw{};
    const int r = 16 * cb + (l & 15);
    if (!is_T && r < Lc) {
      const Tin *src = gv + ((int64_t)(t0 + r) * H + h) * DV + row0 + 4 * (l >> 4);
      pvv = *reinterpret_cast<const VRaw *>(src);
    }
    if (w == 0) {
      pa = Tin(1.f);
      pb = Tin(0.f);
      if (l < Lc) {
        const int64_t gi = (int64_t)(t0 + l) * H + h;
        pa = ga[gi];
        pb = gb[gi];
      }
    }
  };

  // Store a prefetched chunk into K buffer `kb` (and Q), gates into gate
  // buffer `kb`; move the per-wave fragments to their "current" copies.
  auto stage = [&](int kb, int Lc) {
    Tin *sKb = sK0 + kb * (C::KBYTES / sizeof(Tin));
#pragma unroll
    for (int i = 0; i < C::NKP; ++i) {
      const int s = tid + i * NT;
      if (s < CH * C::KSEG) {
        const int r = s / C::KSEG, seg = s % C::KSEG;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sKb[r * C::LDK + seg * 4 + e] = pk[i][e];
          if (WANT_O) sQ[r * C::LDK + seg * 4 + e] = pq[i][e];
        }
      }
    }
    if (w == 0) {
      float *sGb = sGate0 + kb * (C::GBYTES / 4);
      const float g = wave_inclusive_scan((l < Lc) ? log_gate(to_f32(pa)) : 0.f);
      const float gL = lane_value(g, Lc - 1);
      sGb[l] = g;
      sGb[CH + l] = (l < Lc) ? to_f32(pb) : 0.f;
      sGb[2 * CH + l] = __expf(g);
      sGb[3 * CH + l] = (l < Lc) ? __expf(gL - g) : 0.f;
      if (l == 0) sGb[4 * CH] = __expf(gL);
    }
#pragma unroll
    for (int i = 0; i < C::NTF; ++i) ctau[i] = ptau[i];
    cvv = pvv;
  };
  auto store_state_planes = [&]() {
#pragma unroll
    for (int u = 0; u < C::SPW; ++u) {
      const int ct = w + u * NW;
      if (ct < C::NST) store_tile(sSh, C::LDSP, 0, 16 * ct, sacc[u]);
    }
  };

  if (tbeg < tend) {
    prefetch(tbeg, min(CH, tend - tbeg), slot0);
    stage(0, min(CH, tend - tbeg));
    store_state_planes();
    if (tbeg + CH < tend) prefetch(tbeg + CH, min(CH, tend - tbeg - CH), slot0 + 1);
  }
  lds_barrier();

  int64_t slot = slot0;
  int kb = 0;
  for (int t0 = tbeg; t0 < tend; t0 += CH, ++slot, kb ^= 1) {
    const int Lc = min(CH, tend - t0);
    const Tin *sK = sK0 + kb * (C::KBYTES / sizeof(Tin));
    const float *sG = sGate0 + kb * (C::GBYTES / 4);
    const float *sBeta = sG + CH, *sGam = sG + 2 * CH, *sDec = sG + 3 * CH;

    // ================= P1: Y -> R ; Z, P =================
    {
      f32x4 c = zero4();
      mma_f32(c, RowMajor<float>{sSh, C::LDSP}, RowMajor<float>{sK, C::LDK}, 0, 16 * cb, 0, DK);
      const int r = 16 * cb + (l & 15);
      const float bet = sBeta[r], gam = sGam[r];
      f32x4 rv;
#pragma unroll
      for (int i = 0; i < 4; ++i) rv[i] = bet * (cvv[i] - gam * c[i]);
      store_tile(sRh, C::LDRP, 0, 16 * cb, rv);
    }
    f32x4 oacc = zero4();
    if (WANT_O) {
      mma_f32(oacc, RowMajor<float>{sSh, C::LDSP}, RowMajor<float>{sQ, C::LDK}, 0, 16 * cb, 0, DK);
      const float gam = sGam[16 * cb + (l & 15)];
#pragma unroll
      for (int i = 0; i < 4; ++i) oacc[i] *= gam;
      // P = M o Q K^T, lower 16x16 blocks (upper blocks written as zeros)
      for (int t = w; t < 16; t += NW) {
        const int bi = t >> 2, bj = t & 3;
        const int col = 16 * bj + (l & 15);
        const int rb = 16 * bi + 4 * (l >> 4);
        if (bj > bi) {
#pragma unroll
          for (int i = 0; i < 4; ++i) sP[(rb + i) * C::LDC + col] = 0.f;
          continue;
        }
        f32x4 c = zero4();
        mma_f32(c, RowMajor<float>{sQ, C::LDK}, RowMajor<float>{sK, C::LDK}, 16 * bi, 16 * bj, 0, DK);
        const float gc = sG[col];
        const f32x4 gr = *reinterpret_cast<const f32x4 *>(sG + rb);
#pragma unroll
        for (int i = 0; i < 4; ++i) sP[(rb + i) * C::LDC + col] = (col <= rb + i) ? __expf(gr[i] - gc) * c[i] : 0.f;
      }
    }
    lds_barrier();

    // ================= P2: D = R Tau^T =================
    {
      f32x4 c = zero4();
      const int rr = l & 15, kk = l >> 4;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (i < 4 * (cb + 1)) c = mfma_f32(sRh[rr * C::LDRP + 4 * i + kk], ctau[i >> 2][i & 3], c);
      }
      const float dec = sDec[16 * cb + (l & 15)];
      f32x4 cd;
#pragma unroll
      for (int i = 0; i < 4; ++i) cd[i] = c[i] * dec;
      if (WANT_O) store_tile(sDh, C::LDRP, 0, 16 * cb, c);
      store_tile(sDdh, C::LDRP, 0, 16 * cb, cd);
    }
    lds_barrier();

    // ================= P3: outputs; state update; stage the next chunk =================
    if (WANT_O) {
      const int kend = 16 * (cb + 1);
      mma_f32(oacc, RowMajor<float>{sDh, C::LDRP}, RowMajor<float>{sP, C::LDC}, 0, 16 * cb, 0, kend);
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
    {
      const float gl = sG[4 * CH];
#pragma unroll
      for (int u = 0; u < C::SPW; ++u) {
        const int ct = w + u * NW;
        if (ct < C::NST) {
#pragma unroll
          for (int i = 0; i < 4; ++i) sacc[u][i] *= gl;
          mma_f32(sacc[u], RowMajor<float>{sDdh, C::LDRP}, ColMajor<float>{sK, C::LDK}, 0, 16 * ct, 0, CH);
        }
      }
    }
    if (t0 + CH < tend) {
      // the state planes and the other K / gate buffer are free: every read
      // of them in this chunk happened before the P2 barrier
      store_state_planes();
      stage(kb ^ 1, min(CH, tend - t0 - CH));
      if (t0 + 2 * CH < tend) prefetch(t0 + 2 * CH, min(CH, tend - t0 - 2 * CH), slot + 2);
    }
    lds_barrier();
  }

  // ---------------- epilogue: final rows ----------------
  {
    float *out = is_T ? p.T_out : p.S_out;
    const int nrows = is_T ? DK : DV;
#pragma unroll
    for (int u = 0; u < C::SPW; ++u) {
      const int ct = w + u * NW;
      if (ct < C::NST) {
        const int col = 16 * ct + (l & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = row0 + 4 * (l >> 4) + i;
          out[(((int64_t)n * H + h) * nrows + r) * DK + col] = sacc[u][i];
        }
      }
    }
  }
}

template <int DK, bool WANT_O>
hipError_t launch_t(const ChainLaunch &p, hipStream_t stream) {
  const int64_t items = (int64_t)p.n_seqs * p.H * (p.tiles_T + p.tiles_S);
  if (items <= 0) return hipSuccess;
  const int64_t grid = (items + 7) / 8 * 8;
  return launch_kernel(chain_kernel<DK, WANT_O>, dim3((unsigned)grid), dim3(NT), 0, stream, p, (int)items);
}

template <int DK>
hipError_t launch_dk(const ChainLaunch &p, hipStream_t stream) {
  return p.o ? launch_t<DK, true>(p, stream) : launch_t<DK, false>(p, stream);
}

}  // namespace

hipError_t launch_chain(const ChainLaunch &p, hipStream_t stream) {
  if (p.in_bf16) return hipErrorInvalidValue;   // bf16 inputs: launch_chain_bf16
  if (p.dk == 64) return launch_dk<64>(p, stream);
  if (p.dk == 128) return launch_dk<128>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace gdn
