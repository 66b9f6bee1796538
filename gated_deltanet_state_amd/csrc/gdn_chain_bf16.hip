// gdn_chain_bf16.hip -- chunkwise Gated DeltaNet recurrence for bf16 inputs
// on gfx950: one wave per 16 state rows, all operands of a chunk in
// registers.
//
// The recurrence (page "Tail-Replay: Escaping the Curse of Linear Attention
// in Prefix Caching for Hybrid LLMs", section 2 Eq. (1); state S dv x dk):
//     S_t = S_{t-1} alpha_t (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,  o_t = S_t q_t.
// Over a chunk of L <= 64 tokens with cumulative log-gates g and the
// per-chunk factor Tau = (I + A)^{-1} (gdn_prep.hip), for the 16 state rows
// owned by a wave (transposed: tokens x rows):
//     Y = K S^T                        (64 x 16)
//     R = diag(beta) (V - diag(e^g) Y)
//     D = Tau R                        (per-token delta-rule corrections)
//     O = diag(e^g) Q S^T + (M o Q K^T) D,   M_rs = e^{g_r - g_s}, s <= r
//     S^T <- e^{g_L} S^T + K^T diag(e^{g_L - g}) D
//
// Register layout.  S^T (dk x 16) stays in registers as NSB C-layout 16 x 16
// blocks whose rows are a fixed permutation of dk: block d, lane group
// g = l >> 4, element e holds dk index 32 (d >> 1) + 8 g + 4 (d & 1) + e.
// With that order the pair of blocks (2m, 2m + 1) is, element for element,
// the B operand of the k = 32 MFMA over dk = 32m .. 32m + 31 in natural
// order, so K S^T takes K's A fragments straight from row-major K (one
// 16-byte read per fragment) and S^T never leaves the C layout.  Products
// over the token index pair two C-layout token blocks into one B operand
// with the permuted order {4g + e, 16 + 4g + e}; their A operands (Tau, and
// M o Q K^T) are stored in that order, and K^T comes from the gfx950
// transposing LDS read.
//
// Workgroup: NW waves = NW row tiles of one (sequence segment, head).  While
// chunk c runs from one LDS buffer set, the operands of chunk c + 1 are
// copied into the other one by load-to-LDS DMA (buffer_load ... lds; no
// registers, no staging code): K and Q as MFMA A fragments, the per-chunk
// record of gdn_prep.hip (Tau diag(beta) and K^T fragments), and the value
// columns of the workgroup.  Every fragment read is then a conflict-free
// 16-byte LDS read by lane.  One LDS barrier per chunk (two with outputs:
// M o Q K^T of the next chunk is built once its keys and queries landed).
//
// The same kernel builds the affine chunk operator of the page "LinearKV:
// One Cached State Suffices for Position-Independent Caching in Hybrid
// LLMs" (affine chunk operator paragraph): rows of the transition product
// T_C are rows of a "state" that starts as the identity and gets no value
// input.  Time-split replay runs the segments of a sequence as independent
// operators of this kind (composed afterwards by gdn_compose.hip).
//
// Precision: K, Q, V are exact in bf16; S, R, D, Tau and M o Q K^T are split
// into bf16 hi + lo where they enter a product (split-bfloat16), which keeps
// every product within a few fp32 ulps.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int CH = kChunk;

template <int DK, bool WANT_O, int NW>
struct Cfg {
  static constexpr int NT = NW * 64;
  static constexpr int NSB = DK / 16;          // 16-row blocks of S^T
  static constexpr int NKS = DK / 32;          // k = 32 steps over dk
  // LDS buffer set: 1 KiB blocks, one MFMA fragment (64 lanes x 16 bytes) each
  static constexpr int NKA = 4 * NKS;          // K (and Q) A fragments (bt, m)
  static constexpr int NKT = 2 * NSB;          // K^T fragments (d, m)
  static constexpr int NTF = 2 * kTauFrags;    // Tau diag(beta) fragments, hi then lo
  static constexpr int VU = 2 * NW;            // 16-byte units per staged value row
  static constexpr int NVB = CH * VU / 64;     // value slab blocks
  static constexpr int bKA = 0, bKT = NKA, bTF = bKT + NKT, bV = bTF + NTF, bQA = bV + NVB;
  static constexpr int NBLK = bQA + (WANT_O ? NKA : 0);
  static constexpr size_t BUF = (size_t)NBLK * 1024;
  static constexpr int GN = 3 * CH + 4;        // gate floats per buffer set
  static constexpr size_t oP = 2 * BUF;        // M o Q K^T fragments (outputs only)
  static constexpr size_t oG = oP + (WANT_O ? 2 * kTauFragPlane * 2 : 0);
  static constexpr size_t TOTAL = oG + 2 * GN * 4;
  static_assert(TOTAL <= 160 * 1024, "LDS budget");
};

// Gate buffer: [0, 64) e^g, [64, 128) e^{g_L - g} (0 past the chunk),
// [128, 192) g, [192] e^{g_L}.
constexpr int G_EG = 0, G_DEC = 64, G_G = 128, G_EGL = 192;

// Unit swizzle of the staged value slab: 16-byte unit u of row r sits at
// unit u ^ vswz(r), so that the 8 rows x 4 quads of a half-wave's
// transposing read fall in distinct banks.
template <int NW>
__device__ __forceinline__ int vswz(int r) {
  return NW == 8 ? 2 * (r & 7) : 2 * ((r >> 1) & 3);
}

template <int DK, bool WANT_O, int NW>
__global__ void __launch_bounds__(NW * 64, (WANT_O || NW == 4) ? 1 : 1) chain_bf16_kernel(ChainLaunch p, int n_items) {
  using C = Cfg<DK, WANT_O, NW>;
  __shared__ __attribute__((aligned(16))) char smem[C::TOTAL];
  bf16 *sP = reinterpret_cast<bf16 *>(smem + C::oP);
  float *sG0 = reinterpret_cast<float *>(smem + C::oG);

  // ---- work item (XCD-aware order: consecutive items share one XCD's L2) ----
  const int per = (int)(gridDim.x >> 3);
  const int item = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
  if (item >= n_items) return;
  const int tilesA = p.tiles_T + p.tiles_S;
  const int tiles0 = p.skip_T0 ? p.tiles_S : tilesA;
  const int grp0 = (tiles0 + NW - 1) / NW, grpA = (tilesA + NW - 1) / NW;
  const int per_nh = grp0 + (p.n_segs - 1) * grpA;
  const int nh = item / per_nh;
  int rem = item % per_nh, seg = 0, grp = rem;
  if (rem >= grp0) {
    rem -= grp0;
    seg = 1 + rem / grpA;
    grp = rem % grpA;
  }
  const int n = nh / p.H, h = nh % p.H;
  const int H = p.H, DV = p.dv;
  const int w = wave_id(), l = lane_id();
  const int g4 = l >> 4, jl = l & 15;
  const int tT = (seg == 0 && p.skip_T0) ? 0 : p.tiles_T;
  const int tile = grp * NW + w;
  const bool active = tile < tT + p.tiles_S;
  const bool is_T = active && tile < tT;
  const int row0 = is_T ? 16 * tile : 16 * (tile - tT);
  // tile counts are multiples of NW (launcher), so a workgroup holds either
  // transition tiles only or state tiles only; state workgroups stage the
  // value columns vcol0 .. vcol0 + 16 NW - 1
  const bool grp_S = grp * NW >= tT;
  const int vcol0 = 16 * (grp * NW - tT);

  // ---- this segment's token range ----
  const int cbeg = p.cu[n], cend = p.cu[n + 1];
  int64_t seg_len = cend - cbeg;
  if (p.n_segs > 1) seg_len = ((seg_len + p.n_segs - 1) / p.n_segs + CH - 1) / CH * CH;
  const int tbeg = (int)min((int64_t)cend, (int64_t)cbeg + seg * seg_len);
  const int tend = (int)min((int64_t)cend, (int64_t)tbeg + seg_len);
  const int64_t slot0 = (int64_t)(cbeg / CH) + n + (tbeg - cbeg) / CH;

  const bf16 *gk = reinterpret_cast<const bf16 *>(p.k);
  const bf16 *gq = reinterpret_cast<const bf16 *>(p.q);
  const bf16 *gv = reinterpret_cast<const bf16 *>(p.v);
  const unsigned short *ga = reinterpret_cast<const unsigned short *>(p.alpha);
  const char *grec = reinterpret_cast<const char *>(p.tau);

  // ---- S^T in registers (dk order of the header comment) ----
  f32x4 st[C::NSB];
#pragma unroll
  for (int d = 0; d < C::NSB; ++d) {
    const int c0 = 32 * (d >> 1) + 8 * g4 + 4 * (d & 1);
    st[d] = zero4();
    if (active) {
      if (is_T) {
#pragma unroll
        for (int e = 0; e < 4; ++e) st[d][e] = (row0 + jl == c0 + e) ? 1.f : 0.f;
      } else if (p.S0 && seg == 0) {
        st[d] = *reinterpret_cast<const f32x4 *>(p.S0 + (((int64_t)n * H + h) * DV + row0 + jl) * DK + c0);
      }
    }
  }

  // ---- DMA of one chunk's operands into buffer set b ----
  // Rows past the chunk are copies of its last row: they only meet zero
  // coefficients (beta = 0 in the Tau columns, zero K^T rows from the prep
  // kernel, masked M o Q K^T), so any finite value serves.
  auto issue_dma = [&](int b, int t0, int Lc, int64_t slot) {
    char *buf = smem + b * C::BUF;
    const char *rec = grec + (slot * H + h) * (int64_t)(kRecFloats * 4);
    for (int i = w; i < C::NBLK; i += NW) {
      lds_void *dst = (lds_void *)(buf + i * 1024);
      if (i < C::bKT || (WANT_O && i >= C::bQA)) {   // K or Q A fragment (bt, m)
        const int f = i < C::bKT ? i : i - C::bQA;
        const int bt = f / C::NKS, m = f % C::NKS;
        const int r = min(16 * bt + jl, Lc - 1);
        const bf16 *src = (i < C::bKT ? gk : gq) + ((int64_t)(t0 + r) * H + h) * DK + 32 * m + 8 * g4;
        dma16_global(src, dst);
      } else if (i < C::bTF) {                         // K^T fragments (record)
        dma16_global(rec + kRecKtOffsetBytes + (i - C::bKT) * 1024 + 16 * l, dst);
      } else if (i < C::bV) {                          // Tau diag(beta) fragments (record)
        dma16_global(rec + (i - C::bTF) * 1024 + 16 * l, dst);
      } else if (grp_S) {                              // value slab block
        const int u_lds = (i - C::bV) * 64 + l;
        const int r = u_lds / C::VU, u = (u_lds % C::VU) ^ vswz<NW>(r);
        dma16_global(gv + ((int64_t)(t0 + min(r, Lc - 1)) * H + h) * DV + vcol0 + 8 * u, dst);
      }
    }
  };

  unsigned short pa = 0x3f80;   // wave 0: alpha bits of token t0 + l (1.0 past the end)
  auto load_alpha = [&](int t0, int Lc) {
    pa = 0x3f80;
    if (w == 0 && l < Lc) pa = ga[(int64_t)(t0 + l) * H + h];
  };
  auto gates = [&](int b, int Lc) {
    if (w != 0) return;
    float *sG = sG0 + b * C::GN;
    const float g = wave_inclusive_scan((l < Lc) ? logf(__uint_as_float((unsigned)pa << 16)) : 0.f);
    const float gL = lane_value(g, Lc - 1);
    sG[G_EG + l] = __expf(g);
    sG[G_DEC + l] = (l < Lc) ? __expf(gL - g) : 0.f;
    sG[G_G + l] = g;
    if (l == 0) sG[G_EGL] = __expf(gL);
  };

  // M o Q K^T of the chunk in buffer set b, as split-bf16 A fragments in the
  // Tau fragment order (gdn_internal.h): tile (bi, bj) of 16 x 16 lands in
  // fragment (bi, bj >> 1), lane (r & 15) + 16 (c' >> 2), element
  // 4 (bj & 1) + (c' & 3) for row r, column 16 bj + c'.
  auto build_p = [&](int b) {
    const char *buf = smem + b * C::BUF;
    const float *sG = sG0 + b * C::GN;
    for (int t = w; t < 2 * kTauFrags; t += NW) {
      const int f = t >> 1, half = t & 1;
      const int bi = f < 2 ? f : (f - 2) / 2 + 2;
      const int bj = 2 * (f < 2 ? 0 : (f - 2) % 2) + half;
      f32x4 c = zero4();
      if (bj <= bi) {
#pragma unroll
        for (int m = 0; m < C::NKS; ++m) {
          const bf16x8 a = *reinterpret_cast<const bf16x8 *>(buf + (C::bQA + bi * C::NKS + m) * 1024 + 16 * l);
          const bf16x8 bb = *reinterpret_cast<const bf16x8 *>(buf + (C::bKA + bj * C::NKS + m) * 1024 + 16 * l);
          c = mfma_bf16(a, bb, c);
        }
      }
      const int col = 16 * bj + jl;
      const float gc = sG[G_G + col];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * bi + 4 * g4 + e;
        const float x = (col <= r) ? __expf(sG[G_G + r] - gc) * c[e] : 0.f;
        const bf16 hi = (bf16)x;
        const int idx = (f * 64 + (r & 15) + 16 * (jl >> 2)) * 8 + 4 * half + (jl & 3);
        sP[idx] = hi;
        sP[kTauFragPlane + idx] = (bf16)(x - (float)hi);
      }
    }
  };

  // Value columns of the staged chunk in buffer set b, transposed to the
  // C layout of R (lane: column row0 + jl, tokens 16 bt + 4 g4 + e).  The
  // transposing read carries no alias information, so a read issued while
  // a load-to-LDS copy is in flight would make the compiler wait for that
  // copy; the values are therefore read right after each hand-over
  // barrier, before the next copies are issued, and kept in registers.
  // The read is issued by every wave with all lanes on: a transposing read
  // under a partial or empty EXEC mask still writes its destination (the
  // data of a lane comes from other lanes' addresses).  Transition tiles,
  // whose workgroups stage no values, clear the result with a mask.
  uint2 vt[4];
  const uint32_t vmask = (active && !is_T) ? 0xffffffffu : 0u;
  auto read_v = [&](int b) {
    const char *buf = smem + b * C::BUF;
#pragma unroll
    for (int bt = 0; bt < 4; ++bt) {
      const int rr0 = 16 * bt + 4 * g4 + (jl >> 2);
      const int u = 2 * (w & (NW - 1)) + ((jl & 3) >> 1);
      const uint2 x = ds_read_tr16(reinterpret_cast<const bf16 *>(
          buf + C::bV * 1024 + rr0 * (C::VU * 16) + 16 * (u ^ vswz<NW>(rr0)) + 8 * (jl & 1)));
      vt[bt] = uint2{x.x & vmask, x.y & vmask};
    }
  };

  if (tbeg < tend) {
    const int L0 = min(CH, tend - tbeg);
    issue_dma(0, tbeg, L0, slot0);
    load_alpha(tbeg, L0);
    gates(0, L0);
  }
  wait_vmem();
  lds_barrier();
  if (WANT_O && tbeg < tend) {
    build_p(0);
    lds_barrier();
  }
  read_v(0);

  // Outputs of a chunk are stored at the start of the next one, so that
  // the hand-over wait (which also counts stores) finds them complete.
  f32x4 zp[4];
  int tp = 0, Lp = 0;
  auto store_o = [&]() {
#pragma unroll
    for (int bt = 0; bt < 4; ++bt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * bt + 4 * g4 + e;
        if (r < Lp) {
          const int64_t oi = ((int64_t)(tp + r) * H + h) * DV + row0 + jl;
          if (p.o_bf16)
            reinterpret_cast<bf16 *>(p.o)[oi] = (bf16)zp[bt][e];
          else
            reinterpret_cast<float *>(p.o)[oi] = zp[bt][e];
        }
      }
    Lp = 0;
  };

  int64_t slot = slot0;
  int b = 0;
  for (int t0 = tbeg; t0 < tend; t0 += CH, ++slot, b ^= 1) {
    const int Lc = min(CH, tend - t0);
    const bool more = t0 + CH < tend;
    const int L1 = more ? min(CH, tend - t0 - CH) : 0;
    if (WANT_O && active && Lp > 0) store_o();
    // operands of the next chunk: in flight while this one runs
    if (more) {
      issue_dma(b ^ 1, t0 + CH, L1, slot + 1);
      load_alpha(t0 + CH, L1);
    }
    const char *buf = smem + b * C::BUF;
    const float *sG = sG0 + b * C::GN;
    auto frag = [&](int blk) { return *reinterpret_cast<const bf16x8 *>(buf + blk * 1024 + 16 * l); };

    if (active) {
      // ---- S^T as k = 32 B fragments ----
      bf16x8 sh[C::NKS], sl[C::NKS];
#pragma unroll
      for (int m = 0; m < C::NKS; ++m) b_frag_split(st[2 * m], st[2 * m + 1], sh[m], sl[m]);

      // ---- Y = K S^T ----
      f32x4 y[4];
#pragma unroll
      for (int bt = 0; bt < 4; ++bt) y[bt] = zero4();
#pragma unroll
      for (int m = 0; m < C::NKS; ++m)
#pragma unroll
        for (int bt = 0; bt < 4; ++bt) {
          const bf16x8 a = frag(C::bKA + bt * C::NKS + m);
          y[bt] = mfma_bf16(a, sh[m], y[bt]);
          y[bt] = mfma_bf16(a, sl[m], y[bt]);
        }

      // ---- R = V - e^g Y  (beta is folded into the Tau fragments) ----
      f32x4 rr[4];
#pragma unroll
      for (int bt = 0; bt < 4; ++bt) {
        const f32x4 eg = *reinterpret_cast<const f32x4 *>(sG + G_EG + 16 * bt + 4 * g4);
        const float vv[4] = {__uint_as_float(vt[bt].x << 16), __uint_as_float(vt[bt].x & 0xffff0000u),
                             __uint_as_float(vt[bt].y << 16), __uint_as_float(vt[bt].y & 0xffff0000u)};
#pragma unroll
        for (int e = 0; e < 4; ++e) rr[bt][e] = vv[e] - eg[e] * y[bt][e];
      }
      bf16x8 rh[2], rl[2];
      b_frag_split(rr[0], rr[1], rh[0], rl[0]);
      b_frag_split(rr[2], rr[3], rh[1], rl[1]);

      // ---- D = (Tau diag(beta)) R  (f: (bt, m) = (0,0),(1,0),(2,0),(2,1),(3,0),(3,1)) ----
      f32x4 dd[4];
#pragma unroll
      for (int bt = 0; bt < 4; ++bt) dd[bt] = zero4();
#pragma unroll
      for (int f = 0; f < kTauFrags; ++f) {
        const int bt = f < 2 ? f : (f - 2) / 2 + 2;
        const int m = f < 2 ? 0 : (f - 2) % 2;
        const bf16x8 th = frag(C::bTF + f), tl = frag(C::bTF + kTauFrags + f);
        dd[bt] = mfma_bf16(th, rh[m], dd[bt]);
        dd[bt] = mfma_bf16(th, rl[m], dd[bt]);
        dd[bt] = mfma_bf16(tl, rh[m], dd[bt]);
      }

      // ---- O = e^g Q S^T + (M o Q K^T) D ----
      if (WANT_O) {
        bf16x8 dh[2], dl[2];
        b_frag_split(dd[0], dd[1], dh[0], dl[0]);
        b_frag_split(dd[2], dd[3], dh[1], dl[1]);
        f32x4 z[4];
#pragma unroll
        for (int bt = 0; bt < 4; ++bt) z[bt] = zero4();
#pragma unroll
        for (int m = 0; m < C::NKS; ++m)
#pragma unroll
          for (int bt = 0; bt < 4; ++bt) {
            const bf16x8 a = frag(C::bQA + bt * C::NKS + m);
            z[bt] = mfma_bf16(a, sh[m], z[bt]);
            z[bt] = mfma_bf16(a, sl[m], z[bt]);
          }
#pragma unroll
        for (int bt = 0; bt < 4; ++bt) {
          const f32x4 eg = *reinterpret_cast<const f32x4 *>(sG + G_EG + 16 * bt + 4 * g4);
#pragma unroll
          for (int e = 0; e < 4; ++e) z[bt][e] *= eg[e];
        }
#pragma unroll
        for (int f = 0; f < kTauFrags; ++f) {
          const int bt = f < 2 ? f : (f - 2) / 2 + 2;
          const int m = f < 2 ? 0 : (f - 2) % 2;
          const bf16x8 ph = *reinterpret_cast<const bf16x8 *>(sP + (f * 64 + l) * 8);
          const bf16x8 pl = *reinterpret_cast<const bf16x8 *>(sP + kTauFragPlane + (f * 64 + l) * 8);
          z[bt] = mfma_bf16(ph, dh[m], z[bt]);
          z[bt] = mfma_bf16(ph, dl[m], z[bt]);
          z[bt] = mfma_bf16(pl, dh[m], z[bt]);
        }
#pragma unroll
        for (int bt = 0; bt < 4; ++bt) zp[bt] = z[bt];
        tp = t0;
        Lp = Lc;
      }

      // ---- S^T <- e^{g_L} S^T + K^T diag(e^{g_L - g}) D ----
      bf16x8 eh[2], el[2];
      {
        f32x4 de[4];
#pragma unroll
        for (int bt = 0; bt < 4; ++bt) {
          const f32x4 dec = *reinterpret_cast<const f32x4 *>(sG + G_DEC + 16 * bt + 4 * g4);
#pragma unroll
          for (int e = 0; e < 4; ++e) de[bt][e] = dd[bt][e] * dec[e];
        }
        b_frag_split(de[0], de[1], eh[0], el[0]);
        b_frag_split(de[2], de[3], eh[1], el[1]);
      }
      const float gl = sG[G_EGL];
#pragma unroll
      for (int d = 0; d < C::NSB; ++d) {
        f32x4 c = st[d];
#pragma unroll
        for (int e = 0; e < 4; ++e) c[e] *= gl;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const bf16x8 a = frag(C::bKT + 2 * d + m);
          c = mfma_bf16(a, eh[m], c);
          c = mfma_bf16(a, el[m], c);
        }
        st[d] = c;
      }
    }

    // ---- hand over to the next chunk ----
    if (more) gates(b ^ 1, L1);
    wait_vmem();
    lds_barrier();
    if (WANT_O && more) {
      build_p(b ^ 1);
      lds_barrier();
    }
    if (more) read_v(b ^ 1);
  }

  // ---------------- epilogue: final rows ----------------
  if (WANT_O && active && Lp > 0) store_o();
  if (active) {
    const int64_t unit = ((int64_t)n * p.n_segs + seg) * H + h;
#pragma unroll
    for (int d = 0; d < C::NSB; ++d) {
      const int c0 = 32 * (d >> 1) + 8 * g4 + 4 * (d & 1);
      if (is_T) {
        float *out = p.T_out + unit * DK * DK;
        if (p.T_transposed) {
#pragma unroll
          for (int e = 0; e < 4; ++e) out[(int64_t)(c0 + e) * DK + row0 + jl] = st[d][e];
        } else {
          *reinterpret_cast<f32x4 *>(out + (int64_t)(row0 + jl) * DK + c0) = st[d];
        }
      } else {
        *reinterpret_cast<f32x4 *>(p.S_out + unit * DV * DK + (int64_t)(row0 + jl) * DK + c0) = st[d];
      }
    }
  }
}

template <int DK, bool WANT_O, int NW>
hipError_t launch_b(const ChainLaunch &p, hipStream_t stream) {
  const int tilesA = p.tiles_T + p.tiles_S;
  const int tiles0 = p.skip_T0 ? p.tiles_S : tilesA;
  const int64_t per_nh = (tiles0 + NW - 1) / NW + (int64_t)(p.n_segs - 1) * ((tilesA + NW - 1) / NW);
  const int64_t items = (int64_t)p.n_seqs * p.H * per_nh;
  if (items <= 0) return hipSuccess;
  const int64_t grid = (items + 7) / 8 * 8;
  hipLaunchKernelGGL((chain_bf16_kernel<DK, WANT_O, NW>), dim3((unsigned)grid), dim3(NW * 64), 0, stream, p,
                     (int)items);
  return hipGetLastError();
}

template <int DK>
hipError_t launch_dk(const ChainLaunch &p, hipStream_t stream) {
  // eight waves per workgroup when every tile count is a multiple of eight
  // (the operands of a chunk are then shared by eight row tiles)
  const bool eight = p.tiles_S % 8 == 0 && p.tiles_T % 8 == 0;
  if (p.o) return launch_b<DK, true, 4>(p, stream);
  return eight ? launch_b<DK, false, 8>(p, stream) : launch_b<DK, false, 4>(p, stream);
}

}  // namespace

hipError_t launch_chain_bf16(const ChainLaunch &p, hipStream_t stream) {
  if (p.n_segs < 1 || p.tiles_S % 4 != 0 || p.tiles_T % 4 != 0) return hipErrorInvalidValue;
  if (p.dk == 64) return launch_dk<64>(p, stream);
  if (p.dk == 128) return launch_dk<128>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace gdn
