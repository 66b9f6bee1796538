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
// Workgroup: NW waves, each owning RT (one or two) row tiles of one
// (sequence segment, head); with two, every fragment read from LDS feeds
// the products of both tiles.  While
// chunk c runs from one LDS buffer set, the operands of chunk c + 1 are
// copied into the other one by load-to-LDS DMA (buffer_load ... lds; no
// registers, no staging code): K and Q as MFMA A fragments, the Tau
// diag(beta) fragments of the per-chunk record of gdn_prep_wave.h, and the
// value columns of the workgroup; K^T fragments come from the staged keys
// by the transposing LDS read.  Every fragment read is then a
// conflict-free 16-byte LDS read by lane.  With outputs, the waves also
// build the chunk's M o Q K^T from the staged Q and K.  One LDS barrier per
// chunk.
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
#include "gdn_prep_wave.h"

namespace gdn {

namespace {

constexpr int CH = kChunk;

template <int DK, bool WANT_O, int NW, int RT, bool FUSED>
struct Cfg {
  static constexpr int NT = NW * 64;
  static constexpr int TW = NW * RT;           // row tiles per workgroup
  static constexpr int NSB = DK / 16;          // 16-row blocks of S^T
  static constexpr int NKS = DK / 32;          // k = 32 steps over dk
  // LDS buffer set: 1 KiB blocks, one MFMA fragment (64 lanes x 16 bytes) each
  static constexpr int NKA = 4 * NKS;          // K (and Q) A fragments (bt, m)
  static constexpr int NTF = 2 * kTauFrags;    // Tau diag(beta) fragments, hi then lo
  static constexpr int NSV = TW < 8 ? TW : 8;  // state tiles a workgroup can hold (dv <= 128)
  static constexpr int VU = 2 * NSV;           // 16-byte units per staged value row
  static constexpr int NVB = CH * VU / 64;     // value slab blocks
  static constexpr int bKA = 0, bTF = NKA, bV = bTF + NTF, bQA = bV + NVB;
  static constexpr int NBLK = bQA + (WANT_O ? NKA : 0);
  static constexpr size_t BUF = (size_t)NBLK * 1024;
  static constexpr int GN = 6 * CH + 4;        // gate floats per buffer set
  static constexpr size_t oG = 2 * BUF;
  // outputs: M o Q K^T of two chunks as split-bf16 fragments (hi, lo planes)
  static constexpr size_t PSET = (size_t)2 * kTauFragPlane * 2;
  static constexpr size_t oP = oG + 2 * GN * 4;
  static constexpr size_t TOTAL = oP + (WANT_O ? 2 * PSET : 0);
  // the prologue that builds the segment's records (on at most eight
  // waves) uses the LDS above buffer set 0, whose first chunk is in flight
  // meanwhile
  static constexpr int NPW = NW < 8 ? NW : 8;
  static constexpr size_t PSCR = BUF;
  static constexpr size_t SMEM =
      FUSED && PSCR + (size_t)NPW * kPrepWaveLds > TOTAL ? PSCR + (size_t)NPW * kPrepWaveLds : TOTAL;
  static_assert(SMEM <= 160 * 1024, "LDS budget");
};

// Gate buffer (see the running scale gam in the kernel), per token: [0, 64)
// gam e^g / |k| (the state read by the keys), [64, 128) e^{g_L - g} / gam' /
// |k| (0 past the chunk), [128, 192) g, [192, 256) gam e^g (the state read
// by the queries), [256, 320) 1 / |q| (raw inputs with outputs: formed from
// the staged queries during the chunk's own step and applied to its output
// rows when they are stored), [320, 384) 1 / |k|; [384] the factor the chunk
// applies to the state registers (gam e^{g_L}, or 1: none).  The key norms
// are 1 except for raw inputs (ChainLaunch::raw).
constexpr int G_EG = 0, G_DEC = 64, G_G = 128, G_EQ = 192, G_RQ = 256, G_RK = 320, G_EGL = 384;

// Unit swizzle of the staged value slab (VU 16-byte units per row): unit u
// of row r sits at unit u ^ vswz(r), so that the 8 rows x 4 quads of a
// half-wave's transposing read fall in distinct banks.
template <int VU>
__device__ __forceinline__ int vswz(int r) {
  return VU == 16 ? 2 * (r & 7) : 2 * ((r >> 1) & 3);
}

// K^T fragments of the state update S^T += K^T D' for token half m, all
// NSB dk blocks d, read from the staged K A-fragments (fragment (bt, ks) at
// (bt NKS + ks) KiB, lane (r & 15) + 16 ((c >> 3) & 3) holding key row r,
// columns c .. c + 7 of its 32-column step) by the transposing LDS read:
// fragment (d, m), lane (q, g) gets K[32 m + 4 g + e (+16)][32 (d >> 1) +
// 8 (q >> 2) + 4 (d & 1) + (q & 3)], e < 4 -- the dk order of the S^T blocks
// and the token order of the paired right-hand sides.  Inline assembly, one
// group of reads per token half with its own lgkmcnt wait (one LDS round
// trip per half): the transposing read carries no alias information,
// and as a compiler builtin it would be made to wait for the load-to-LDS
// copies of the next chunk that are in flight meanwhile.  The results are
// early-clobber operands: a read's data may land before the next read of
// the group has taken its address, so no result may share a register with
// the address.
template <int NKS, int NSB>
__device__ __forceinline__ void kt_frags(int m, uint32_t addr, bf16x8 (&a)[NSB]) {
  // all NSB fragments of token half m in one group, one wait: fragment d
  // from the 8-byte reads at (d >> 1) KiB + 8 (d & 1) and that plus NKS KiB
  // (the next 16 key rows)
  static_assert((NKS == 4 && NSB == 8) || (NKS == 2 && NSB == 4), "dk = 128 or 64");
  const uint32_t base = addr + (uint32_t)(2 * m * NKS * 1024);
  uint2 r[2 * NSB];
  if constexpr (NSB == 8) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %16 offset:0\n\t"
        "ds_read_b64_tr_b16 %1, %16 offset:4096\n\t"
        "ds_read_b64_tr_b16 %2, %16 offset:8\n\t"
        "ds_read_b64_tr_b16 %3, %16 offset:4104\n\t"
        "ds_read_b64_tr_b16 %4, %16 offset:1024\n\t"
        "ds_read_b64_tr_b16 %5, %16 offset:5120\n\t"
        "ds_read_b64_tr_b16 %6, %16 offset:1032\n\t"
        "ds_read_b64_tr_b16 %7, %16 offset:5128\n\t"
        "ds_read_b64_tr_b16 %8, %16 offset:2048\n\t"
        "ds_read_b64_tr_b16 %9, %16 offset:6144\n\t"
        "ds_read_b64_tr_b16 %10, %16 offset:2056\n\t"
        "ds_read_b64_tr_b16 %11, %16 offset:6152\n\t"
        "ds_read_b64_tr_b16 %12, %16 offset:3072\n\t"
        "ds_read_b64_tr_b16 %13, %16 offset:7168\n\t"
        "ds_read_b64_tr_b16 %14, %16 offset:3080\n\t"
        "ds_read_b64_tr_b16 %15, %16 offset:7176\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7]),
          "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]), "=&v"(r[12]), "=&v"(r[13]), "=&v"(r[14]),
          "=&v"(r[15])
        : "v"(base));
  } else {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8 offset:0\n\t"
        "ds_read_b64_tr_b16 %1, %8 offset:2048\n\t"
        "ds_read_b64_tr_b16 %2, %8 offset:8\n\t"
        "ds_read_b64_tr_b16 %3, %8 offset:2056\n\t"
        "ds_read_b64_tr_b16 %4, %8 offset:1024\n\t"
        "ds_read_b64_tr_b16 %5, %8 offset:3072\n\t"
        "ds_read_b64_tr_b16 %6, %8 offset:1032\n\t"
        "ds_read_b64_tr_b16 %7, %8 offset:3080\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
        : "v"(base));
  }
#pragma unroll
  for (int d = 0; d < NSB; ++d) a[d] = cat_bf16x8(r[2 * d], r[2 * d + 1]);
}

// Segments of whole chunks: chunks [cb, cb + cl) of segment seg of a
// sequence of nch chunks, cut into P = n_segs segments.
//   * Plain layout: segment 0 carries state rows only (no transition rows)
//     and steps about 1.6 times faster, so it takes a larger share:
//     e = round(chunks / (P - 1 + 1.6)) chunks for each later segment, the
//     rest for segment 0.  When the workgroups build their own records
//     first (fused), segment 0 keeps to one record per prologue wave
//     (npw; a second round of the prologue costs more than a chunk step
//     elsewhere) and the later segments take ceil(rest / (P - 1)) each.
//   * Lead layout (time split with outputs): the later segments, which all
//     run the output recurrence from their composed start states, take e =
//     round(chunks / P) each and the lead the rest.  The lead runs its
//     outputs beside the transition segments, which also build the last
//     segment's records (lead_extras).  (32768-token prefill: leads of
//     0.75, 0.875, 1.125 and 1.25 times e took 1.7%, 0.6%, 2.2% and 5.8%
//     longer than e; with the lead building the last segment's records
//     itself, 0.75 e was best.)
// Segments past the end are empty.
__device__ __forceinline__ void seg_chunks(const ChainLaunch &p, int nch, int seg, int npw, int &cb, int &cl) {
  const int P = p.n_segs;
  int e, c0;
  if (p.lead) {
    e = max(1, (nch + P / 2) / P);
    c0 = max(0, nch - (P - 1) * e);
  } else {
    const int den = 5 * (P - 1) + 8;
    e = max(1, (5 * nch + den / 2) / den);
    c0 = max(0, nch - (P - 1) * e);
    if (npw > 0 && c0 > npw) {
      c0 = npw;
      e = (nch - c0 + P - 2) / (P - 1);
    }
  }
  cb = seg == 0 ? 0 : c0 + (seg - 1) * e;
  cl = seg == 0 ? c0 : e;
  cb = min(cb, nch);
  cl = min(cl, nch - cb);
}

// Lead layout: the records of the last segment (which the segment launch
// does not run) that segment seg builds in its prologue, chunks xb .. xb +
// nx - 1 of the sequence: an equal share for each transition segment
// 1 .. P - 2, or all of them for the lead when there is none.
__device__ __forceinline__ void lead_extras(const ChainLaunch &p, int nch, int seg, int &xb, int &nx) {
  const int P = p.n_segs;
  int lb, ln;
  seg_chunks(p, nch, P - 1, 0, lb, ln);
  xb = lb;
  nx = 0;
  if (P == 2) {
    if (seg == 0) nx = ln;
    return;
  }
  if (seg == 0) return;
  const int q = (ln + P - 3) / (P - 2);
  xb = lb + min(ln, (seg - 1) * q);
  nx = min(q, lb + ln - xb);
}

// Workgroups of one (sequence, head) in a launch: the segments first ..
// first + count - 1, grp0 workgroups for segment 0 (when it runs; tw0 row
// tiles each) and grpA for every later one (tw row tiles each).
struct SegGroups {
  int first, count, grp0, grpA, per_nh;
};
__host__ __device__ inline SegGroups seg_groups(const ChainLaunch &p, int tw, int tw0) {
  SegGroups g;
  const int tilesA = p.tiles_T + p.tiles_S;
  const int tiles0 = p.skip_T0 ? p.tiles_S : tilesA;
  g.first = (p.lead && p.tiles_T == 0) ? 1 : 0;
  g.count = p.lead ? p.n_segs - 1 : p.n_segs;
  g.grp0 = g.first == 0 ? (tiles0 + tw0 - 1) / tw0 : 0;
  g.grpA = (tilesA + tw - 1) / tw;
  g.per_nh = g.grp0 + (g.count - (g.first == 0 ? 1 : 0)) * g.grpA;
  return g;
}

// One workgroup: row-tile group grp of segment seg of (sequence n, head h).
// QN (with outputs of raw inputs, ChainLaunch::raw): the query norms are
// formed from the staged queries and applied to the stored output rows.
// MULTI (chunk operators without a time split, state and transition rows in
// one workgroup per (sequence, head)): the workgroup runs the items it ..
// it_end - 1 (item i: sequence i / H, head i % H) as one stream of chunks.
// Its prologue writes the operators of the empty items (identity, zero)
// and builds the records of all the others; the copies of an item's first
// chunk go out during the previous item's last chunk, whose operator is
// written as the registers start over.
template <int DK, bool WANT_O, int NW, int RT, bool FUSED, bool QN = false, bool MULTI = false>
__device__ __forceinline__ void chain_body(const ChainLaunch &p, int n, int h, const int seg, const int grp,
                                           char *smem, int it = 0, const int it_end = 0) {
  static_assert(!MULTI || (FUSED && !WANT_O), "item streams: chunk operators only");
  static_assert(RT == 1 || RT == 2, "one or two row tiles per wave");
  using C = Cfg<DK, WANT_O, NW, RT, FUSED>;
  constexpr int TW = C::TW;
  float *sG0 = reinterpret_cast<float *>(smem + C::oG);
  const int H = p.H, DV = p.dv;
  const int w = __builtin_amdgcn_readfirstlane(wave_id()), l = lane_id();
  const int g4 = l >> 4, jl = l & 15;
  const int tT = (seg == 0 && p.skip_T0) ? 0 : p.tiles_T;
  // wave w owns row tiles tile .. tile + RT - 1, all of one kind (the
  // launcher makes both tile counts multiples of RT)
  const int tile = grp * TW + w * RT;
  const bool active = tile < tT + p.tiles_S;
  const bool is_T = active && tile < tT;
  const int row0 = is_T ? 16 * tile : 16 * (tile - tT);  // first row; tile rt adds 16 rt
  // state tiles of this workgroup: sfirst .. sfirst + nS - 1 (at most NSV;
  // the launcher keeps transition and state tiles of a segment in one
  // workgroup or makes tile counts multiples of NW); the workgroup stages
  // the value columns vcol0 .. vcol0 + 16 nS - 1
  const int s_lo = max(grp * TW, tT), s_hi = min(grp * TW + TW, tT + p.tiles_S);
  const bool grp_S = s_hi > s_lo;
  const int sfirst = s_lo - tT, nS = s_hi - s_lo;
  const int vcol0 = 16 * sfirst;

  // MULTI: this lane's first operator element of item (n2, h2) (row row0 +
  // jl, column 8 g4); element (rt, d, e) sits 16 rt DK + 32 (d >> 1) + 4 (d & 1)
  // + e floats on
  auto op_base = [&](int n2, int h2) {
    const int64_t u2 = (int64_t)n2 * H + h2;
    return (is_T ? p.T_out + u2 * DK * DK : p.S_out + u2 * DV * DK) + (int64_t)(row0 + jl) * DK + 8 * g4;
  };
  auto op_off = [](int rt, int d) { return 16 * rt * DK + 32 * (d >> 1) + 4 * (d & 1); };
  auto start_value = [&](int rt, int d, int e) {   // identity transition rows, zero state rows
    const int c0 = 32 * (d >> 1) + 8 * g4 + 4 * (d & 1), r = row0 + 16 * rt + jl;
    return (is_T && r == c0 + e) ? 1.f : 0.f;
  };
  if constexpr (MULTI) {
    // the operators of the empty items (identity, zero) first
    for (int i2 = it; i2 < it_end; ++i2) {
      if (!active || p.cu[i2 / H + 1] > p.cu[i2 / H]) continue;
      float *ob = op_base(i2 / H, i2 % H);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int d = 0; d < C::NSB; ++d)
          *reinterpret_cast<f32x4 *>(ob + op_off(rt, d)) =
              f32x4{start_value(rt, d, 0), start_value(rt, d, 1), start_value(rt, d, 2), start_value(rt, d, 3)};
    }
    while (it < it_end && p.cu[it / H + 1] == p.cu[it / H]) ++it;
    if (it >= it_end) return;
    n = it / H;
    h = it % H;
  }
  int hn = h;   // head of the chunk being staged (MULTI: the next item's, near an item's end)

  // ---- this segment's token range ----
  const int cbeg = p.cu[n], cend = p.cu[n + 1];
  const int nch_seq = (cend - cbeg + CH - 1) / CH;
  int tbeg = cbeg, tend = cend;
  if (p.n_segs > 1) {
    int cb, cl;
    seg_chunks(p, nch_seq, seg, FUSED ? C::NPW : 0, cb, cl);
    tbeg = cbeg + cb * CH;
    tend = min(cend, tbeg + cl * CH);
  }
  const int64_t slot0 = (int64_t)(cbeg / CH) + n + (tbeg - cbeg) / CH;

  // Staged K and Q fragments.  Element (row r, 8-column group g) of a 1 KiB
  // fragment block -- lane r + 16 g of the MFMA A operand -- sits in 16-byte
  // slot 16 g + (r ^ 12 (g & 1)) (kq_slot).  A 16-byte read by lane services
  // each half-wave in two passes of 16 lanes, the quads whose index has even,
  // then odd, bit parity; with this order each pass meets 16 distinct
  // 16-byte bank groups, as in the plain order.  The transposing 8-byte
  // reads of K^T service 32 lanes at once and read the same half of 32
  // slots: in the plain order those fall on 8 bank groups (4-way conflicts),
  // in this one on 16 (2-way, the least for same-half reads).  (Lane grouping
  // and conflict counts measured with SQ_LDS_BANK_CONFLICT on MI355X.)
  auto kq_slot = [](int r, int g) { return 16 * g + (r ^ (12 * (g & 1))); };
  const int kq_l = kq_slot(jl, g4);   // this lane's own slot (A operand reads)
  // LDS byte address (buffer set 0) of this lane's transposing reads of the
  // staged keys: key row 4 g + (jl >> 2) of a 16-row block, 8-column group
  // jl & 3 (see kt_frags)
  const uint32_t kt_lds = (uint32_t)(uintptr_t)(lds_void *)(smem + C::bKA * 1024) +
                          16u * (uint32_t)kq_slot(4 * g4 + (jl >> 2), jl & 3);
  const bf16 *gk = reinterpret_cast<const bf16 *>(p.k);
  const bf16 *gq = reinterpret_cast<const bf16 *>(p.q);
  const bf16 *gv = reinterpret_cast<const bf16 *>(p.v);
  const unsigned short *ga = reinterpret_cast<const unsigned short *>(p.alpha);
  const char *grec = reinterpret_cast<const char *>(p.tau);

  // ---- S^T in registers (dk order of the header comment) ----
  // Transition rows start at the identity; state rows at the segment's start
  // state, S0 (segment 0) or zero.  The start state's loads sit in one
  // branch, so they are issued together and waited for once (a branch per
  // load made the compiler wait for each load before issuing the next).
  f32x4 st[RT][C::NSB];
  const float *s_src = nullptr;
  if (active && !is_T) {
    if (p.S0_seg)
      s_src = p.S0_seg + (((int64_t)n * p.n_segs + seg) * H + h) * DV * DK;
    else if (p.S0 && seg == 0)
      s_src = p.S0 + ((int64_t)n * H + h) * DV * DK;
  }
  if (s_src) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int d = 0; d < C::NSB; ++d) {
        const int c0 = 32 * (d >> 1) + 8 * g4 + 4 * (d & 1), r = row0 + 16 * rt + jl;
        st[rt][d] = *reinterpret_cast<const f32x4 *>(s_src + (int64_t)r * DK + c0);
      }
  } else {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int d = 0; d < C::NSB; ++d) {
        const int c0 = 32 * (d >> 1) + 8 * g4 + 4 * (d & 1), r = row0 + 16 * rt + jl;
#pragma unroll
        for (int e = 0; e < 4; ++e) st[rt][d][e] = (is_T && r == c0 + e) ? 1.f : 0.f;
      }
  }

  // ---- DMA of one chunk's operands into buffer set b ----
  // Every wave issues whole 1 KiB blocks (one 16-byte copy per lane); the
  // loops are unrolled over compile-time block ranges with the wave index
  // uniform, so the issue is straight-line scalar-branch code.  The copies
  // go through buffer descriptors whose base is the chunk's first token (a
  // uniform address, rebuilt per chunk by scalar code) and whose range ends
  // with the tensor, so each lane's byte offset is fixed for the whole
  // sequence.  Rows past a short chunk read the tokens that follow it, or
  // zeros past the end of the tensor: they only meet zero coefficients
  // (beta = 0 in the Tau columns, zero decayed corrections in the state
  // update, masked M o Q K^T entries, outputs past the chunk not stored),
  // so any finite value serves.
  const uint32_t tok_k = (uint32_t)H * DK * 2, tok_v = (uint32_t)H * DV * 2;  // bytes per token
  const int64_t T_all = p.cu[p.n_seqs];
  constexpr int JK = (C::NKA + NW - 1) / NW, JT = (C::NTF + NW - 1) / NW, JV = (C::NVB + NW - 1) / NW;
  uint32_t off_kq[JK], off_v[JV];
#pragma unroll
  for (int j = 0; j < JK; ++j) {                 // K (and Q) A fragment (bt, m): slot l holds key row
    const int f = j * NW + w, bt = f / C::NKS, m = f % C::NKS;   // 16 bt + r, group g with kq_slot(r, g) = l
    off_kq[j] = (uint32_t)(16 * bt + (jl ^ (12 * (g4 & 1)))) * tok_k + 64 * m + 16 * g4;
  }
#pragma unroll
  for (int j = 0; j < JV; ++j) {                 // value slab: logical unit u (8 columns) of row r
    const int u_lds = (j * NW + w) * 64 + l;
    // units past this workgroup's state columns re-read its last unit (never used)
    const int r = u_lds / C::VU, u = min((u_lds % C::VU) ^ vswz<C::VU>(r), 2 * max(nS, 1) - 1);
    off_v[j] = (uint32_t)r * tok_v + 16 * u;
  }
  // part 0: K (and Q) fragments; part 1: the record and the value slab;
  // -1: all of them
  auto issue_dma = [&](int b, int t0, int64_t slot, bool with_rec = true, int part = -1) {
    char *buf = smem + b * C::BUF;
    const int64_t left = T_all - t0;   // tokens from the chunk's first to the end of the tensor
    const int64_t lim = 0xFFFFFFFFll;
    const char *kb = reinterpret_cast<const char *>(gk + ((int64_t)t0 * H + hn) * DK);
    const uint32_t nk = (uint32_t)min(left * tok_k - (int64_t)hn * DK * 2, lim);
    const char *qb = WANT_O ? reinterpret_cast<const char *>(gq + ((int64_t)t0 * H + hn) * DK) : nullptr;
    const char *rec = grec + (slot * H + hn) * (int64_t)(kRecFloats * 4);
#pragma unroll
    for (int j = 0; j < JK; ++j) {                           // K (and Q) A fragments
      const int f = j * NW + w;
      if (part != 1 && (C::NKA % NW == 0 || f < C::NKA)) {
        dma16_buffer(kb, nk, (lds_void *)(buf + (C::bKA + f) * 1024), off_kq[j]);
        if (WANT_O) dma16_buffer(qb, nk, (lds_void *)(buf + (C::bQA + f) * 1024), off_kq[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < JT; ++j) {                           // Tau diag(beta) fragments (record)
      const int f = j * NW + w;
      if (part != 0 && with_rec && (C::NTF % NW == 0 || f < C::NTF)) {
        dma16_buffer(rec, kRecFloats * 4, (lds_void *)(buf + (C::bTF + f) * 1024), 16 * l, f * 1024);
      }
    }
    if (part != 0 && grp_S) {                                // value slab of the workgroup
      const char *vb = reinterpret_cast<const char *>(gv + ((int64_t)t0 * H + hn) * DV + vcol0);
      const uint32_t nv = (uint32_t)min(left * tok_v - ((int64_t)hn * DV + vcol0) * 2, lim);
#pragma unroll
      for (int j = 0; j < JV; ++j) {
        const int f = j * NW + w;
        if (C::NVB % NW == 0 || f < C::NVB) dma16_buffer(vb, nv, (lds_void *)(buf + (C::bV + f) * 1024), off_v[j]);
      }
    }
  };

  // wave 0: alpha bits of token t0 + l (1.0 past the end; raw inputs: the
  // log-gate, 0 past the end) and, for raw inputs, the token's reciprocal
  // key norm
  unsigned short pa = 0;
  float rk = 1.f;
  auto load_alpha = [&](int t0, int Lc) {
    pa = p.raw ? 0 : 0x3f80;
    if (w == 0 && l < Lc) pa = ga[(int64_t)(t0 + l) * H + hn];
  };
  auto load_norms = [&](int64_t slot, int Lc) {
    if (p.raw && w == 0 && l < Lc) {
      rk = p.norms[(slot * H + hn) * kNormFloats + l];
    }
  };
  // Running scale of the state.  The registers hold S / gam, gam a scalar
  // of the workgroup's (sequence, segment, head) that wave 0 tracks.  A
  // chunk folds its decay e^{g_L} into gam and leaves the registers alone;
  // the per-token vectors are scaled to match (e^g by gam for the reads of
  // the state, e^{g_L - g} by 1 / gam' for the corrections added to it).
  // When gam' would drop below 2^-40, and at a sequence's last chunk, the
  // chunk instead scales the registers by gam e^{g_L} and resets gam to 1,
  // so that the state written out is S itself.  This spares the multiply of
  // every state element by e^{g_L} in most chunks.
  float gam = 1.f;
  auto gates = [&](int b, int Lc, bool last) {
    if (w != 0) return;
    float *sG = sG0 + b * C::GN;
    const float x = __uint_as_float((unsigned)pa << 16);
    const float lg = p.raw ? fmaxf(x, kLogGateFloor) : log_gate(x);
    const float g = wave_inclusive_scan((l < Lc) ? lg : 0.f);
    const float gL = lane_value(g, Lc - 1);
    const float cand = gam * __expf(gL);
    const bool apply = last || !(cand >= 0x1p-40f);
    const float gnew = apply ? 1.f : cand;
    const float inv = 1.f / gnew;
    const float eg = gam * __expf(g);
    sG[G_EG + l] = eg * rk;
    sG[G_EQ + l] = eg;
    sG[G_DEC + l] = (l < Lc) ? __expf(gL - g) * inv * rk : 0.f;
    sG[G_G + l] = g;
    sG[G_RK + l] = rk;
    if (l == 0) sG[G_EGL] = apply ? cand : 1.f;   // the registers' scale factor (1: none)
    gam = gnew;
  };
  // the registers' scale factor of the chunk in gate set sG, uniform
  auto state_scale = [&](const float *sG) {
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(sG[G_EGL])));
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
  uint2 vt[RT][4];
  const uint32_t vmask = (active && !is_T) ? 0xffffffffu : 0u;
  const int vtile = (active && !is_T) ? tile - tT - sfirst : 0;  // first staged state tile of the wave
  auto read_v = [&](int b) {
    const char *buf = smem + b * C::BUF;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int bt = 0; bt < 4; ++bt) {
        const int rr0 = 16 * bt + 4 * g4 + (jl >> 2);
        const int u = min(2 * (vtile + rt), C::VU - 2) + ((jl & 3) >> 1);
        const uint2 x = ds_read_tr16(reinterpret_cast<const bf16 *>(
            buf + C::bV * 1024 + rr0 * (C::VU * 16) + 16 * (u ^ vswz<C::VU>(rr0)) + 8 * (jl & 1)));
        if constexpr (WANT_O)   // (no transition tiles; an idle wave never reads vt)
          vt[rt][bt] = x;
        else
          vt[rt][bt] = uint2{x.x & vmask, x.y & vmask};
      }
  };

  // ---- prologue (fused mode): the workgroup builds the per-chunk records of
  // its own segment, one chunk per wave at a time, before the recurrence
  // reads them ----
  // The first chunk's keys and values are copied meanwhile; its record
  // goes straight into buffer set 0 as well.
  if constexpr (FUSED) {
    if (tbeg < tend) {
      const int L0 = min(CH, tend - tbeg);
      issue_dma(0, tbeg, slot0, false);
      load_alpha(tbeg, L0);
    }
    float *scr = reinterpret_cast<float *>(smem + C::PSCR) + (w % C::NPW) * (kPrepWaveLds / 4);
    const int nch = (tend - tbeg + CH - 1) / CH;
    // lead layout: a share of the records of the last segment (chunks xb ..
    // xb + nx - 1 of the sequence), which the segment launch does not run
    int xb = 0, nx = 0;
    if (p.lead && p.tiles_T > 0) lead_extras(p, nch_seq, seg, xb, nx);
    if constexpr (MULTI) {
      // the records of every chunk of the items it .. it_end - 1,
      // round-robin over the waves
      int c = 0;
      for (int i2 = it; i2 < it_end; ++i2) {
        const int n2 = i2 / H, h2 = i2 % H, b2 = p.cu[n2], e2 = p.cu[n2 + 1];
        for (int tc = b2; tc < e2; tc += CH, ++c) {
          if (w >= C::NPW || c % C::NPW != w) continue;
          const int64_t sl = (int64_t)(b2 / CH) + n2 + (tc - b2) / CH;
          char *rec = const_cast<char *>(grec) + (sl * H + h2) * (int64_t)(kRecFloats * 4);
          char *lrec = c == 0 ? smem + C::bTF * 1024 : nullptr;
          if (p.raw)
            prep_chunk_wave<DK, true>(gk, reinterpret_cast<const bf16 *>(p.alpha),
                                      reinterpret_cast<const bf16 *>(p.beta), H, h2, tc, min(CH, e2 - tc), rec, scr,
                                      lrec, p.norms + (sl * H + h2) * kNormFloats);
          else
            prep_chunk_wave<DK>(gk, reinterpret_cast<const bf16 *>(p.alpha), reinterpret_cast<const bf16 *>(p.beta),
                                H, h2, tc, min(CH, e2 - tc), rec, scr, lrec);
        }
      }
    } else {
      for (int c = w; c < nch + nx && w < C::NPW; c += C::NPW) {
        const bool own = c < nch;
        const int tc = own ? tbeg + c * CH : cbeg + (xb + c - nch) * CH;
        const int64_t sl = (int64_t)(cbeg / CH) + n + (tc - cbeg) / CH;
        char *rec = const_cast<char *>(grec) + (sl * H + h) * (int64_t)(kRecFloats * 4);
        char *lrec = (own && c == 0) ? smem + C::bTF * 1024 : nullptr;
        if (p.raw)
          prep_chunk_wave<DK, true>(gk, reinterpret_cast<const bf16 *>(p.alpha), reinterpret_cast<const bf16 *>(p.beta),
                                    H, h, tc, min(CH, cend - tc), rec, scr, lrec, p.norms + (sl * H + h) * kNormFloats);
        else
          prep_chunk_wave<DK>(gk, reinterpret_cast<const bf16 *>(p.alpha), reinterpret_cast<const bf16 *>(p.beta), H,
                              h, tc, min(CH, cend - tc), rec, scr, lrec);
      }
    }
    wait_vmem();
    __syncthreads();
    if (tbeg < tend) {
      load_norms(slot0, min(CH, tend - tbeg));
      gates(0, min(CH, tend - tbeg), tend - tbeg <= CH);
    }
  } else if (tbeg < tend) {
    const int L0 = min(CH, tend - tbeg);
    issue_dma(0, tbeg, slot0);
    load_alpha(tbeg, L0);
    load_norms(slot0, L0);
    gates(0, L0, tend - tbeg <= CH);
  }
  wait_vmem();
  lds_barrier();
  read_v(0);

  // Outputs.  O = diag(e^g) Q S^T + (M o Q K^T) D: the first part is
  // formed in the chunk itself; M o Q K^T of the chunk is built during the
  // chunk (split between the waves, into one of two LDS sets) and becomes
  // visible to every wave at the chunk's hand-over barrier, so the second
  // part and the store of a chunk's outputs follow in the next chunk (or
  // after the last one).  Both parts are formed transposed, O^T = e^g S Q^T
  // + D^T (M o Q K^T)^T: the split state and D fragments serve as A operands
  // and the Q and M o Q K^T fragments as B operands with the registers they
  // have in the other role, and a lane of the result holds four consecutive
  // value columns of one token.  zp holds the pending outputs (block bt:
  // tokens 16 bt + lane column), dph / dpl the pending D as split-bf16
  // fragments, tp / Lp its token range.
  f32x4 zp[RT][4];
  bf16x8 dph[RT][2], dpl[RT][2];
  int tp = 0, Lp = 0;
  // M o Q K^T (M_rs = e^{g_r - g_s}, s <= r) of the chunk in buffer set b
  // into set b of the M o Q K^T fragments: the twelve 16 x 16 halves of
  // the six fragments (gdn_internal.h order) round-robin over the waves.
  // Half (bi, bj) (rows r of block bi, columns s of block bj) is formed
  // transposed, K Q^T, so that lane (q, g) holds the four consecutive
  // columns s = 16 bj + 4 g + e of row r = 16 bi + q: exactly elements
  // 4 (bj & 1) .. + 3 of that lane's slot in fragment (bi, bj >> 1), one
  // 8-byte LDS write per plane.
  auto build_p = [&](int b) {
    const char *buf = smem + b * C::BUF;
    const float *sG = sG0 + b * C::GN;
    bf16 *sP = reinterpret_cast<bf16 *>(smem + C::oP + b * C::PSET);
    for (int t = w; t < 2 * kTauFrags; t += NW) {
      const int f = t >> 1, half = t & 1;
      const int bi = f < 2 ? f : (f - 2) / 2 + 2;
      const int bj = 2 * (f < 2 ? 0 : (f - 2) % 2) + half;
      f32x4 c = zero4();
      if (bj <= bi) {
#pragma unroll
        for (int m = 0; m < C::NKS; ++m) {
          const bf16x8 ka = *reinterpret_cast<const bf16x8 *>(buf + (C::bKA + bj * C::NKS + m) * 1024 + 16 * kq_l);
          const bf16x8 qb = *reinterpret_cast<const bf16x8 *>(buf + (C::bQA + bi * C::NKS + m) * 1024 + 16 * kq_l);
          c = mfma_bf16(ka, qb, c);
        }
      }
      const int r = 16 * bi + jl, s0 = 16 * bj + 4 * g4;
      const float gr = sG[G_G + r];
      const f32x4 gs = *reinterpret_cast<const f32x4 *>(sG + G_G + s0);
      f32x4 x;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = (s0 + e <= r) ? __expf(gr - gs[e]) * c[e] : 0.f;
      if (p.raw) {   // the normalised key rows (the query norms are applied to the outputs)
        const f32x4 ks = *reinterpret_cast<const f32x4 *>(sG + G_RK + s0);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] *= ks[e];
      }
      bf16x4 hi, lo;
      split4(x, hi, lo);
      *reinterpret_cast<bf16x4 *>(sP + (f * 64 + l) * 8 + 4 * half) = hi;
      *reinterpret_cast<bf16x4 *>(sP + kTauFragPlane + (f * 64 + l) * 8 + 4 * half) = lo;
    }
  };
  // the pending outputs: zp plus (M o Q K^T) D from set b, into dst (the
  // first product of each block reads zp and writes dst, so finished outputs
  // move to the stash without copies; dst may be zp)
  auto finish_o = [&](int b, f32x4 (&dst)[RT][4]) {
    const bf16 *sP = reinterpret_cast<const bf16 *>(smem + C::oP + b * C::PSET);
    constexpr int ford[kTauFrags] = {0, 2, 4, 1, 3, 5};
    constexpr bool first[kTauFrags] = {true, true, true, true, false, false};   // token blocks 0, 2, 3, 1, 2, 3
    bf16x8 ph[kTauFrags], pl[kTauFrags];
#pragma unroll
    for (int f = 0; f < kTauFrags; ++f) {
      ph[f] = *reinterpret_cast<const bf16x8 *>(sP + (f * 64 + l) * 8);
      pl[f] = *reinterpret_cast<const bf16x8 *>(sP + kTauFragPlane + (f * 64 + l) * 8);
    }
#pragma unroll
    for (int pass = 0; pass < 3; ++pass)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int i = 0; i < kTauFrags; ++i) {
          const int f = ford[i];
          const int bt = f < 2 ? f : (f - 2) / 2 + 2;
          const int m = f < 2 ? 0 : (f - 2) % 2;
          dst[rt][bt] = mfma_bf16(pass == 1 ? dpl[rt][m] : dph[rt][m], pass == 2 ? pl[f] : ph[f],
                                  pass == 0 && first[i] ? zp[rt][bt] : dst[rt][bt]);
        }
  };
  // Finished outputs wait in zs (tokens ts .. ts + Ls - 1) until the end of
  // the chunk step and are stored after its wait for the load-to-LDS copies:
  // that wait (vmcnt 0) covers every outstanding vector memory operation of
  // the wave, stores included, so stores issued earlier in the step hold up
  // the hand-over barrier (and every wave with it); issued after the wait,
  // they have the whole next step to drain.  (32768-token prefill -1.9%,
  // packed tails -3.4% against storing right after the outputs are
  // finished, in the middle of the step.)
  f32x4 zs[RT][4];
  int ts = 0, Ls = 0;
  auto stash_o = [&]() {   // (the outputs themselves went to zs in finish_o)
    ts = tp;
    Ls = Lp;
    Lp = 0;
  };
  // raw inputs with outputs: 1 / |q_t| of the chunk staged in buffer set b,
  // into its gate set (waves 0..3, 16 tokens each: the squares of the wave's
  // query fragments summed over the four lanes that hold a token)
  auto query_norms = [&](int b) {
    if (!(WANT_O && QN) || w >= 4) return;
    const char *buf = smem + b * C::BUF;
    float q2 = 0.f;
#pragma unroll
    for (int m = 0; m < C::NKS; ++m) {
      const bf16x8 f = *reinterpret_cast<const bf16x8 *>(buf + (C::bQA + w * C::NKS + m) * 1024 + 16 * kq_l);
#pragma unroll
      for (int i = 0; i < 8; ++i) q2 += (float)f[i] * (float)f[i];
    }
    q2 += __shfl_xor(q2, 16, 64);
    q2 += __shfl_xor(q2, 32, 64);
    if (g4 == 0) sG0[b * C::GN + G_RQ + 16 * w + jl] = q2 > 0.f ? rsqrtf(q2) : 0.f;
  };
  // an output row is linear in its token's query: raw inputs scale it by
  // 1 / |q_t| (gate set gs) as it is stored
  auto out_scale = [&](int gs, int bt) { return sG0[gs * C::GN + G_RQ + 16 * bt + jl]; };
  auto store_s = [&](int gs) {
    const int64_t tok = (int64_t)H * DV;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int64_t ob = ((int64_t)(ts + jl) * H + h) * DV + row0 + 16 * rt + 4 * g4;
#pragma unroll
      for (int bt = 0; bt < 4; ++bt) {
        if constexpr (QN) zs[rt][bt] *= out_scale(gs, bt);
        if (16 * bt + jl < Ls) {
          if (p.o_bf16) {
            *reinterpret_cast<uint2 *>(reinterpret_cast<bf16 *>(p.o) + ob + 16 * bt * tok) =
                uint2{pack_bf16x2(zs[rt][bt][0], zs[rt][bt][1]), pack_bf16x2(zs[rt][bt][2], zs[rt][bt][3])};
          } else {
            *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(p.o) + ob + 16 * bt * tok) = zs[rt][bt];
          }
        }
      }
    }
    Ls = 0;
  };
  auto store_o = [&](int gs) {
    // lane (q, g) of block bt holds token tp + 16 bt + q, value columns
    // row0 + 16 rt + 4 g .. + 3: one 16-byte (8-byte in bf16) store each
    const int64_t tok = (int64_t)H * DV;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int64_t ob = ((int64_t)(tp + jl) * H + h) * DV + row0 + 16 * rt + 4 * g4;
#pragma unroll
      for (int bt = 0; bt < 4; ++bt) {
        if constexpr (QN) zp[rt][bt] *= out_scale(gs, bt);
        if (16 * bt + jl < Lp) {
          if (p.o_bf16) {
            *reinterpret_cast<uint2 *>(reinterpret_cast<bf16 *>(p.o) + ob + 16 * bt * tok) =
                uint2{pack_bf16x2(zp[rt][bt][0], zp[rt][bt][1]), pack_bf16x2(zp[rt][bt][2], zp[rt][bt][3])};
          } else {
            *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(p.o) + ob + 16 * bt * tok) = zp[rt][bt];
          }
        }
      }
    }
    Lp = 0;
  };

  int64_t slot = slot0;
  int b = 0;
  for (int t0 = tbeg; t0 < tend; t0 += CH, ++slot, b ^= 1) {
    const int Lc = min(CH, tend - t0);
    // the next chunk: tokens nt0 .. min(nt0 + CH, ntend) - 1, record slot
    // nslot (MULTI: past this item's end, the first chunk of item nit)
    int nt0 = t0 + CH, ntend = tend, nn = n;
    int64_t nslot = slot + 1;
    if constexpr (MULTI) {
      if (nt0 >= tend) {
        // the next item with chunks: the next head of this sequence, else
        // head 0 of the next sequence that has chunks (all heads of a
        // sequence have its chunks)
        hn = h + 1;
        if (hn == H) {
          hn = 0;
          do ++nn; while (nn * H < it_end && p.cu[nn + 1] == p.cu[nn]);
        }
        if (nn * H + hn < it_end) {
          nt0 = p.cu[nn];
          ntend = p.cu[nn + 1];
          nslot = (int64_t)(nt0 / CH) + nn;
        }
      }
    }
    const bool more = nt0 < ntend;
    const int L1 = more ? min(CH, ntend - nt0) : 0;
    // Operands of the next chunk: in flight while this one runs.  With
    // outputs the copies go out in two halves, the second one in the middle
    // of the step next to the stores of the previous chunk's outputs: issued
    // by every wave at once right after the hand-over barrier, all of them
    // together stall the waves' instruction issue for about 2,000 cycles
    // (timed in-kernel with s_memtime on the 32768-token prefill).
    //
    // Wave priority falls along the step (3 at the top, 0 for the state
    // update): the two waves of a SIMD otherwise issue oldest first, the
    // younger one finishes its step alone with nothing to hide its MFMA and
    // LDS latencies, and the barrier waits for it.  A wave behind in the
    // step now wins issue, so both reach the barrier together (3% on the
    // 32768-token prefill and the 3277-token tail, 1% on packed tails).
    __builtin_amdgcn_s_setprio(3);
    if (more) {
      issue_dma(b ^ 1, nt0, nslot, true, WANT_O ? 0 : -1);
      load_alpha(nt0, L1);
      load_norms(nslot, L1);
    }
    query_norms(b);   // (raw inputs with outputs; read when this chunk's outputs are stored)
    const char *buf = smem + b * C::BUF;
    const float *sG = sG0 + b * C::GN;
    auto frag = [&](int blk) { return *reinterpret_cast<const bf16x8 *>(buf + blk * 1024 + 16 * l); };
    auto kqfrag = [&](int blk) { return *reinterpret_cast<const bf16x8 *>(buf + blk * 1024 + 16 * kq_l); };

    if constexpr (RT == 2 && !WANT_O) {
      // ---- two row tiles, skewed by one stage: tile 1's vector-ALU work
      // (fragment splits, residuals) sits next to tile 0's MFMAs and the
      // other way round, so the two can overlap.  The fragments both tiles
      // read (K, Tau, K^T) stay in registers across the skewed pair ----
      if (active) {
        constexpr int NKS = C::NKS, NSB = C::NSB;
        auto split_s = [&](const f32x4 (&sv)[NSB], bf16x8 (&hh)[NKS], bf16x8 (&ll)[NKS]) {
#pragma unroll
          for (int m = 0; m < NKS; ++m) b_frag_split(sv[2 * m], sv[2 * m + 1], hh[m], ll[m]);
        };
        // Y = K S^T: each accumulator is touched once every four products
        auto y_mfma = [&](const bf16x8 (&ka)[4][NKS], const bf16x8 (&hh)[NKS], const bf16x8 (&ll)[NKS],
                          f32x4 (&yy)[4]) {
#pragma unroll
          for (int bt = 0; bt < 4; ++bt) yy[bt] = zero4();
#pragma unroll
          for (int m = 0; m < NKS; ++m) {
#pragma unroll
            for (int bt = 0; bt < 4; ++bt) yy[bt] = mfma_bf16(ka[bt][m], hh[m], yy[bt]);
#pragma unroll
            for (int bt = 0; bt < 4; ++bt) yy[bt] = mfma_bf16(ka[bt][m], ll[m], yy[bt]);
          }
        };
        // R = V - e^g Y, split into B fragments (beta is in the Tau fragments)
        auto r_valu = [&](const uint2 (&vv4)[4], const f32x4 (&yy)[4], bf16x8 (&rh)[2], bf16x8 (&rl)[2]) {
          f32x4 rr[4];
#pragma unroll
          for (int bt = 0; bt < 4; ++bt) {
            const f32x4 eg = *reinterpret_cast<const f32x4 *>(sG + G_EG + 16 * bt + 4 * g4);
            const uint2 x = vv4[bt];
            const float vv[4] = {__uint_as_float(x.x << 16), __uint_as_float(x.x & 0xffff0000u),
                                 __uint_as_float(x.y << 16), __uint_as_float(x.y & 0xffff0000u)};
#pragma unroll
            for (int e = 0; e < 4; ++e) rr[bt][e] = vv[e] - eg[e] * yy[bt][e];
          }
          b_frag_split(rr[0], rr[1], rh[0], rl[0]);
          b_frag_split(rr[2], rr[3], rh[1], rl[1]);
        };
        // D = (Tau diag(beta)) R, fragments in the order 0, 2, 4, 1, 3, 5
        auto d_mfma = [&](const bf16x8 (&th)[kTauFrags], const bf16x8 (&tl)[kTauFrags], const bf16x8 (&rh)[2],
                          const bf16x8 (&rl)[2], f32x4 (&dd)[4]) {
          constexpr int ford[kTauFrags] = {0, 2, 4, 1, 3, 5};
#pragma unroll
          for (int bt = 0; bt < 4; ++bt) dd[bt] = zero4();
#pragma unroll
          for (int pass = 0; pass < 3; ++pass)
#pragma unroll
            for (int i = 0; i < kTauFrags; ++i) {
              const int f = ford[i];
              const int bt = f < 2 ? f : (f - 2) / 2 + 2;
              const int m = f < 2 ? 0 : (f - 2) % 2;
              dd[bt] = mfma_bf16(pass == 2 ? tl[f] : th[f], pass == 1 ? rl[m] : rh[m], dd[bt]);
            }
        };
        // e^{g_L} S^T, and the decayed corrections as B fragments
        auto de_valu = [&](const f32x4 (&dd)[4], f32x4 (&sv)[NSB], bf16x8 (&eh)[2], bf16x8 (&el)[2]) {
          f32x4 de[4];
#pragma unroll
          for (int bt = 0; bt < 4; ++bt) {
            const f32x4 dec = *reinterpret_cast<const f32x4 *>(sG + G_DEC + 16 * bt + 4 * g4);
#pragma unroll
            for (int e = 0; e < 4; ++e) de[bt][e] = dd[bt][e] * dec[e];
          }
          b_frag_split(de[0], de[1], eh[0], el[0]);
          b_frag_split(de[2], de[3], eh[1], el[1]);
          const float gl = state_scale(sG);
          if (gl != 1.f) {
#pragma unroll
            for (int d = 0; d < NSB; ++d)
#pragma unroll
              for (int e = 0; e < 4; ++e) sv[d][e] *= gl;
          }
        };
        // S^T += K^T D': each state block is touched once every NSB products
        auto upd_mfma = [&](const bf16x8 (&kt)[2][NSB], const bf16x8 (&eh)[2], const bf16x8 (&el)[2],
                            f32x4 (&sv)[NSB]) {
#pragma unroll
          for (int m = 0; m < 2; ++m) {
#pragma unroll
            for (int d = 0; d < NSB; ++d) sv[d] = mfma_bf16(kt[m][d], eh[m], sv[d]);
#pragma unroll
            for (int d = 0; d < NSB; ++d) sv[d] = mfma_bf16(kt[m][d], el[m], sv[d]);
          }
        };

        bf16x8 sh0[NKS], sl0[NKS], sh1[NKS], sl1[NKS];
        f32x4 y0[4], y1[4], d0[4], d1[4];
        bf16x8 rh0[2], rl0[2], rh1[2], rl1[2], eh0[2], el0[2], eh1[2], el1[2];
        {
          bf16x8 ka[4][NKS];
#pragma unroll
          for (int bt = 0; bt < 4; ++bt)
#pragma unroll
            for (int m = 0; m < NKS; ++m) ka[bt][m] = kqfrag(C::bKA + bt * NKS + m);
          split_s(st[0], sh0, sl0);
          y_mfma(ka, sh0, sl0, y0);
          split_s(st[1], sh1, sl1);
          r_valu(vt[0], y0, rh0, rl0);
          y_mfma(ka, sh1, sl1, y1);
        }
        __builtin_amdgcn_s_setprio(2);
        {
          bf16x8 th[kTauFrags], tl[kTauFrags];
#pragma unroll
          for (int f = 0; f < kTauFrags; ++f) {
            th[f] = frag(C::bTF + f);
            tl[f] = frag(C::bTF + kTauFrags + f);
          }
          d_mfma(th, tl, rh0, rl0, d0);
          r_valu(vt[1], y1, rh1, rl1);
          de_valu(d0, st[0], eh0, el0);
          d_mfma(th, tl, rh1, rl1, d1);
        }
        __builtin_amdgcn_s_setprio(1);
        {
          bf16x8 kt[2][NSB];
          kt_frags<NKS, NSB>(0, kt_lds + (uint32_t)(b * C::BUF), kt[0]);
          kt_frags<NKS, NSB>(1, kt_lds + (uint32_t)(b * C::BUF), kt[1]);
          upd_mfma(kt, eh0, el0, st[0]);
          de_valu(d1, st[1], eh1, el1);
          upd_mfma(kt, eh1, el1, st[1]);
        }
      }
    } else {
      // ---- S^T as k = 32 B fragments ----
      bf16x8 sh[RT][C::NKS], sl[RT][C::NKS];
      f32x4 dd[RT][4];
      if (active) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int m = 0; m < C::NKS; ++m) b_frag_split(st[rt][2 * m], st[rt][2 * m + 1], sh[rt][m], sl[rt][m]);

      // ---- Y = K S^T (each K fragment read once for the wave's row tiles) ----
      // A dependent MFMA (same accumulator) waits about three issue slots:
      // every loop below rotates over at least four accumulators (the hi
      // and lo passes of a product share them where four or more rotate,
      // and accumulate separately where fewer would).
      f32x4 y[RT][4];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int bt = 0; bt < 4; ++bt) y[rt][bt] = zero4();
#pragma unroll
      for (int m = 0; m < C::NKS; ++m) {
        bf16x8 a[4];
#pragma unroll
        for (int bt = 0; bt < 4; ++bt) a[bt] = kqfrag(C::bKA + bt * C::NKS + m);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int bt = 0; bt < 4; ++bt) y[rt][bt] = mfma_bf16(a[bt], sh[rt][m], y[rt][bt]);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int bt = 0; bt < 4; ++bt) y[rt][bt] = mfma_bf16(a[bt], sl[rt][m], y[rt][bt]);
      }

      __builtin_amdgcn_s_setprio(2);
      // ---- R = V - e^g Y  (beta is folded into the Tau fragments) ----
      bf16x8 rh[RT][2], rl[RT][2];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        f32x4 rr[4];
#pragma unroll
        for (int bt = 0; bt < 4; ++bt) {
          const f32x4 eg = *reinterpret_cast<const f32x4 *>(sG + G_EG + 16 * bt + 4 * g4);
          const uint2 x = vt[rt][bt];
          const float vv[4] = {__uint_as_float(x.x << 16), __uint_as_float(x.x & 0xffff0000u),
                               __uint_as_float(x.y << 16), __uint_as_float(x.y & 0xffff0000u)};
#pragma unroll
          for (int e = 0; e < 4; ++e) rr[bt][e] = vv[e] - eg[e] * y[rt][bt][e];
        }
        b_frag_split(rr[0], rr[1], rh[rt][0], rl[rt][0]);
        b_frag_split(rr[2], rr[3], rh[rt][1], rl[rt][1]);
      }

      // ---- D = (Tau diag(beta)) R  (f: (bt, m) = (0,0),(1,0),(2,0),(2,1),(3,0),(3,1)) ----
      // fragments in the order 0, 2, 4, 1, 3, 5 (token blocks 0, 2, 3, 1, 2, 3)
      // so that a block's two products are three issue slots apart; all
      // three split passes share the accumulators
      {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int bt = 0; bt < 4; ++bt) dd[rt][bt] = zero4();
        constexpr int ford[kTauFrags] = {0, 2, 4, 1, 3, 5};
        bf16x8 th[kTauFrags], tl[kTauFrags];
#pragma unroll
        for (int f = 0; f < kTauFrags; ++f) {
          th[f] = frag(C::bTF + f);
          tl[f] = frag(C::bTF + kTauFrags + f);
        }
#pragma unroll
        for (int pass = 0; pass < 3; ++pass)
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int i = 0; i < kTauFrags; ++i) {
              const int f = ford[i];
              const int bt = f < 2 ? f : (f - 2) / 2 + 2;
              const int m = f < 2 ? 0 : (f - 2) % 2;
              dd[rt][bt] = mfma_bf16(pass == 2 ? tl[f] : th[f], pass == 1 ? rl[rt][m] : rh[rt][m], dd[rt][bt]);
            }
      }
      }  // active

      __builtin_amdgcn_s_setprio(1);
      if constexpr (WANT_O) {
        // the previous chunk's outputs (its M o Q K^T became visible at the
        // hand-over barrier), then the second half of the next chunk's copies
        if (active && Lp > 0) {
          finish_o(b ^ 1, zs);
          stash_o();
        }
        if (more) issue_dma(b ^ 1, nt0, nslot, true, 1);
      }

      if (active) {
      // ---- outputs: the previous chunk's finished and stored; this one's
      // e^g Q S^T (every Q fragment read once for the wave's row tiles) and
      // its D, pending ----
      if (WANT_O) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          b_frag_split(dd[rt][0], dd[rt][1], dph[rt][0], dpl[rt][0]);
          b_frag_split(dd[rt][2], dd[rt][3], dph[rt][1], dpl[rt][1]);
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int bt = 0; bt < 4; ++bt) zp[rt][bt] = zero4();
#pragma unroll
        for (int m = 0; m < C::NKS; ++m) {
          bf16x8 a[4];
#pragma unroll
          for (int bt = 0; bt < 4; ++bt) a[bt] = kqfrag(C::bQA + bt * C::NKS + m);
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int bt = 0; bt < 4; ++bt) zp[rt][bt] = mfma_bf16(sh[rt][m], a[bt], zp[rt][bt]);
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int bt = 0; bt < 4; ++bt) zp[rt][bt] = mfma_bf16(sl[rt][m], a[bt], zp[rt][bt]);
        }
#pragma unroll
        for (int bt = 0; bt < 4; ++bt) {
          const float eg = sG[G_EQ + 16 * bt + jl];
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int e = 0; e < 4; ++e) zp[rt][bt][e] *= eg;
        }
        tp = t0;
        Lp = Lc;
      }

      __builtin_amdgcn_s_setprio(0);
      // ---- S^T <- e^{g_L} S^T + K^T diag(e^{g_L - g}) D ----
      bf16x8 eh[RT][2], el[RT][2];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        f32x4 de[4];
#pragma unroll
        for (int bt = 0; bt < 4; ++bt) {
          const f32x4 dec = *reinterpret_cast<const f32x4 *>(sG + G_DEC + 16 * bt + 4 * g4);
#pragma unroll
          for (int e = 0; e < 4; ++e) de[bt][e] = dd[rt][bt][e] * dec[e];
        }
        b_frag_split(de[0], de[1], eh[rt][0], el[rt][0]);
        b_frag_split(de[2], de[3], eh[rt][1], el[rt][1]);
      }
      // K^T fragments of one token half m for all dk blocks, then the four
      // (m, pass) sweeps over the dk blocks: each state block is touched
      // once every NSB products
      const float gl = state_scale(sG);
      if (gl != 1.f) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int d = 0; d < C::NSB; ++d)
#pragma unroll
            for (int e = 0; e < 4; ++e) st[rt][d][e] *= gl;
      }
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        bf16x8 a[C::NSB];
        kt_frags<C::NKS, C::NSB>(m, kt_lds + (uint32_t)(b * C::BUF), a);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int d = 0; d < C::NSB; ++d) st[rt][d] = mfma_bf16(a[d], eh[rt][m], st[rt][d]);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int d = 0; d < C::NSB; ++d) st[rt][d] = mfma_bf16(a[d], el[rt][m], st[rt][d]);
      }
      }  // active
    }

    __builtin_amdgcn_s_setprio(0);
    if (WANT_O) build_p(b);
    // ---- hand over to the next chunk ----
    if (more) gates(b ^ 1, L1, nt0 + CH >= ntend);
    wait_vmem();
    if (WANT_O && active && Ls > 0) store_s(b ^ 1);   // the previous chunk's outputs
    if constexpr (MULTI) {
      if (t0 + CH >= tend) {
        // this item's operator out (the stores drain during the next
        // steps), the registers back to their start, the stream on to item nit
        if (active) {
          float *ob = op_base(n, h);
          // the start values from the lane's diagonal positions (kept opaque,
          // so that the compiler does not hold all 64 of them in registers
          // across the loop)
          int dg[RT];
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            const int c = row0 + 16 * rt + jl;   // the diagonal element's column
            dg[rt] = (is_T && g4 == (c & 31) >> 3) ? 4 * (2 * (c >> 5) + ((c & 7) >> 2)) + (c & 3) : -1;
            asm volatile("" : "+v"(dg[rt]));
          }
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int d = 0; d < C::NSB; ++d) {
              *reinterpret_cast<f32x4 *>(ob + op_off(rt, d)) = st[rt][d];
#pragma unroll
              for (int e = 0; e < 4; ++e) st[rt][d][e] = dg[rt] == 4 * d + e ? 1.f : 0.f;
            }
        }
        if (more) {
          n = nn;
          h = hn;
          tend = ntend;
          t0 = nt0 - CH;     // (the loop's increments then land on the next chunk)
          slot = nslot - 1;
        }
      }
    }
    lds_barrier();
    if (more) read_v(b ^ 1);
  }

  if constexpr (MULTI) {
    wait_vmem();   // (the last operator's stores, before the workgroup ends)
    return;        // (every item's operator was written in the loop)
  }
  // ---------------- epilogue: final rows ----------------
  if (WANT_O && active && Lp > 0) {
    finish_o(b ^ 1, zp);   // the last chunk's set (b has moved past it)
    store_o(b ^ 1);
  }
  const int64_t unit = ((int64_t)n * p.n_segs + seg) * H + h;
  if (p.T_frags) {
    // Segment operator as composition fragments: the transition rows go to
    // LDS (all waves passed the last hand-over barrier, so the chunk
    // buffers are free) and come back as column slices, split into bf16
    // hi and lo.  The barrier is workgroup-uniform (T_frags is a launch
    // argument).
    constexpr int LDT = DK + 4;
    float *sw = reinterpret_cast<float *>(smem);
    if (is_T) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int d = 0; d < C::NSB; ++d) {
          const int c0 = 32 * (d >> 1) + 8 * g4 + 4 * (d & 1);
          *reinterpret_cast<f32x4 *>(sw + (row0 + 16 * rt + jl) * LDT + c0) = st[rt][d];
        }
    }
    __syncthreads();
    if (is_T) {
      const int n_tw = tT / RT, tw = row0 / (16 * RT);
      bf16 *fh = reinterpret_cast<bf16 *>(p.T_out) + unit * DK * DK * 2, *fl = fh + DK * DK;
      for (int f = tw; f < C::NSB * C::NKS; f += n_tw) {
        const int jb = f / C::NKS, ks = f % C::NKS;
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = sw[(32 * ks + 8 * g4 + i) * LDT + 16 * jb + jl];
        bf16x8 hi, lo;
        split8(x, hi, lo);
        *reinterpret_cast<bf16x8 *>(fh + (f * 64 + l) * 8) = hi;
        *reinterpret_cast<bf16x8 *>(fl + (f * 64 + l) * 8) = lo;
      }
    }
  }
  if (active && !(p.T_frags && is_T) && (is_T || p.S_out)) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int d = 0; d < C::NSB; ++d) {
        const int c0 = 32 * (d >> 1) + 8 * g4 + 4 * (d & 1), r = row0 + 16 * rt + jl;
        float *out = is_T ? p.T_out + unit * DK * DK : p.S_out + unit * DV * DK;
        *reinterpret_cast<f32x4 *>(out + (int64_t)r * DK + c0) = st[rt][d];
      }
  }
  if (active && !is_T && p.S_last && seg == p.n_segs - 1) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int d = 0; d < C::NSB; ++d) {
        const int c0 = 32 * (d >> 1) + 8 * g4 + 4 * (d & 1), r = row0 + 16 * rt + jl;
        *reinterpret_cast<f32x4 *>(p.S_last + (((int64_t)n * H + h) * DV + r) * DK + c0) = st[rt][d];
      }
  }
}

// The launch: one workgroup per (sequence, head, segment, row-tile group).
// With LEAD (segment launch of the lead layout) segment 0 runs the output
// recurrence, one row tile per wave, and the other segments this body.
template <int DK, bool WANT_O, int NW, int RT, bool FUSED, bool LEAD = false, bool QN = false, bool MULTI = false>
__global__ void __launch_bounds__(NW * 64) chain_bf16_kernel(ChainLaunch p, int n_items) {
  using C = Cfg<DK, WANT_O, NW, RT, FUSED>;
  using CL = Cfg<DK, true, NW, 1, FUSED>;
  constexpr size_t SM = (LEAD && CL::SMEM > C::SMEM) ? CL::SMEM : C::SMEM;
  __shared__ __attribute__((aligned(16))) char smem[SM];
  if constexpr (MULTI) {
    // block b: items b per .. (b + 1) per - 1 (one (sequence, head) each)
    const int per = (n_items + (int)gridDim.x - 1) / (int)gridDim.x;
    const int i0 = (int)blockIdx.x * per, i1 = min(n_items, i0 + per);
    if (i0 >= i1) return;
    chain_body<DK, WANT_O, NW, RT, FUSED, false, true>(p, i0 / p.H, i0 % p.H, 0, 0, smem, i0, i1);
    return;
  }
  const SegGroups sg = seg_groups(p, C::TW, LEAD ? NW : C::TW);
  // One workgroup per (sequence, head) with a longest-first sequence order:
  // items in block order (the dispatcher deals blocks round-robin over the
  // XCDs, so the longest items start first everywhere).  Otherwise
  // XCD-aware: consecutive items (workgroups of one sequence and head,
  // which stage the same operands) share one XCD's L2.
  const bool ordered = p.order != nullptr && sg.per_nh == 1;
  const int per = (int)(gridDim.x >> 3);
  const int item = ordered ? (int)blockIdx.x : (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
  if (item >= n_items) return;
  const int nh = item / sg.per_nh;
  int rem = item % sg.per_nh, seg = sg.first, grp = rem;
  if (rem >= sg.grp0) {
    rem -= sg.grp0;
    seg = sg.first + (sg.grp0 > 0 ? 1 : 0) + rem / sg.grpA;
    grp = rem % sg.grpA;
  }
  const int n = ordered ? p.order[nh / p.H] : nh / p.H, h = nh % p.H;
  if constexpr (LEAD) {
    if (seg == 0) {
      chain_body<DK, true, NW, 1, FUSED, QN>(p, n, h, 0, grp, smem);
      return;
    }
  }
  chain_body<DK, WANT_O, NW, RT, FUSED, WANT_O && QN>(p, n, h, seg, grp, smem);
}

template <int DK, bool WANT_O, int NW, int RT, bool FUSED = false, bool LEAD = false, bool QN = false,
          bool MULTI = false>
hipError_t launch_b(const ChainLaunch &p, hipStream_t stream) {
  constexpr int TW = NW * RT;
  if (p.tiles_T % RT != 0 || p.tiles_S % RT != 0 || p.tiles_T > 8 || p.tiles_S > 8) return hipErrorInvalidValue;
  if (LEAD && p.tiles_S > NW) return hipErrorInvalidValue;
  const SegGroups sg = seg_groups(p, TW, LEAD ? NW : TW);
  const int64_t items = (int64_t)p.n_seqs * p.H * sg.per_nh;
  if (items <= 0) return hipSuccess;
  if (MULTI && (sg.per_nh != 1 || p.multi_wgs <= 0)) return hipErrorInvalidValue;
  const int64_t grid = MULTI ? (items < p.multi_wgs ? items : p.multi_wgs) : (items + 7) / 8 * 8;
  return launch_kernel(chain_bf16_kernel<DK, WANT_O, NW, RT, FUSED, LEAD, QN, MULTI>, dim3((unsigned)grid),
                       dim3(NW * 64), 0, stream, p, (int)items);
}

template <int DK>
hipError_t launch_dk(const ChainLaunch &p, hipStream_t stream) {
  if (p.lead && (p.n_segs < 2 || !p.o)) return hipErrorInvalidValue;
  if (p.o && p.tiles_T == 0) {
    if (p.fuse_prep || (p.lead && !p.S0_seg)) return hipErrorInvalidValue;
    // one eight-wave workgroup per (sequence, segment, head): two waves per
    // SIMD interleave their work (measured on 16 packed tails: 668 us
    // against 933 us for two four-wave workgroups per head and 826 us for
    // four waves with two row tiles each)
    // (raw inputs: the variant that forms the query norms)
    if (p.tiles_S % 8 == 0)
      return p.raw ? launch_b<DK, true, 8, 1, false, false, true>(p, stream) : launch_b<DK, true, 8, 1>(p, stream);
    return p.raw ? launch_b<DK, true, 4, 1, false, false, true>(p, stream) : launch_b<DK, true, 4, 1>(p, stream);
  }
  // Transition and state tiles of a segment share one workgroup, two row
  // tiles per wave: every fragment read from LDS then feeds two products,
  // and one staged copy of the chunk operands serves all the tiles.
  // State-only replays keep one row tile per wave (shorter chunk steps).
  const int tilesA = p.tiles_T + p.tiles_S;
  if (p.T_frags && p.tiles_T * 16 != p.dk) return hipErrorInvalidValue;
  if (p.tiles_T > 0 && p.lead) {
    // segment launch of the lead layout: segment 0 with its outputs
    if (!p.fuse_prep || p.S0_seg) return hipErrorInvalidValue;
    if (tilesA <= 8)
      return p.raw ? launch_b<DK, false, 4, 2, true, true, true>(p, stream)
                   : launch_b<DK, false, 4, 2, true, true>(p, stream);
    if (tilesA <= 16)
      return p.raw ? launch_b<DK, false, 8, 2, true, true, true>(p, stream)
                   : launch_b<DK, false, 8, 2, true, true>(p, stream);
    return hipErrorInvalidValue;
  }
  if (p.o) return hipErrorInvalidValue;
  if (p.tiles_T > 0) {
    // one workgroup per (sequence, segment, head): it may build its own
    // segment's records first
    if (p.multi_wgs > 0) {
      // chunk operators in several rounds of workgroups: one stream of items
      // per workgroup
      if (!p.fuse_prep || p.n_segs != 1 || p.T_frags || p.S0 || p.S0_seg || p.S_last || tilesA <= 8 ||
          tilesA > 16)
        return hipErrorInvalidValue;
      return launch_b<DK, false, 8, 2, true, false, false, true>(p, stream);
    }
    if (tilesA <= 8)
      return p.fuse_prep ? launch_b<DK, false, 4, 2, true>(p, stream) : launch_b<DK, false, 4, 2>(p, stream);
    if (tilesA <= 16)
      return p.fuse_prep ? launch_b<DK, false, 8, 2, true>(p, stream) : launch_b<DK, false, 8, 2>(p, stream);
    return hipErrorInvalidValue;
  }
  if (p.fuse_prep) return hipErrorInvalidValue;
  return p.tiles_S % 8 == 0 ? launch_b<DK, false, 8, 1>(p, stream) : launch_b<DK, false, 4, 1>(p, stream);
}

}  // namespace

hipError_t launch_chain_bf16(const ChainLaunch &p, hipStream_t stream) {
  if (p.n_segs < 1 || p.tiles_S % 4 != 0 || p.tiles_T % 4 != 0) return hipErrorInvalidValue;
  if (p.dk == 64) return launch_dk<64>(p, stream);
  if (p.dk == 128) return launch_dk<128>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace gdn
