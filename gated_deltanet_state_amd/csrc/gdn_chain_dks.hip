// gdn_chain_dks.hip -- state-only Gated DeltaNet recurrence for bf16 inputs
// when there are few (sequence, head) pairs and long sequences: one
// workgroup per 16 state rows of one (sequence, head), its waves splitting
// the key dimension.
//
// The recurrence (page "Tail-Replay: Escaping the Curse of Linear Attention
// in Prefix Caching for Hybrid LLMs", section 2 Eq. (1); state S dv x dk):
//     S_t = S_{t-1} alpha_t (I - beta_t k_t k_t^T) + beta_t v_t k_t^T.
// Per 64-token chunk, with cumulative log-gates g, the record
// Tau diag(beta) (gdn_prep_wave.h) and the 16 state rows of the workgroup
// (transposed: tokens x rows):
//     Y = K S^T,  R = V - diag(e^g) Y,  D' = diag(e^{g_L - g}) Tau diag(beta) R,
//     S^T <- e^{g_L} S^T + K^T D'.
// A chunk step of one row tile is a chain of small products, so its time
// is latency, not throughput: with few row tiles in flight the GPU would
// idle.  Here the dk / 32 waves of a workgroup share one row tile:
//   * wave w holds S^T rows 32 w .. 32 w + 31 (two C-layout blocks in the
//     permuted dk order of gdn_chain_bf16.hip, which are exactly the B
//     operand of the k = 32 step w) and computes the partial product
//     Y_w = K[:, 32w..] S^T[32w.., :] for all 64 tokens;
//   * the partials meet in LDS; wave w sums token blocks w, w + W, ..
//     (16 tokens each, fixed order), forms R for them and publishes R as
//     split-bf16 B fragments;
//   * wave w applies the rows of Tau diag(beta) of its token blocks (lower
//     triangular: k = 32 steps m <= bt / 2), scales by the decay and
//     publishes D' the same way;
//   * wave w updates its S^T rows with K^T (transposing LDS reads of the
//     staged keys) times all of D'.
// Three workgroup barriers per chunk.  Each chunk's keys, record (with
// its gates) and value columns arrive in one of three LDS buffer sets by
// load-to-LDS DMA issued three chunks ahead; after the second barrier of
// the chunk before, every wave reads its operands of the chunk from there
// into registers, overlapping the rest of that chunk, which frees the
// buffer set for the chunk three ahead.
//
// Precision as in gdn_chain_bf16.hip: K, V exact in bf16; S, R, D' and Tau
// as split bf16 (hi + lo) where they enter a product; fp32 accumulation.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int CH = kChunk;

template <int DK>
struct DksCfg {
  static constexpr int W = DK / 32;          // waves; wave w owns dk 32 w .. 32 w + 31
  static constexpr int NKS = DK / 32;
  static constexpr int NB = 4 / W;           // token blocks per wave: w, w + W, ..
  static constexpr int NKA = 4 * NKS;        // staged K A fragments (bt, m), 1 KiB each
  static constexpr int NTF = 2 * kTauFrags;  // Tau diag(beta) fragments, hi then lo
  static constexpr int NVB = 2;              // value columns: 64 tokens x 16 bf16 = 2 KiB
  static constexpr int bKA = 0, bTF = NKA, bG = bTF + NTF, bV = bG + 1;   // bG: the record's gates
  static constexpr int NBUF = 3;
  static constexpr size_t BUF = (size_t)(bV + NVB) * 1024;
  static constexpr size_t oY = NBUF * BUF;                 // partials of Y: [W][4 token blocks] x 1 KiB
  static constexpr size_t oR = oY + (size_t)W * 4 * 1024;  // R fragments: [m][hi, lo] x 1 KiB
  static constexpr size_t oD = oR + 4096;                  // D' fragments, same layout
  static constexpr size_t TOTAL = oD + 4096;
  // load-to-LDS copies every wave issues per chunk (the same count on
  // every wave, so that "all but the latest k chunks' copies" is one
  // vmcnt): K, record, gates, one value block
  static constexpr int VM = 4 + NTF / W + 1 + 1;
  static_assert(NTF % W == 0 && NKS == W && W <= 4, "per-wave copy pattern");
  static_assert(TOTAL <= 160 * 1024, "LDS budget");
};

// 8-byte LDS store at a run-time address, opaque to the compiler's wait
// insertion: as a plain store it would be made to wait for every
// load-to-LDS copy in flight (they might alias).  Ordered against later
// reads by the workgroup barrier (which waits for this wave's LDS traffic).
__device__ __forceinline__ void lds_store8(uint32_t addr, uint2 v) {
  asm volatile("ds_write_b64 %0, %1" : : "v"(addr), "v"(v));
}

// Wait until at most N vector-memory operations of this wave remain.
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

template <int DK>
__global__ void __launch_bounds__(DK / 32 * 64) chain_dks_kernel(ChainLaunch p, int n_items) {
  using C = DksCfg<DK>;
  constexpr int NKS = C::NKS, W = C::W, NB = C::NB;
  __shared__ __attribute__((aligned(16))) char smem[C::TOTAL];

  // ---- work item (XCD-aware: the row tiles of a head share one XCD's L2) ----
  const int per = (int)(gridDim.x >> 3);
  const int item = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
  if (item >= n_items) return;
  const int tiles = p.dv / 16;
  const int nh = item / tiles, tile = item % tiles;
  const int n = nh / p.H, h = nh % p.H;
  const int H = p.H, DV = p.dv;
  const int w = __builtin_amdgcn_readfirstlane(wave_id()), l = lane_id();
  const int g4 = l >> 4, jl = l & 15;
  const int row = 16 * tile + jl;              // this lane's state row (C-layout column)
  const int tbeg = p.cu[n], tend = p.cu[n + 1];
  const int nch = (tend - tbeg + CH - 1) / CH;
  const int64_t slot0 = (int64_t)(tbeg / CH) + n;

  // ---- S^T rows of this wave: block j holds dk 32 w + 8 g4 + 4 j + e ----
  f32x4 st[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    st[j] = zero4();
    if (p.S0)
      st[j] = *reinterpret_cast<const f32x4 *>(p.S0 + (((int64_t)n * H + h) * DV + row) * DK + 32 * w + 8 * g4 + 4 * j);
  }

  const bf16 *gk = reinterpret_cast<const bf16 *>(p.k);
  const bf16 *gv = reinterpret_cast<const bf16 *>(p.v);
  const char *grec = reinterpret_cast<const char *>(p.tau);
  const uint32_t tok_k = (uint32_t)H * DK * 2, tok_v = (uint32_t)H * DV * 2;   // bytes per token

  // ---- chunk c into buffer set b.  Rows past the chunk repeat its last
  // row: they meet zero coefficients only.  Straight-line per wave, C::VM
  // copies: K fragments (bt, m = w), record fragments w, w + W, .., the
  // gate block and one value block (copies beyond the blocks' count repeat
  // the last one: the same bytes to the same place) ----
  auto issue_chunk = [&](int b, int c) {
    char *buf = smem + b * C::BUF;
    const int t0 = tbeg + c * CH, lm = min(CH, tend - t0) - 1;
    const char *kb = reinterpret_cast<const char *>(gk + ((int64_t)t0 * H + h) * DK) + 16 * g4 + 64 * w;
    const char *rec = grec + ((slot0 + c) * H + h) * (int64_t)(kRecFloats * 4) + 16 * l;
    const char *vb = reinterpret_cast<const char *>(gv + ((int64_t)t0 * H + h) * DV + 16 * tile);
#pragma unroll
    for (int bt = 0; bt < 4; ++bt)
      dma16_global(kb + (uint32_t)min(16 * bt + jl, lm) * tok_k, (lds_void *)(buf + (C::bKA + bt * NKS + w) * 1024));
#pragma unroll
    for (int j = 0; j < C::NTF / W; ++j)
      dma16_global(rec + (j * W + w) * 1024, (lds_void *)(buf + (C::bTF + j * W + w) * 1024));
    dma16_global(rec + kRecGateOffsetBytes, (lds_void *)(buf + C::bG * 1024));
    {
      const int f = min(w, C::NVB - 1);
      const int u = f * 64 + l;   // token u / 2, columns 8 (u & 1) ..
      dma16_global(vb + (uint32_t)min(u >> 1, lm) * tok_v + 16 * (u & 1), (lds_void *)(buf + (C::bV + f) * 1024));
    }
  };
  static_assert(C::NVB <= 2 && (W >= 2), "value blocks: one per wave");
  // wait until the copies of chunk c have landed, when chunks up to c + k
  // (k = 0, 1, 2) have been issued after it
  auto wait_chunk = [&](int k) {
    if (k >= 2)
      wait_vmem_le<2 * C::VM>();
    else if (k == 1)
      wait_vmem_le<C::VM>();
    else
      wait_vmem();
  };

  // LDS byte addresses (buffer set 0): transposing reads of the staged keys
  // for S^T blocks 2w, 2w + 1 (key row 4 g4 + (jl >> 2) of a 16-row block,
  // 8-column group jl & 3, k-step w), and of the value columns of token
  // block w (token 16 w + 4 g4 + (jl >> 2), columns 4 (jl & 3) ..; block
  // w + W is 512 W bytes further).
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void *)smem;
  const uint32_t kt_lds = lds0 + C::bKA * 1024 + 1024u * w + 16u * (4 * g4 + (jl >> 2) + 16 * (jl & 3));
  const uint32_t v_lds = lds0 + C::bV * 1024 + 32u * (16 * w + 4 * g4 + (jl >> 2)) + 8u * (jl & 3);
  char *sY = smem + C::oY, *sR = smem + C::oR, *sD = smem + C::oD;
  // R / D' of token block bt: hi at [bt >> 1][0][lane][8 (bt & 1)], lo at [bt >> 1][1]
  const uint32_t r_lds = lds0 + (uint32_t)C::oR + 16u * l;

  // ---- a chunk's operands in registers ----
  struct Ops {
    bf16x8 ka[4];                 // K fragments (bt, m = w)
    bf16x8 th[NB][2], tl[NB][2];  // Tau diag(beta) fragments (bt, m) of the wave's token blocks
    f32x4 eg[NB], dec[NB];        // e^g, e^{g_L - g} at the wave's tokens (C layout)
    float egl;
    uint2 vt[NB];                 // value columns of the wave's token blocks (C layout)
    uint2 kr[2][2][2];            // K^T fragment halves: block 2w + j, token half m, +16 tokens
  };
  // operand reads from buffer set b; the transposing reads are waited for
  // by tr_wait (they are older than any LDS read the compiler issues after
  // them, so its own counted waits stay valid); within a group of reads the
  // results are early-clobber operands, since a read's data may land before
  // a later read of the group has taken its address
  auto load_ops = [&](int b, Ops &o) {
    const char *buf = smem + b * C::BUF;
    const uint32_t boff = (uint32_t)(b * C::BUF);
#pragma unroll
    for (int i = 0; i < NB; ++i)
      asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(o.vt[i]) : "v"(v_lds + boff + (uint32_t)(512 * W * i)));
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const uint32_t a0 = kt_lds + boff + (uint32_t)(2 * m * NKS * 1024), a1 = a0 + (uint32_t)(NKS * 1024);
      asm volatile(
          "ds_read_b64_tr_b16 %0, %4\n\t"
          "ds_read_b64_tr_b16 %1, %5\n\t"
          "ds_read_b64_tr_b16 %2, %4 offset:8\n\t"
          "ds_read_b64_tr_b16 %3, %5 offset:8"
          : "=&v"(o.kr[0][m][0]), "=&v"(o.kr[0][m][1]), "=&v"(o.kr[1][m][0]), "=&v"(o.kr[1][m][1])
          : "v"(a0), "v"(a1));
    }
#pragma unroll
    for (int bt = 0; bt < 4; ++bt)
      o.ka[bt] = *reinterpret_cast<const bf16x8 *>(buf + (C::bKA + bt * NKS + w) * 1024 + 16 * l);
    const float *gr = reinterpret_cast<const float *>(buf + C::bG * 1024);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int bt = w + W * i;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        // fragments (bt, m), m <= bt / 2: f = bt for bt < 2, else 2 + 2 (bt - 2) + m
        const int f = bt < 2 ? bt : 2 + 2 * (bt - 2) + m;
        if (2 * m <= bt) {
          o.th[i][m] = *reinterpret_cast<const bf16x8 *>(buf + (C::bTF + f) * 1024 + 16 * l);
          o.tl[i][m] = *reinterpret_cast<const bf16x8 *>(buf + (C::bTF + kTauFrags + f) * 1024 + 16 * l);
        }
      }
      o.eg[i] = *reinterpret_cast<const f32x4 *>(gr + 16 * bt + 4 * g4);
      o.dec[i] = *reinterpret_cast<const f32x4 *>(gr + 64 + 16 * bt + 4 * g4);
    }
    o.egl = gr[128];
  };
  auto tr_wait = [&](Ops &o) {
    if constexpr (NB == 1)
      asm volatile("s_waitcnt lgkmcnt(0)"
                   : "+v"(o.vt[0]), "+v"(o.kr[0][0][0]), "+v"(o.kr[0][0][1]), "+v"(o.kr[1][0][0]),
                     "+v"(o.kr[1][0][1]), "+v"(o.kr[0][1][0]), "+v"(o.kr[0][1][1]), "+v"(o.kr[1][1][0]),
                     "+v"(o.kr[1][1][1]));
    else
      asm volatile("s_waitcnt lgkmcnt(0)"
                   : "+v"(o.vt[0]), "+v"(o.vt[1]), "+v"(o.kr[0][0][0]), "+v"(o.kr[0][0][1]), "+v"(o.kr[1][0][0]),
                     "+v"(o.kr[1][0][1]), "+v"(o.kr[0][1][0]), "+v"(o.kr[0][1][1]), "+v"(o.kr[1][1][0]),
                     "+v"(o.kr[1][1][1]));
  };

  // ---- prologue: chunks 0 .. 2 in flight, chunk 0's operands ----
  Ops cur;
  if (nch > 0) {
    issue_chunk(0, 0);
    if (nch > 1) issue_chunk(1, 1);
    if (nch > 2) issue_chunk(2, 2);
    wait_chunk(min(nch - 1, 2));
    lds_barrier();
    load_ops(0, cur);
    tr_wait(cur);
  }
  bf16x8 sh, sl;
  b_frag_split(st[0], st[1], sh, sl);

  int b = 0;   // buffer set of chunk c
  for (int c = 0; c < nch; ++c) {
    const int b1 = b == 2 ? 0 : b + 1;   // buffer set of chunk c + 1
    // ---- Y_w = K[:, 32w..] S^T[32w.., :], all four token blocks ----
    {
      f32x4 y[4], yl[4];
#pragma unroll
      for (int bt = 0; bt < 4; ++bt) {
        y[bt] = mfma_bf16(cur.ka[bt], sh, zero4());
        yl[bt] = mfma_bf16(cur.ka[bt], sl, zero4());
      }
#pragma unroll
      for (int bt = 0; bt < 4; ++bt)
        *reinterpret_cast<f32x4 *>(sY + (w * 4 + bt) * 1024 + 16 * l) = y[bt] + yl[bt];
    }
    lds_barrier();
    // every wave has read chunk c's buffer set (a chunk earlier): it takes
    // chunk c + 3
    if (c + 3 < nch) issue_chunk(b, c + 3);

    // ---- token blocks bt = w, w + W, ..: Y, R = V - e^g Y, split-bf16 R ----
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int bt = w + W * i;
      f32x4 y = *reinterpret_cast<const f32x4 *>(sY + bt * 1024 + 16 * l);
#pragma unroll
      for (int v = 1; v < W; ++v) y += *reinterpret_cast<const f32x4 *>(sY + (v * 4 + bt) * 1024 + 16 * l);
      const uint2 x = cur.vt[i];
      const float vv[4] = {__uint_as_float(x.x << 16), __uint_as_float(x.x & 0xffff0000u),
                           __uint_as_float(x.y << 16), __uint_as_float(x.y & 0xffff0000u)};
      uint2 rh, rl;
      split2(vv[0] - cur.eg[i][0] * y[0], vv[1] - cur.eg[i][1] * y[1], rh.x, rl.x);
      split2(vv[2] - cur.eg[i][2] * y[2], vv[3] - cur.eg[i][3] * y[3], rh.y, rl.y);
      const uint32_t a = r_lds + (uint32_t)((bt >> 1) * 2048 + 8 * (bt & 1));
      lds_store8(a, rh);
      lds_store8(a + 1024, rl);
    }
    // the copies of chunk c + 1 (issued before those of c + 2 and c + 3)
    // have landed; the barrier covers every wave's
    const bool more = c + 1 < nch;
    if (more) wait_chunk(min(nch - 1, c + 3) - (c + 1));
    lds_barrier();
    Ops nxt;
    if (more) load_ops(b1, nxt);

    // ---- token blocks bt: D = (Tau diag(beta)) R, D' = e^{g_L - g} D ----
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int bt = w + W * i;
      f32x4 d0 = zero4(), d1 = zero4(), d2 = zero4();
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        if (2 * m <= bt) {
          const bf16x8 rh = *reinterpret_cast<const bf16x8 *>(sR + m * 2048 + 16 * l);
          const bf16x8 rl = *reinterpret_cast<const bf16x8 *>(sR + m * 2048 + 1024 + 16 * l);
          d0 = mfma_bf16(cur.th[i][m], rh, d0);
          d1 = mfma_bf16(cur.th[i][m], rl, d1);
          d2 = mfma_bf16(cur.tl[i][m], rh, d2);
        }
      }
      const f32x4 d = d0 + d1 + d2;
      uint2 eh, el;
      split2(d[0] * cur.dec[i][0], d[1] * cur.dec[i][1], eh.x, el.x);
      split2(d[2] * cur.dec[i][2], d[3] * cur.dec[i][3], eh.y, el.y);
      const uint32_t a = r_lds + (uint32_t)(C::oD - C::oR + (bt >> 1) * 2048 + 8 * (bt & 1));
      lds_store8(a, eh);
      lds_store8(a + 1024, el);
    }
    lds_barrier();

    // ---- S^T <- e^{g_L} S^T + K^T D' (this wave's two dk blocks) ----
    {
      bf16x8 eh[2], el[2];
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        eh[m] = *reinterpret_cast<const bf16x8 *>(sD + m * 2048 + 16 * l);
        el[m] = *reinterpret_cast<const bf16x8 *>(sD + m * 2048 + 1024 + 16 * l);
      }
      f32x4 u[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int e = 0; e < 4; ++e) st[j][e] *= cur.egl;
        u[j] = zero4();
      }
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const bf16x8 kt = cat_bf16x8(cur.kr[j][m][0], cur.kr[j][m][1]);
          st[j] = mfma_bf16(kt, eh[m], st[j]);
          u[j] = mfma_bf16(kt, el[m], u[j]);
        }
      if (more) tr_wait(nxt);
#pragma unroll
      for (int j = 0; j < 2; ++j) st[j] += u[j];
    }
    b_frag_split(st[0], st[1], sh, sl);
    if (more) cur = nxt;
    b = b1;
  }

  if (p.S_out) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
      *reinterpret_cast<f32x4 *>(p.S_out + (((int64_t)n * H + h) * DV + row) * DK + 32 * w + 8 * g4 + 4 * j) = st[j];
  }
}

template <int DK>
hipError_t launch_d(const ChainLaunch &p, hipStream_t stream) {
  if (p.dv % 16 != 0) return hipErrorInvalidValue;
  const int64_t items = (int64_t)p.n_seqs * p.H * (p.dv / 16);
  if (items <= 0) return hipSuccess;
  const int64_t grid = (items + 7) / 8 * 8;
  hipLaunchKernelGGL((chain_dks_kernel<DK>), dim3((unsigned)grid), dim3(DK / 32 * 64), 0, stream, p, (int)items);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chain_dks(const ChainLaunch &p, hipStream_t stream) {
  if (p.o || p.tiles_T != 0 || p.n_segs != 1) return hipErrorInvalidValue;
  if (p.dk == 64) return launch_d<64>(p, stream);
  if (p.dk == 128) return launch_d<128>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace gdn
