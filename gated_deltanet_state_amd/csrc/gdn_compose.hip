// gdn_compose.hip -- back-to-back composition of affine chunk operators.
//
// Page "LinearKV: One Cached State Suffices for Position-Independent Caching
// in Hybrid LLMs", composition paragraph: chunk c's output state is chunk
// c+1's input, S <- S T_C[c] + S_local[c], in context order.
//
// Per head this is a chain of dv x dk x dk products.  Rows of S are
// independent, so a workgroup owns 32 rows of one head and walks the
// operators; each operator enters the products as split-bf16 MFMA
// fragments (three products per step keep the result within a few fp32
// ulps of the fp32 product).  Operators that arrive as fp32 matrices
// (gdn_compose) are first converted to that fragment form by a fully
// parallel pass; the time-split replay writes its segment operators in that
// form directly.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

// ---------------------------------------------------------------------------
// fp32 operators [n, dk, dk] (row-major) -> composition fragments (the
// layout of gdn_internal.h: fragment f = jb * (dk / 32) + ks, lane (q, g)
// holds T[32 ks + 8 g + i][16 jb + q], i < 8, hi plane then lo plane).  One
// workgroup per (operator, 32-row step ks): coalesced reads of its 32 rows
// into LDS, then every wave reads the columns of its fragments and writes
// them split, 1 KiB per fragment.  (16 KiB of LDS per workgroup, so many
// workgroups share a compute unit and hide each other's load latency.)
// ---------------------------------------------------------------------------
constexpr int FNW = 4;

template <int DK>
__global__ void __launch_bounds__(FNW * 64) op_frag_kernel(const float *T, char *frag) {
  constexpr int LD = DK + 4, NKS = DK / 32, NSB = DK / 16, NF = NSB * NKS;
  __shared__ __attribute__((aligned(16))) float sT[32 * LD];
  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), g4 = l >> 4, jl = l & 15;
  const int64_t op = blockIdx.x / NKS;
  const int ks = (int)(blockIdx.x % NKS);
  const float *src = T + op * DK * DK + (int64_t)32 * ks * DK;
  char *dst = frag + op * (2 * NF * 1024);
  for (int i = tid; i < 32 * DK / 4; i += FNW * 64) {
    const int m = i / (DK / 4), j4 = (i % (DK / 4)) * 4;
    *reinterpret_cast<f32x4 *>(sT + m * LD + j4) = *reinterpret_cast<const f32x4 *>(src + (int64_t)m * DK + j4);
  }
  __syncthreads();
  for (int jb = w; jb < NSB; jb += FNW) {
    const int f = jb * NKS + ks;
    float x[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) x[t] = sT[(8 * g4 + t) * LD + 16 * jb + jl];
    bf16x8 hi, lo;
    split8(x, hi, lo);
    *reinterpret_cast<bf16x8 *>(dst + f * 1024 + 16 * l) = hi;
    *reinterpret_cast<bf16x8 *>(dst + (NF + f) * 1024 + 16 * l) = lo;
  }
}

template <int DK>
hipError_t launch_of(const float *T, int64_t n_ops, void *frag, hipStream_t stream) {
  if (n_ops <= 0) return hipSuccess;
  return launch_kernel(op_frag_kernel<DK>, dim3((unsigned)(n_ops * (DK / 32))), dim3(FNW * 64), 0, stream, T,
                       static_cast<char *>(frag));
}

// ---------------------------------------------------------------------------
// Composition of one sequence's operators in order: S = S_seg[0] (time
// split: segment 0 already started from S0), or S = S0 with every operator
// applied (from_start: gdn_compose), then S <- S T_seg[s] + S_seg[s],
// computed as S_new^T = T^T S^T + S_seg^T.  The operators arrive as
// split-bf16 MFMA fragments (gdn_internal.h).
// Workgroup = 4 waves on 32 rows (RTC = 2 row tiles) of one (sequence,
// head), or on 16 rows (RTC = 1) when the 32-row workgroups would leave
// compute units idle (the chain is bound by its per-step latency, so twice
// the workgroups halve each one's products: 64 operators over 32 heads in
// 0.130 against 0.149 ms); wave w owns dk
// blocks JBW w .. JBW w + JBW - 1 of S^T (C layout) for its row tiles,
// so it needs only its own fragments of each operator: those, and its rows
// of each local state, are loaded straight into registers two steps ahead
// (three register sets in rotation), which hides the load latency of the
// serial chain.  Per step the waves exchange the new S rows through LDS,
// already split into bf16 hi and lo planes.
// ---------------------------------------------------------------------------
constexpr int SNW = 4;

template <int DK>
struct SegCfg {
  static constexpr int NSB = DK / 16, NKS = DK / 32;
  static constexpr int JBW = NSB / SNW;              // dk blocks per wave
  static constexpr int NF = NSB * NKS;               // fragments per plane
  static constexpr int OPB = 2 * NF * 1024;          // bytes of one operator (both planes)
  static constexpr int LDB = DK + 8;                 // row pitch of the split S planes (bf16)
};

// One step's operands of a wave: its operator fragments (hi, lo) and its
// rows of the local state.
template <int DK, int RTC>
struct StepRegs {
  bf16x8 h[SegCfg<DK>::JBW][SegCfg<DK>::NKS], l[SegCfg<DK>::JBW][SegCfg<DK>::NKS];
  f32x4 loc[RTC][SegCfg<DK>::JBW];
};

template <int DK, int RTC, bool PRE>
__global__ void __launch_bounds__(SNW * 64) seg_compose_kernel(SegComposeLaunch p, int n_items) {
  using C = SegCfg<DK>;
  constexpr int NKS = C::NKS, JBW = C::JBW, NF = C::NF, LDB = C::LDB;
  constexpr int NP = RTC == 1 ? 3 : 1;   // accumulators per product (the split passes apart when few rotate)
  __shared__ __attribute__((aligned(16))) bf16 sSh[16 * RTC * LDB];
  __shared__ __attribute__((aligned(16))) bf16 sSl[16 * RTC * LDB];

  const int per = (int)(gridDim.x >> 3);
  const int item = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
  if (item >= n_items) return;
  const int groups = p.dv / (16 * RTC);
  const int nh = item / groups, rg = item % groups;
  const int n = nh / p.H, h = nh % p.H;
  const int H = p.H, DV = p.dv, P = p.n_segs;
  const int w = __builtin_amdgcn_readfirstlane(wave_id()), l = lane_id(), g4 = l >> 4, jl = l & 15;
  const int jb0 = JBW * w;
  // lane's element offset of row tile rt, dk block jb0 + i: row 32 rg + 16 rt + jl, columns 16 jb + 4 g4 ..
  auto eoff = [&](int rt, int i) { return (int64_t)(16 * RTC * rg + 16 * rt + jl) * DK + 16 * (jb0 + i) + 4 * g4; };
  const int64_t head = ((int64_t)n * H + h) * DV * DK;

  auto load = [&](int s, StepRegs<DK, RTC> &R) {
    const char *op = reinterpret_cast<const char *>(p.T_frag) + (((int64_t)n * P + s) * H + h) * (int64_t)C::OPB + 16 * l;
#pragma unroll
    for (int i = 0; i < JBW; ++i)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int f = (jb0 + i) * NKS + ks;
        R.h[i][ks] = *reinterpret_cast<const bf16x8 *>(op + f * 1024);
        R.l[i][ks] = *reinterpret_cast<const bf16x8 *>(op + (NF + f) * 1024);
      }
    const float *Ls = p.S_seg + (((int64_t)n * P + s) * H + h) * DV * DK;
#pragma unroll
    for (int rt = 0; rt < RTC; ++rt)
#pragma unroll
      for (int i = 0; i < JBW; ++i) R.loc[rt][i] = *reinterpret_cast<const f32x4 *>(Ls + eoff(rt, i));
  };

  f32x4 acc[RTC][JBW];
  const int s0 = p.from_start ? 0 : 1;   // first operator applied
  {
    // the state entering the chain: S0 (or zero), or segment 0's own state
    // (S0 may alias S_out: every workgroup reads its own rows here, first)
    const float *src = (p.from_start || PRE) ? (p.S0 ? p.S0 + head : nullptr) : nullptr;
#pragma unroll
    for (int rt = 0; rt < RTC; ++rt)
#pragma unroll
      for (int i = 0; i < JBW; ++i) acc[rt][i] = src ? *reinterpret_cast<const f32x4 *>(src + eoff(rt, i)) : zero4();
    if (PRE) {   // the state entering segment 0
      float *pre = p.S_prefix + ((int64_t)n * P * H + h) * DV * DK;
#pragma unroll
      for (int rt = 0; rt < RTC; ++rt)
#pragma unroll
        for (int i = 0; i < JBW; ++i) *reinterpret_cast<f32x4 *>(pre + eoff(rt, i)) = acc[rt][i];
    }
    if (!p.from_start) {
      const float *L0 = p.S_seg + ((int64_t)n * P * H + h) * DV * DK;
#pragma unroll
      for (int rt = 0; rt < RTC; ++rt)
#pragma unroll
        for (int i = 0; i < JBW; ++i) acc[rt][i] = *reinterpret_cast<const f32x4 *>(L0 + eoff(rt, i));
    }
  }

  auto step = [&](int s, const StepRegs<DK, RTC> &R) {
    if (PRE) {   // the state entering segment s
      float *pre = p.S_prefix + (((int64_t)n * P + s) * H + h) * DV * DK;
#pragma unroll
      for (int rt = 0; rt < RTC; ++rt)
#pragma unroll
        for (int i = 0; i < JBW; ++i) *reinterpret_cast<f32x4 *>(pre + eoff(rt, i)) = acc[rt][i];
    }
    // this wave's columns of both row tiles, split, to LDS
#pragma unroll
    for (int rt = 0; rt < RTC; ++rt)
#pragma unroll
      for (int i = 0; i < JBW; ++i) {
        bf16x4 hi, lo;
        split4(acc[rt][i], hi, lo);
        const int o = (16 * rt + jl) * LDB + 16 * (jb0 + i) + 4 * g4;
        *reinterpret_cast<bf16x4 *>(sSh + o) = hi;
        *reinterpret_cast<bf16x4 *>(sSl + o) = lo;
      }
    lds_barrier();
    f32x4 c[NP][RTC][JBW];
#pragma unroll
    for (int rt = 0; rt < RTC; ++rt)
#pragma unroll
      for (int i = 0; i < JBW; ++i) {
        c[0][rt][i] = R.loc[rt][i];
#pragma unroll
        for (int q = 1; q < NP; ++q) c[q][rt][i] = zero4();
      }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      bf16x8 bh[RTC], bl[RTC];
#pragma unroll
      for (int rt = 0; rt < RTC; ++rt) {
        const int o = (16 * rt + jl) * LDB + 32 * ks + 8 * g4;
        bh[rt] = *reinterpret_cast<const bf16x8 *>(sSh + o);
        bl[rt] = *reinterpret_cast<const bf16x8 *>(sSl + o);
      }
      // the three split passes share each accumulator when 2 JBW of them
      // rotate (two row tiles), else each pass has its own
#pragma unroll
      for (int rt = 0; rt < RTC; ++rt)
#pragma unroll
        for (int i = 0; i < JBW; ++i) c[0][rt][i] = mfma_bf16(R.h[i][ks], bh[rt], c[0][rt][i]);
#pragma unroll
      for (int rt = 0; rt < RTC; ++rt)
#pragma unroll
        for (int i = 0; i < JBW; ++i) c[NP > 1 ? 1 : 0][rt][i] = mfma_bf16(R.h[i][ks], bl[rt], c[NP > 1 ? 1 : 0][rt][i]);
#pragma unroll
      for (int rt = 0; rt < RTC; ++rt)
#pragma unroll
        for (int i = 0; i < JBW; ++i) c[NP > 1 ? 2 : 0][rt][i] = mfma_bf16(R.l[i][ks], bh[rt], c[NP > 1 ? 2 : 0][rt][i]);
    }
    lds_barrier();   // every wave has read the planes before the next step rewrites them
#pragma unroll
    for (int rt = 0; rt < RTC; ++rt)
#pragma unroll
      for (int i = 0; i < JBW; ++i) {
        acc[rt][i] = c[0][rt][i];
#pragma unroll
        for (int q = 1; q < NP; ++q) acc[rt][i] += c[q][rt][i];
      }
  };

  // operators applied: s0 .. PE - 1 (lead layout: the last segment has none,
  // and the state entering it is the result)
  const int PE = p.lead ? P - 1 : P;
  if (s0 < PE) {
    // The waits for the prefetched registers are counted by the compiler
    // from the order of the memory operations, which is therefore the same
    // on every path: the entering state has landed before the first
    // prefetch, the prefetches are unconditional (past the last operator
    // they load the last one again) and stores depend on a template
    // argument only.  Otherwise a use inside the loop waits for every load
    // outstanding, the prefetch of two steps ahead included.
    wait_vmem();
    auto nxt = [&](int s) { return s < PE ? s : PE - 1; };
    StepRegs<DK, RTC> R0, R1, R2;
    load(s0, R0);
    load(nxt(s0 + 1), R1);
    for (int s = s0; s < PE; s += 3) {
      load(nxt(s + 2), R2);
      step(s, R0);
      if (s + 1 >= PE) break;
      load(nxt(s + 3), R0);
      step(s + 1, R1);
      if (s + 2 >= PE) break;
      load(nxt(s + 4), R1);
      step(s + 2, R2);
    }
  }
  float *out = PRE && p.lead ? p.S_prefix + (((int64_t)n * P + P - 1) * H + h) * DV * DK : p.S_out + head;
#pragma unroll
  for (int rt = 0; rt < RTC; ++rt)
#pragma unroll
    for (int i = 0; i < JBW; ++i) *reinterpret_cast<f32x4 *>(out + eoff(rt, i)) = acc[rt][i];
}

template <int DK>
hipError_t launch_sc(const SegComposeLaunch &p, hipStream_t stream) {
  if (p.dv % 32 != 0 || (p.lead && (p.from_start || !p.S_prefix || p.n_segs < 2))) return hipErrorInvalidValue;
  const int64_t items32 = (int64_t)p.n_seqs * p.H * (p.dv / 32);
  if (items32 <= 0) return hipSuccess;
  // 32-row workgroups, or 16-row ones while 32-row ones leave compute units idle
  const bool pre = p.S_prefix != nullptr;
  if (items32 >= 256) {
    const int64_t grid = (items32 + 7) / 8 * 8;
    return launch_kernel(pre ? seg_compose_kernel<DK, 2, true> : seg_compose_kernel<DK, 2, false>, dim3((unsigned)grid),
                         dim3(SNW * 64), 0, stream, p, (int)items32);
  }
  const int64_t items = 2 * items32, grid = (items + 7) / 8 * 8;
  return launch_kernel(pre ? seg_compose_kernel<DK, 1, true> : seg_compose_kernel<DK, 1, false>, dim3((unsigned)grid),
                       dim3(SNW * 64), 0, stream, p, (int)items);
}

}  // namespace

hipError_t launch_seg_compose(const SegComposeLaunch &p, hipStream_t stream) {
  if (p.dk == 64) return launch_sc<64>(p, stream);
  if (p.dk == 128) return launch_sc<128>(p, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_op_frags(const float *T, int64_t n_ops, int32_t dk, void *frag, hipStream_t stream) {
  if (dk == 64) return launch_of<64>(T, n_ops, frag, stream);
  if (dk == 128) return launch_of<128>(T, n_ops, frag, stream);
  return hipErrorInvalidValue;
}

}  // namespace gdn
