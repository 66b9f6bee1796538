// gdn_compose.hip -- back-to-back composition of affine chunk operators.
//
// Page "LinearKV: One Cached State Suffices for Position-Independent Caching
// in Hybrid LLMs", composition paragraph: chunk c's output state is chunk
// c+1's input, S <- S T_C[c] + S_local[c], in context order.
//
// Per head this is a chain of dv x dk x dk products.  Rows of S are
// independent, so a workgroup owns 16 rows of one head and walks the chunks;
// the dk x dk operator of each step is staged transposed in LDS (all row
// tiles of a head read the same operator, on the same XCD, through L2).
// Both operands are fp32 and carried as split bf16 (three products), which
// keeps the product within a few fp32 ulps of the fp32 result.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int CNW = 8;
constexpr int CNT = CNW * 64;

template <int DK>
__global__ void __launch_bounds__(CNT) compose_kernel(ComposeLaunch p, int n_items) {
  constexpr int LDT = DK + 4;  // sTt [DK][LDT]: sTt[j][m] = T_C[m][j]
  constexpr int LDS_ = DK + 4; // sS  [16][LDS_]
  __shared__ __attribute__((aligned(16))) float sTt[DK * LDT];
  __shared__ __attribute__((aligned(16))) float sS[16 * LDS_];

  const int per = (int)(gridDim.x >> 3);
  const int item = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
  if (item >= n_items) return;
  const int tiles = p.dv / 16;
  const int h = item / tiles, row0 = 16 * (item % tiles);
  const int H = p.H, DV = p.dv;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id();
  constexpr int NST = DK / 16;
  const bool owns = w < NST;
  const int col = 16 * w + (l & 15);

  f32x4 sacc = zero4();
  if (owns && p.S_in) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      sacc[i] = p.S_in[((int64_t)h * DV + row0 + 4 * (l >> 4) + i) * DK + col];
  }
  for (int c = 0; c < p.n_chunks; ++c) {
    if (owns) store_tile(sS, LDS_, 0, 16 * w, sacc);
    const float *T = p.T_C + ((int64_t)c * H + h) * DK * DK;
    for (int s = tid; s < DK * DK / 4; s += CNT) {
      const int m = s / (DK / 4), j4 = (s % (DK / 4)) * 4;
      const f32x4 x = *reinterpret_cast<const f32x4 *>(T + m * DK + j4);
#pragma unroll
      for (int e = 0; e < 4; ++e) sTt[(j4 + e) * LDT + m] = x[e];
    }
    f32x4 loc = zero4();
    if (owns) {
      const float *Lp = p.S_local + ((int64_t)c * H + h) * DV * DK;
#pragma unroll
      for (int i = 0; i < 4; ++i) loc[i] = Lp[(int64_t)(row0 + 4 * (l >> 4) + i) * DK + col];
    }
    __syncthreads();
    if (owns) {
      f32x4 acc = loc;
      mma_bf16<2, 2>(acc, RowMajor<float>{sS, LDS_}, RowMajor<float>{sTt, LDT}, 0, 16 * w, 0, DK);
      sacc = acc;
    }
    __syncthreads();
  }
  if (owns) {
#pragma unroll
    for (int i = 0; i < 4; ++i) p.S_out[((int64_t)h * DV + row0 + 4 * (l >> 4) + i) * DK + col] = sacc[i];
  }
}

template <int DK>
hipError_t launch_c(const ComposeLaunch &p, hipStream_t stream) {
  const int64_t items = (int64_t)p.H * (p.dv / 16);
  if (items <= 0) return hipSuccess;
  const int64_t grid = (items + 7) / 8 * 8;
  hipLaunchKernelGGL((compose_kernel<DK>), dim3((unsigned)grid), dim3(CNT), 0, stream, p, (int)items);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Composition of time-split segments (one sequence's segment operators, in
// order): S = S_seg[0], then S <- S T_seg[s] + S_seg[s].  T_seg arrives
// transposed (T^T row-major), so the A operand of S_new^T = T^T S^T comes
// straight from global memory, 8 consecutive floats per lane.  Workgroup =
// 4 waves on 16 rows of one (sequence, head); wave w owns dk blocks
// w * NOB .. w * NOB + NOB - 1 of S^T (C layout, natural dk order) and the
// full S^T operand is exchanged through LDS once per step.  The operands of
// step s + 1 (which do not depend on the running state) are loaded into
// registers while step s computes.
// ---------------------------------------------------------------------------
constexpr int SNW = 4;

template <int DK>
struct SegOps {
  static constexpr int NOB = DK / 16 / SNW;
  static constexpr int NKS = DK / 32;
  f32x4 t[NOB][NKS][2];  // rows 16 jb + (l & 15) of T^T, 8 floats per k = 32 step
  f32x4 loc[NOB];        // S_seg rows
};

template <int DK>
__global__ void __launch_bounds__(SNW * 64) seg_compose_kernel(SegComposeLaunch p, int n_items) {
  constexpr int LDS_ = DK + 4;
  constexpr int NOB = SegOps<DK>::NOB;
  constexpr int NKS = SegOps<DK>::NKS;
  __shared__ __attribute__((aligned(16))) float sS[16 * LDS_];

  const int per = (int)(gridDim.x >> 3);
  const int item = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
  if (item >= n_items) return;
  const int tiles = p.dv / 16;
  const int nh = item / tiles, row0 = 16 * (item % tiles);
  const int n = nh / p.H, h = nh % p.H;
  const int H = p.H, DV = p.dv, P = p.n_segs;
  const int w = __builtin_amdgcn_readfirstlane(wave_id()), l = lane_id(), g4 = l >> 4, jl = l & 15;

  auto seg_state = [&](int s) { return p.S_seg + (((int64_t)n * P + s) * H + h) * DV * DK; };
  auto load = [&](int s, SegOps<DK> &o) {
    const float *Tt = p.Tt_seg + (((int64_t)n * P + s) * H + h) * DK * DK;
    const float *Ls = seg_state(s);
#pragma unroll
    for (int i = 0; i < NOB; ++i) {
      const int jb = w * NOB + i;
      o.loc[i] = *reinterpret_cast<const f32x4 *>(Ls + (int64_t)(row0 + jl) * DK + 16 * jb + 4 * g4);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const float *a = Tt + (int64_t)(16 * jb + jl) * DK + 32 * ks + 8 * g4;
        o.t[i][ks][0] = *reinterpret_cast<const f32x4 *>(a);
        o.t[i][ks][1] = *reinterpret_cast<const f32x4 *>(a + 4);
      }
    }
  };
  f32x4 acc[NOB];
#pragma unroll
  for (int i = 0; i < NOB; ++i)
    acc[i] = *reinterpret_cast<const f32x4 *>(seg_state(0) + (int64_t)(row0 + jl) * DK + 16 * (w * NOB + i) + 4 * g4);

  auto step = [&](const SegOps<DK> &o) {
#pragma unroll
    for (int i = 0; i < NOB; ++i)
      *reinterpret_cast<f32x4 *>(sS + jl * LDS_ + 16 * (w * NOB + i) + 4 * g4) = acc[i];
    lds_barrier();
    bf16x8 bh[NKS], bl[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const f32x4 x0 = *reinterpret_cast<const f32x4 *>(sS + jl * LDS_ + 32 * ks + 8 * g4);
      const f32x4 x1 = *reinterpret_cast<const f32x4 *>(sS + jl * LDS_ + 32 * ks + 8 * g4 + 4);
      b_frag_split(x0, x1, bh[ks], bl[ks]);
    }
    // three accumulators per block (one per split pass), rotated so that no
    // product waits on the one just issued
    f32x4 c0[NOB], c1[NOB], c2[NOB];
#pragma unroll
    for (int i = 0; i < NOB; ++i) {
      c0[i] = o.loc[i];
      c1[i] = c2[i] = zero4();
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      bf16x8 ah[NOB], al[NOB];
#pragma unroll
      for (int i = 0; i < NOB; ++i) b_frag_split(o.t[i][ks][0], o.t[i][ks][1], ah[i], al[i]);
#pragma unroll
      for (int i = 0; i < NOB; ++i) c0[i] = mfma_bf16(ah[i], bh[ks], c0[i]);
#pragma unroll
      for (int i = 0; i < NOB; ++i) c1[i] = mfma_bf16(ah[i], bl[ks], c1[i]);
#pragma unroll
      for (int i = 0; i < NOB; ++i) c2[i] = mfma_bf16(al[i], bh[ks], c2[i]);
    }
#pragma unroll
    for (int i = 0; i < NOB; ++i) acc[i] = c0[i] + c1[i] + c2[i];
    lds_barrier();
  };

  SegOps<DK> o0, o1;
  if (P > 1) load(1, o0);
  for (int s = 1; s < P; s += 2) {
    if (s + 1 < P) load(s + 1, o1);
    step(o0);
    if (s + 1 >= P) break;
    if (s + 2 < P) load(s + 2, o0);
    step(o1);
  }
  float *out = p.S_out + ((int64_t)n * H + h) * DV * DK;
#pragma unroll
  for (int i = 0; i < NOB; ++i)
    *reinterpret_cast<f32x4 *>(out + (int64_t)(row0 + jl) * DK + 16 * (w * NOB + i) + 4 * g4) = acc[i];
}

template <int DK>
hipError_t launch_sc(const SegComposeLaunch &p, hipStream_t stream) {
  const int64_t items = (int64_t)p.n_seqs * p.H * (p.dv / 16);
  if (items <= 0) return hipSuccess;
  const int64_t grid = (items + 7) / 8 * 8;
  hipLaunchKernelGGL((seg_compose_kernel<DK>), dim3((unsigned)grid), dim3(SNW * 64), 0, stream, p, (int)items);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_seg_compose(const SegComposeLaunch &p, hipStream_t stream) {
  if (p.dk == 64) return launch_sc<64>(p, stream);
  if (p.dk == 128) return launch_sc<128>(p, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_compose(const ComposeLaunch &p, hipStream_t stream) {
  if (p.dk == 64) return launch_c<64>(p, stream);
  if (p.dk == 128) return launch_c<128>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace gdn
