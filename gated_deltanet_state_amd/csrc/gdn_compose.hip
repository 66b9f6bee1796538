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
// order): S = S_seg[0], then S <- S T_seg[s] + S_seg[s], computed as
// S_new^T = T^T S^T + S_seg^T.  The operators arrive as split-bf16 MFMA
// fragments (gdn_internal.h), so a workgroup copies each step's operator
// into LDS once (load-to-LDS DMA, one step ahead, two buffers) and its
// waves read their A operands from there without converting anything.
// Workgroup = 4 waves on 32 rows of one (sequence, head): wave w owns rows
// 16 (w & 1) .. + 15 of the group and dk blocks (w >> 1) * NSB / 2 .. of
// S^T (C layout); the two halves of a row tile meet in LDS once per step.
// ---------------------------------------------------------------------------
constexpr int SNW = 4;

template <int DK>
struct SegCfg {
  static constexpr int NSB = DK / 16, NKS = DK / 32, HALF = NSB / 2;
  static constexpr int NF = NSB * NKS;               // fragments per plane
  static constexpr int OPB = 2 * NF * 1024;          // bytes of one operator (both planes)
  static constexpr int LDS_ = DK + 4;                // sS row pitch (floats)
  static constexpr size_t TOTAL = 2 * (size_t)OPB + 32 * LDS_ * 4;
  static_assert(TOTAL <= 160 * 1024, "LDS budget");
};

template <int DK>
__global__ void __launch_bounds__(SNW * 64) seg_compose_kernel(SegComposeLaunch p, int n_items) {
  using C = SegCfg<DK>;
  constexpr int NKS = C::NKS, HALF = C::HALF, NF = C::NF, LDS_ = C::LDS_;
  __shared__ __attribute__((aligned(16))) char smem[C::TOTAL];
  float *sS = reinterpret_cast<float *>(smem + 2 * C::OPB);

  const int per = (int)(gridDim.x >> 3);
  const int item = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
  if (item >= n_items) return;
  const int groups = p.dv / 32;
  const int nh = item / groups, rg = item % groups;
  const int n = nh / p.H, h = nh % p.H;
  const int H = p.H, DV = p.dv, P = p.n_segs;
  const int w = __builtin_amdgcn_readfirstlane(wave_id()), l = lane_id(), g4 = l >> 4, jl = l & 15;
  const int rsub = w & 1, jb0 = (w >> 1) * HALF;
  const int row = 32 * rg + 16 * rsub + jl;   // this lane's S row (C-layout column)

  auto seg_state = [&](int s) { return p.S_seg + (((int64_t)n * P + s) * H + h) * DV * DK; };
  auto seg_op = [&](int s) {
    return reinterpret_cast<const char *>(p.T_frag) + (((int64_t)n * P + s) * H + h) * (int64_t)C::OPB;
  };
  // operator of step s into LDS buffer b: 2 NF blocks of 1 KiB, NF / 2 per wave
  auto issue_op = [&](int s, int b) {
    const char *src = seg_op(s) + 16 * l;
    char *dst = smem + b * C::OPB;
#pragma unroll
    for (int j = 0; j < 2 * NF / SNW; ++j) {
      const int f = j * SNW + w;
      dma16_global(src + f * 1024, (lds_void *)(dst + f * 1024));
    }
  };
  auto load_loc = [&](int s, f32x4 (&loc)[HALF]) {
    const float *Ls = seg_state(s) + (int64_t)row * DK + 4 * g4;
#pragma unroll
    for (int i = 0; i < HALF; ++i) loc[i] = *reinterpret_cast<const f32x4 *>(Ls + 16 * (jb0 + i));
  };

  f32x4 acc[HALF], loc[HALF];
  if (p.S_prefix) {   // the state entering segment 0 (S0 may alias S_out: read it here, first)
    float *pre = p.S_prefix + ((int64_t)n * P * H + h) * DV * DK + (int64_t)row * DK + 4 * g4;
    const float *s0 = p.S0 ? p.S0 + ((int64_t)n * H + h) * DV * DK + (int64_t)row * DK + 4 * g4 : nullptr;
#pragma unroll
    for (int i = 0; i < HALF; ++i)
      *reinterpret_cast<f32x4 *>(pre + 16 * (jb0 + i)) = s0 ? *reinterpret_cast<const f32x4 *>(s0 + 16 * (jb0 + i)) : zero4();
  }
  load_loc(0, acc);
  if (P > 1) {
    issue_op(1, 0);
    load_loc(1, loc);
  }
  for (int s = 1; s < P; ++s) {
    const int b = (s - 1) & 1;
    if (p.S_prefix) {   // the state entering segment s
      float *pre = p.S_prefix + (((int64_t)n * P + s) * H + h) * DV * DK + (int64_t)row * DK + 4 * g4;
#pragma unroll
      for (int i = 0; i < HALF; ++i) *reinterpret_cast<f32x4 *>(pre + 16 * (jb0 + i)) = acc[i];
    }
    // this wave's half of its row tile to LDS; the operator of step s landed
#pragma unroll
    for (int i = 0; i < HALF; ++i)
      *reinterpret_cast<f32x4 *>(sS + (16 * rsub + jl) * LDS_ + 16 * (jb0 + i) + 4 * g4) = acc[i];
    f32x4 c0[HALF], c1[HALF], c2[HALF];
#pragma unroll
    for (int i = 0; i < HALF; ++i) {
      c0[i] = loc[i];
      c1[i] = c2[i] = zero4();
    }
    wait_vmem();
    lds_barrier();
    // next step's operator and local state are in flight while this one runs
    if (s + 1 < P) {
      issue_op(s + 1, b ^ 1);
      load_loc(s + 1, loc);
    }
    const char *op = smem + b * C::OPB;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      bf16x8 bh, bl;
      {
        const float *x = sS + (16 * rsub + jl) * LDS_ + 32 * ks + 8 * g4;
        b_frag_split(*reinterpret_cast<const f32x4 *>(x), *reinterpret_cast<const f32x4 *>(x + 4), bh, bl);
      }
      bf16x8 ah[HALF], al[HALF];
#pragma unroll
      for (int i = 0; i < HALF; ++i) {
        const int f = (jb0 + i) * NKS + ks;
        ah[i] = *reinterpret_cast<const bf16x8 *>(op + f * 1024 + 16 * l);
        al[i] = *reinterpret_cast<const bf16x8 *>(op + (NF + f) * 1024 + 16 * l);
      }
      // three accumulators per block (one per split pass), rotated so that
      // no product waits on the one just issued
#pragma unroll
      for (int i = 0; i < HALF; ++i) c0[i] = mfma_bf16(ah[i], bh, c0[i]);
#pragma unroll
      for (int i = 0; i < HALF; ++i) c1[i] = mfma_bf16(ah[i], bl, c1[i]);
#pragma unroll
      for (int i = 0; i < HALF; ++i) c2[i] = mfma_bf16(al[i], bh, c2[i]);
    }
#pragma unroll
    for (int i = 0; i < HALF; ++i) acc[i] = c0[i] + c1[i] + c2[i];
    lds_barrier();
  }
  float *out = p.S_out + ((int64_t)n * H + h) * DV * DK + (int64_t)row * DK + 4 * g4;
#pragma unroll
  for (int i = 0; i < HALF; ++i) *reinterpret_cast<f32x4 *>(out + 16 * (jb0 + i)) = acc[i];
}

template <int DK>
hipError_t launch_sc(const SegComposeLaunch &p, hipStream_t stream) {
  if (p.dv % 32 != 0) return hipErrorInvalidValue;
  const int64_t items = (int64_t)p.n_seqs * p.H * (p.dv / 32);
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
