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
  hipLaunchKernelGGL((op_frag_kernel<DK>), dim3((unsigned)(n_ops * (DK / 32))), dim3(FNW * 64), 0, stream, T,
                     static_cast<char *>(frag));
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Composition of one sequence's operators in order: S = S_seg[0] (time
// split: segment 0 already started from S0), or S = S0 with every operator
// applied (from_start: gdn_compose), then S <- S T_seg[s] + S_seg[s],
// computed as S_new^T = T^T S^T + S_seg^T.  The operators arrive as split-bf16 MFMA
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
  const int s0 = p.from_start ? 0 : 1;   // first operator applied
  if (p.from_start) {   // (S0 may alias S_out: every workgroup reads its own rows here, first)
    const float *s0p = p.S0 ? p.S0 + ((int64_t)n * H + h) * DV * DK + (int64_t)row * DK + 4 * g4 : nullptr;
#pragma unroll
    for (int i = 0; i < HALF; ++i) acc[i] = s0p ? *reinterpret_cast<const f32x4 *>(s0p + 16 * (jb0 + i)) : zero4();
  } else {
    load_loc(0, acc);
  }
  if (s0 < P) {
    issue_op(s0, 0);
    load_loc(s0, loc);
  }
  for (int s = s0; s < P; ++s) {
    const int b = (s - s0) & 1;
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

hipError_t launch_op_frags(const float *T, int64_t n_ops, int32_t dk, void *frag, hipStream_t stream) {
  if (dk == 64) return launch_of<64>(T, n_ops, frag, stream);
  if (dk == 128) return launch_of<128>(T, n_ops, frag, stream);
  return hipErrorInvalidValue;
}

}  // namespace gdn
