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

}  // namespace

hipError_t launch_compose(const ComposeLaunch &p, hipStream_t stream) {
  if (p.dk == 64) return launch_c<64>(p, stream);
  if (p.dk == 128) return launch_c<128>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace gdn
