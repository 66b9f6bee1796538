// gdn_front.hip -- the step before the recurrence: queries and keys
// L2-normalised per (token, head), the decay alpha from its log-gate and the
// write strength beta from its logit.
//
// Page "Tail-Replay: Escaping the Curse of Linear Attention in Prefix Caching
// for Hybrid LLMs": section 3 (during the replay the hidden states of the
// group produce the keys, values, transitions and write strengths that the
// recurrence consumes) and section 2 Eq. (1) (alpha in (0, 1] scales the
// state).  Per (token, head):
//     q <- q / |q|,  k <- k / |k|   (a zero row stays zero)
//     alpha = exp(g),  beta = 1 / (1 + exp(-b))
// computed in fp32 and rounded once to the input dtype, so every later
// kernel (records, recurrence, output pass, decode) reads the same values.
//
// One pass over the tensors, bound by HBM bandwidth: 16 lanes share a row
// (dk / 16 contiguous values each), a lane loads its values of FU rows before
// it reduces any, the squared norm is summed across the 16 lanes by DPP and
// its reciprocal square root scales the row, and each lane writes back only
// the values it read, so the outputs may alias the inputs.  The gates are
// one element per lane in a grid-stride loop of their own.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int FNT = 256;   // threads per workgroup
constexpr int FU = 2;      // rows a 16-lane group loads before reducing (1, 2 and 4 measured
                           // with unconditional loads: 22.6, 20.7 and 21.7 us on 3277 x 32 rows
                           // of q and k, against 22.2-23.8 us for one row loaded under a branch)

template <typename TI>
__device__ __forceinline__ TI from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// PER values at p (PER * sizeof(TI) bytes, 16-byte aligned for PER * sizeof(TI) >= 16)
template <int PER, typename TI>
__device__ __forceinline__ void load_row(const TI *p, float (&x)[PER]) {
  if constexpr (sizeof(TI) == 2 && PER == 8) {
    const bf16x8 v = *reinterpret_cast<const bf16x8 *>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (float)v[i];
  } else if constexpr (sizeof(TI) == 2 && PER == 4) {
    const bf16x4 v = *reinterpret_cast<const bf16x4 *>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = (float)v[i];
  } else {
#pragma unroll
    for (int i = 0; i < PER; i += 4) {
      const f32x4 v = *reinterpret_cast<const f32x4 *>(p + i);
      x[i] = v[0];
      x[i + 1] = v[1];
      x[i + 2] = v[2];
      x[i + 3] = v[3];
    }
  }
}

template <int PER, typename TI>
__device__ __forceinline__ void store_row(TI *p, const float (&x)[PER]) {
  if constexpr (sizeof(TI) == 2 && PER == 8) {
    bf16x8 v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (bf16)x[i];
    *reinterpret_cast<bf16x8 *>(p) = v;
  } else if constexpr (sizeof(TI) == 2 && PER == 4) {
    bf16x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (bf16)x[i];
    *reinterpret_cast<bf16x4 *>(p) = v;
  } else {
#pragma unroll
    for (int i = 0; i < PER; i += 4)
      *reinterpret_cast<f32x4 *>(p + i) = f32x4{x[i], x[i + 1], x[i + 2], x[i + 3]};
  }
}

template <int DK, typename TI>
__global__ void __launch_bounds__(FNT) front_kernel(FrontLaunch p) {
  constexpr int PER = DK / 16;
  const int64_t rows = p.n_tokens * p.H;                 // rows per tensor
  const int64_t n_rows = p.q_in ? 2 * rows : rows;       // q rows first, then k rows
  const int64_t groups = (int64_t)gridDim.x * (FNT / 16);
  const int64_t g0 = (int64_t)blockIdx.x * (FNT / 16) + (threadIdx.x >> 4);
  const int c = threadIdx.x & 15;
  for (int64_t r0 = g0; r0 < n_rows; r0 += FU * groups) {
    float x[FU][PER];
    bool live[FU];
    // every row slot is loaded (a slot past the end reloads the last row and
    // is not stored): loads under a branch would each be waited for at once
#pragma unroll
    for (int u = 0; u < FU; ++u) {
      const int64_t r = min(r0 + u * groups, n_rows - 1);
      live[u] = r0 + u * groups < n_rows;
      const bool is_q = p.q_in && r < rows;
      const TI *src = reinterpret_cast<const TI *>(is_q ? p.q_in : p.k_in);
      load_row<PER>(src + (is_q ? r : r - (p.q_in ? rows : 0)) * DK + PER * c, x[u]);
    }
#pragma unroll
    for (int u = 0; u < FU; ++u) {
      // live[u] is the same for the 16 lanes of a row, so the row sum below
      // only combines lanes of rows that are all live
      if (live[u]) {
        const int64_t r = r0 + u * groups;
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < PER; ++i) s += x[u][i] * x[u][i];
        s = row16_sum(s);
        const float inv = s > 0.f ? rsqrtf(s) : 0.f;   // (a zero row stays zero)
#pragma unroll
        for (int i = 0; i < PER; ++i) x[u][i] *= inv;
        const bool is_q = p.q_in && r < rows;
        TI *dst = reinterpret_cast<TI *>(is_q ? p.q_out : p.k_out);
        store_row<PER>(dst + (is_q ? r : r - (p.q_in ? rows : 0)) * DK + PER * c, x[u]);
      }
    }
  }
  const int64_t threads = (int64_t)gridDim.x * FNT;
  const TI *g = reinterpret_cast<const TI *>(p.g), *b = reinterpret_cast<const TI *>(p.b);
  TI *alpha = reinterpret_cast<TI *>(p.alpha), *beta = reinterpret_cast<TI *>(p.beta);
  for (int64_t e = (int64_t)blockIdx.x * FNT + threadIdx.x; e < rows; e += threads) {
    const TI ge = g[e], be = b[e];   // both loads in flight before either is used
    alpha[e] = from_f32<TI>(expf(to_f32(ge)));
    beta[e] = from_f32<TI>(1.f / (1.f + expf(-to_f32(be))));
  }
}

template <int DK>
hipError_t launch_f(const FrontLaunch &p, hipStream_t stream) {
  const int64_t rows = p.n_tokens * p.H;
  if (rows <= 0) return hipSuccess;
  const int64_t n_rows = p.q_in ? 2 * rows : rows;
  // one round of FU rows per 16-lane group where that fits; at most 65536
  // workgroups, the rest by the grid-stride loops
  const int64_t want = (n_rows + FU * (FNT / 16) - 1) / (FU * (FNT / 16));
  const unsigned grid = (unsigned)(want < 65536 ? want : 65536);
  if (p.in_bf16)
    return launch_kernel(front_kernel<DK, bf16>, dim3(grid), dim3(FNT), 0, stream, p);
  return launch_kernel(front_kernel<DK, float>, dim3(grid), dim3(FNT), 0, stream, p);
}

}  // namespace

hipError_t launch_front(const FrontLaunch &p, hipStream_t stream) {
  if (p.dk == 64) return launch_f<64>(p, stream);
  if (p.dk == 128) return launch_f<128>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace gdn
