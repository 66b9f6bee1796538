// gdn_scalar.hip -- the chunk operator and its composition when the per-token
// transition is a scalar decay (the Mamba-2 family) instead of Gated
// DeltaNet's dense rank-1 update.
//
// Page "LinearKV: One Cached State Suffices for Position-Independent Caching
// in Hybrid LLMs", the affine-operator paragraph: a chunk maps S_in to
// S_in T_C + S_local, and with a scalar per-token transition T_t = a_t I the
// chunk's T_C is the scalar gamma = prod_t a_t.  With the write term of the
// gated delta rule (Tail-Replay, section 2 Eq. (1)) and T_t = a_t I:
//     S_t = a_t S_{t-1} + beta_t v_t k_t^T
// so, from an empty start over the chunk,
//     S_local = sum_t u_t v_t k_t^T,   u_t = beta_t prod_{s > t} a_s,
// a contraction over the chunk's tokens: S_local = V^T diag(u) K.
//
// scalar_op_kernel: one workgroup (dv / 16 waves) per (chunk, head).  The chunk is
// taken 32 tokens at a time from its end backwards: keys and values staged in
// LDS as token rows, and the weights u_t = beta_t W exp(-(P_t - P_end)) from a
// wave scan of log a within the step (P the step's inclusive prefix) times the
// product W of the alphas of the later steps, so every decay is a product of
// factors near 1 or the exponential of a short sum, never the difference of two
// long sums.  gamma is a product of the alphas (per-lane partial products and
// a tree of multiplications), all in fp32.  The loads of the next step are
// issued before the current step's products (two register buffers, with
// at least four waves per SIMD asked of the register allocator so that two
// workgroups share a compute unit: without that bound the two buffers took
// 164 registers and 0.31 ms on 64 x 512 tokens x 32 heads, with it 0.20 ms,
// the same as one buffer and four waves).  Wave w owns dv rows
// [16 w, 16 w + 16) of S_local and all dk columns; per 32
// tokens it forms A(m, t) = v_t[m] u_t (fp32, split into hi + lo bf16) and
// takes B(n, t) = k_t[n] (exact for bf16 inputs, split for fp32), and
// accumulates on v_mfma_f32_16x16x32_bf16 in fp32.  For bf16 inputs both
// operands come from the token rows in LDS through the gfx950 transposing
// read, two 8-byte reads per fragment (single-element column reads took
// 0.21 ms on 64 x 512 tokens x 32 heads, the transposing reads 0.17 ms).
//
// scalar_compose_kernel: S <- gamma[c] S + S_local[c] for c in order, one
// lane per 4 consecutive state elements of a head, streaming S_local once.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int SNT = 256;   // threads per workgroup (4 waves)
constexpr int SB = 32;     // tokens per step (one MFMA k block)

// MINW: waves per SIMD asked of the register allocator (4 for bf16 at
// dk = dv = 128, where it lets two workgroups share a compute unit; 1, no
// bound, elsewhere, where a bound of 4 would spill registers)
template <int DK, int DV, typename TI, int MINW>
__global__ void __launch_bounds__(4 * DV) __attribute__((amdgpu_waves_per_eu(MINW))) scalar_op_kernel(ScalarOpLaunch p) {
  constexpr bool EXACT_K = sizeof(TI) == 2;   // bf16 keys are exact MFMA operands
  constexpr int LDK = DK + 8, LDV = DV + 8;   // row padding (elements)
  constexpr int NT = 4 * DV;                  // threads: one wave per 16 rows of S_local
  constexpr int NB = DK / 16;                 // 16-column blocks
  __shared__ __align__(16) TI sK[SB * LDK];
  __shared__ __align__(16) TI sV[SB * LDV];
  __shared__ __align__(16) float sU[SB];
  const int c = blockIdx.x / p.H, h = blockIdx.x % p.H;
  const int t0 = p.cu[c], L = p.cu[c + 1] - t0;
  const int w = wave_id(), l = lane_id();
  const TI *alpha = reinterpret_cast<const TI *>(p.alpha), *beta = reinterpret_cast<const TI *>(p.beta);

  // gamma = the product of the chunk's alphas (wave 0)
  if (w == 0) {
    float g = 1.f;
    for (int j = l; j < L; j += 64) g *= to_f32(alpha[(int64_t)(t0 + j) * p.H + h]);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) g *= __shfl_xor(g, m, 64);
    if (l == 0) p.gamma[(int64_t)c * p.H + h] = g;
  }
  if (!p.S_local) return;

  f32x4 acc[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) acc[j] = zero4();

  const TI *k = reinterpret_cast<const TI *>(p.k), *v = reinterpret_cast<const TI *>(p.v);
  // 16-byte pieces of one step's 32 token rows of k then v; each thread moves NPT of them
  constexpr int EPP = 16 / (int)sizeof(TI);   // elements per piece
  constexpr int PK = DK / EPP, PV = DV / EPP;
  constexpr int NPT = (SB * (PK + PV) + NT - 1) / NT;
  // two register buffers: the loads of the next two steps are in flight
  // while a step's products run
  uint4 preA[NPT], preB[NPT];
  float paA = 1.f, pbA = 0.f, paB = 1.f, pbB = 0.f;   // wave 0, lane < 32: alpha, beta
  auto fetch = [&](uint4 (&pre)[NPT], float &pa, float &pb, int s0) {  // zeros past the chunk's end
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
      const int e = threadIdx.x + j * NT;
      const bool isk = e < SB * PK;
      const int ee = isk ? e : e - SB * PK, P = isk ? PK : PV;
      const int r = ee / P, q = ee % P;
      pre[j] = make_uint4(0, 0, 0, 0);
      if (s0 >= 0 && e < SB * (PK + PV) && s0 + r < L)
        pre[j] = *reinterpret_cast<const uint4 *>((isk ? k : v) + ((int64_t)(t0 + s0 + r) * p.H + h) * (isk ? DK : DV) +
                                                  q * EPP);
    }
    pa = 1.f;
    pb = 0.f;
    if (s0 >= 0 && w == 0 && l < SB && s0 + l < L) {
      const int64_t gi = (int64_t)(t0 + s0 + l) * p.H + h;
      pa = to_f32(alpha[gi]);
      pb = to_f32(beta[gi]);
    }
  };
  float later = 1.f;   // product of the alphas of the steps after this one (wave 0)
  const int r = l & 15, kq = (l >> 4) * 8;
  // one step: registers -> LDS (token rows) and the step's weights, then the
  // loads two steps ahead into the same buffer, then the products
  auto step = [&](uint4 (&pre)[NPT], float &pa, float &pb, int s0) {
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
      const int e = threadIdx.x + j * NT;
      const bool isk = e < SB * PK;
      const int ee = isk ? e : e - SB * PK, P = isk ? PK : PV;
      const int rr = ee / P, q = ee % P;
      if (e < SB * (PK + PV)) *reinterpret_cast<uint4 *>((isk ? sK + rr * LDK : sV + rr * LDV) + q * EPP) = pre[j];
    }
    if (w == 0) {
      const float P = wave_inclusive_scan(log_gate(pa));
      const float tot = lane_value(P, 63);
      if (l < SB) sU[l] = pb * later * expf(tot - P);
      later *= expf(tot);
    }
    __syncthreads();
    fetch(pre, pa, pb, s0 - 2 * SB);
    bf16x8 bh[NB], bl[NB];
    float a[8];
    if constexpr (EXACT_K) {
      // transposing reads: lane (g, i) gets column i of a 16-column block at
      // tokens 4g + e and 16 + 4g + e (e < 4), the same permuted token order
      // for both operands
      const int g4 = l >> 4, q = l & 15;
      const int src = (4 * g4 + (q >> 2)) * LDK + 4 * (q & 3);
      const int srv = (4 * g4 + (q >> 2)) * LDV + 4 * (q & 3);
#pragma unroll
      for (int j = 0; j < NB; ++j)
        bh[j] = cat_bf16x8(ds_read_tr16(sK + src + 16 * j), ds_read_tr16(sK + src + 16 * LDK + 16 * j));
      const bf16x8 vv = cat_bf16x8(ds_read_tr16(sV + srv + 16 * w), ds_read_tr16(sV + srv + 16 * LDV + 16 * w));
      const f32x4 u0 = *reinterpret_cast<const f32x4 *>(sU + 4 * g4);
      const f32x4 u1 = *reinterpret_cast<const f32x4 *>(sU + 16 + 4 * g4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a[e] = (float)vv[e] * u0[e];
        a[4 + e] = (float)vv[4 + e] * u1[e];
      }
    } else {
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int n = 16 * j + r;
        float b[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) b[e] = to_f32(sK[(kq + e) * LDK + n]);
        split8(b, bh[j], bl[j]);
      }
      const int m = 16 * w + r;
#pragma unroll
      for (int e = 0; e < 8; ++e) a[e] = to_f32(sV[(kq + e) * LDV + m]) * sU[kq + e];
    }
    bf16x8 ah, al;
    split8(a, ah, al);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      acc[j] = mfma_bf16(ah, bh[j], acc[j]);
      acc[j] = mfma_bf16(al, bh[j], acc[j]);
      if constexpr (!EXACT_K) acc[j] = mfma_bf16(ah, bl[j], acc[j]);
    }
    __syncthreads();
  };
  const int first = L > 0 ? (L - 1) / SB * SB : -SB;   // steps run from the chunk's end backwards
  fetch(preA, paA, pbA, first);
  fetch(preB, paB, pbB, first - SB);
  for (int s0 = first; s0 >= 0; s0 -= 2 * SB) {
    step(preA, paA, pbA, s0);
    if (s0 < SB) break;
    step(preB, paB, pbB, s0 - SB);
  }
  // S_local[c, h] row-major [DV][DK]: lane holds rows 4 (l >> 4) + i, column l & 15
  float *out = p.S_local + ((int64_t)c * p.H + h) * DV * DK;
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) out[(16 * w + 4 * (l >> 4) + e) * DK + 16 * j + (l & 15)] = acc[j][e];
}

__global__ void __launch_bounds__(SNT) scalar_compose_kernel(ScalarComposeLaunch p) {
  const int64_t per_head = (int64_t)p.dv * p.dk / 4;   // f32x4 per head
  const int64_t n4 = per_head * p.H;
  const int64_t i = (int64_t)blockIdx.x * SNT + threadIdx.x;
  if (i >= n4) return;
  const int h = (int)(i / per_head);
  f32x4 s = p.S_in ? reinterpret_cast<const f32x4 *>(p.S_in)[i] : zero4();
  const f32x4 *Ls = reinterpret_cast<const f32x4 *>(p.S_local);
#pragma unroll 4
  for (int c = 0; c < p.n_chunks; ++c) {
    const float g = p.gamma[(int64_t)c * p.H + h];
    const f32x4 x = Ls[(int64_t)c * n4 + i];
    s = f32x4{g * s[0] + x[0], g * s[1] + x[1], g * s[2] + x[2], g * s[3] + x[3]};
  }
  reinterpret_cast<f32x4 *>(p.S_out)[i] = s;
}

template <int DK, int DV>
hipError_t launch_op(const ScalarOpLaunch &p, hipStream_t stream) {
  const int64_t items = (int64_t)p.n_chunks * p.H;
  if (items <= 0) return hipSuccess;
  if (p.in_bf16)
    return launch_kernel(scalar_op_kernel<DK, DV, bf16, (DK == 128 && DV == 128) ? 4 : 1>, dim3((unsigned)items),
                         dim3(4 * DV), 0, stream, p);
  return launch_kernel(scalar_op_kernel<DK, DV, float, 1>, dim3((unsigned)items), dim3(4 * DV), 0, stream, p);
}

}  // namespace

hipError_t launch_scalar_op(const ScalarOpLaunch &p, hipStream_t stream) {
  if (p.dk == 64 && p.dv == 64) return launch_op<64, 64>(p, stream);
  if (p.dk == 64 && p.dv == 128) return launch_op<64, 128>(p, stream);
  if (p.dk == 128 && p.dv == 64) return launch_op<128, 64>(p, stream);
  if (p.dk == 128 && p.dv == 128) return launch_op<128, 128>(p, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_scalar_compose(const ScalarComposeLaunch &p, hipStream_t stream) {
  const int64_t n4 = (int64_t)p.H * p.dv * p.dk / 4;
  if (n4 <= 0) return hipSuccess;
  return launch_kernel(scalar_compose_kernel, dim3((unsigned)((n4 + SNT - 1) / SNT)), dim3(SNT), 0, stream, p);
}

}  // namespace gdn
