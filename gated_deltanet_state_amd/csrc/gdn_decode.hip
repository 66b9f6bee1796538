// gdn_decode.hip -- one token per sequence from a given state: the step that
// follows a replay when serving continues token by token.
//
// Page "Tail-Replay: Escaping the Curse of Linear Attention in Prefix Caching
// for Hybrid LLMs": section 2 Eq. (1) (the per-token update) and section 3
// (after the replay the model continues serving the request from the
// reconstructed states).  For one token with state S (dv x dk):
//     y = S k,   S <- alpha S + beta (v - alpha y) k^T,   o = S q
// (Eq. (1) multiplied out; o with the updated state).
//
// Rows of S are independent, so the step is one streaming pass over the
// state: 64 KiB read and 64 KiB written per (sequence, head) at dk = dv =
// 128, bound by HBM bandwidth.  A workgroup of four waves takes one
// (sequence, head); 16 lanes share a row (dk / 16 values each, 16- or
// 32-byte contiguous pieces, so a wave reads four whole rows per step), a
// wave loads all of its rows before it updates any (its reads are then in
// flight together), the two dot products are reduced across the 16 lanes
// by DPP, and each updated row is written back in place (S_out
// may alias S_in).  All arithmetic is fp32.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int DNW = 4;

template <typename T>
__device__ __forceinline__ float to_f32(T x);
template <>
__device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ float to_f32<bf16>(bf16 x) { return (float)x; }

template <int DK, int DV, typename TI>
__global__ void __launch_bounds__(DNW * 64) decode_kernel(DecodeLaunch p) {
  constexpr int PER = DK / 16;   // values of a row per lane
  const int nh = blockIdx.x;
  const int w = wave_id(), l = lane_id(), r4 = l >> 4, c = l & 15;
  const TI *q = reinterpret_cast<const TI *>(p.q), *k = reinterpret_cast<const TI *>(p.k);
  const TI *v = reinterpret_cast<const TI *>(p.v);
  const float alpha = to_f32(reinterpret_cast<const TI *>(p.alpha)[nh]);
  const float beta = to_f32(reinterpret_cast<const TI *>(p.beta)[nh]);
  // Every load is issued unconditionally (a missing q or S_in is read from
  // k or S_out and the values replaced by zeros): the compiler counts the
  // wait for each loaded register from the order of the loads, and a load
  // under a branch would make it wait for all loads outstanding right there.
  const TI *qs = p.o ? q : k;
  const float *Ss = p.S_in ? p.S_in : p.S_out;
  float kk[PER], qq[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    kk[i] = to_f32(k[(int64_t)nh * DK + PER * c + i]);
    qq[i] = to_f32(qs[(int64_t)nh * DK + PER * c + i]);
  }
  const int64_t base = (int64_t)nh * DV * DK;
  // rows w * DV / 4 + 4 it + r4.  Every row of the wave is loaded first, so
  // all of its reads are in flight together (S_out may alias S_in, which
  // would otherwise keep a read behind the previous row's write).
  constexpr int IT = DV / (4 * DNW);   // rows per lane
  float s[IT][PER];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int64_t off = base + (int64_t)(w * (DV / DNW) + 4 * it + r4) * DK + PER * c;
#pragma unroll
    for (int i = 0; i < PER; i += 4) {
      const f32x4 x = *reinterpret_cast<const f32x4 *>(Ss + off + i);
      s[it][i] = x[0];
      s[it][i + 1] = x[1];
      s[it][i + 2] = x[2];
      s[it][i + 3] = x[3];
    }
  }
  float vr[IT];   // v of each row
#pragma unroll
  for (int it = 0; it < IT; ++it) vr[it] = to_f32(v[(int64_t)nh * DV + w * (DV / DNW) + 4 * it + r4]);
  const bool has_s = p.S_in != nullptr;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    {
      const int row = w * (DV / DNW) + 4 * it + r4;
      const int64_t off = base + (int64_t)row * DK + PER * c;
      if (!has_s) {
#pragma unroll
        for (int i = 0; i < PER; ++i) s[it][i] = 0.f;
      }
      float y = 0.f;
#pragma unroll
      for (int i = 0; i < PER; ++i) y += s[it][i] * kk[i];
      y = row16_sum(y);
      const float coef = beta * (vr[it] - alpha * y);
      float o = 0.f;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        s[it][i] = alpha * s[it][i] + coef * kk[i];
        o += s[it][i] * qq[i];
      }
#pragma unroll
      for (int i = 0; i < PER; i += 4)
        *reinterpret_cast<f32x4 *>(p.S_out + off + i) = f32x4{s[it][i], s[it][i + 1], s[it][i + 2], s[it][i + 3]};
      if (p.o) {
        o = row16_sum(o);
        if (c == 0) {
          if (p.o_bf16)
            reinterpret_cast<bf16 *>(p.o)[(int64_t)nh * DV + row] = (bf16)o;
          else
            reinterpret_cast<float *>(p.o)[(int64_t)nh * DV + row] = o;
        }
      }
    }
  }
}

template <int DK, int DV>
hipError_t launch_d(const DecodeLaunch &p, hipStream_t stream) {
  const int64_t items = (int64_t)p.n_seqs * p.H;
  if (items <= 0) return hipSuccess;
  if (p.in_bf16)
    return launch_kernel(decode_kernel<DK, DV, bf16>, dim3((unsigned)items), dim3(DNW * 64), 0, stream, p);
  return launch_kernel(decode_kernel<DK, DV, float>, dim3((unsigned)items), dim3(DNW * 64), 0, stream, p);
}

}  // namespace

hipError_t launch_decode(const DecodeLaunch &p, hipStream_t stream) {
  if (p.dk == 64 && p.dv == 64) return launch_d<64, 64>(p, stream);
  if (p.dk == 64 && p.dv == 128) return launch_d<64, 128>(p, stream);
  if (p.dk == 128 && p.dv == 64) return launch_d<128, 64>(p, stream);
  if (p.dk == 128 && p.dv == 128) return launch_d<128, 128>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace gdn
