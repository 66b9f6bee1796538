// gdn_prep_wave.h -- the per-chunk UT transform for bf16 inputs, done by one
// wave with no workgroup barriers; shared by the stand-alone prep kernel
// (gdn_prep_bf16.hip) and the prologue of the segment recurrence kernel
// (gdn_chain_bf16.hip).
//
// For a chunk of L <= 64 tokens (page "Tail-Replay: Escaping the Curse of
// Linear Attention in Prefix Caching for Hybrid LLMs", section 2 Eq. (1),
// unrolled over the chunk) the per-token delta-rule corrections D satisfy
//     (I + A) D = diag(beta) (V - diag(e^g) K S^T),
//     A = strictly lower part of  beta_r exp(g_r - g_s) (k_r . k_s),
// with g the cumulative log-gate.  A depends only on keys and gates, so
// Tau = (I + A)^{-1} is built once per (chunk, head) for every row tile of
// the recurrence.  Steps:
//   1. keys straight into registers as MFMA fragments (rows past the chunk
//      repeat its last row; they meet beta = 0 below); cumulative
//      log-gates by a wave-wide scan
//   2. the 10 lower 16 x 16 blocks of A on bf16 MFMA (keys are exact in
//      bf16), ten independent accumulators
//   3. the four diagonal blocks inverted at once by forward substitution:
//      lane (b, c) = (l >> 4, l & 15) computes column c of (I + A_bb)^{-1}
//   4. off-diagonal blocks Tau_ij = -Tau_ii sum_{m=j}^{i-1} A_im Tau_mj on
//      split-bf16 k = 16 MFMAs, in three dependency levels
//   5. Tau diag(beta) as split-bf16 A fragments of the recurrence kernel's
//      k = 32 products (record layout of gdn_internal.h).
// Raw inputs (RAW, gdn_internal.h kNormFloats): the gates come from the
// log-gates and logits, and the keys are normalised on the way: the
// diagonal blocks of K K^T hold |k_t|^2, so A takes the factor
// 1 / (|k_r| |k_s|), and the reciprocal key norms go to the chunk's norms
// block.
// LDS per wave: kPrepWaveLds bytes (A blocks, overwritten in place by the
// Tau blocks; gates; reciprocal norms).
#pragma once

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

constexpr int kPrepWaveLds = (10 * 256 + 3 * 64) * 4;

namespace prep_detail {

__device__ __forceinline__ constexpr int blk(int i, int j) { return i * (i + 1) / 2 + j; }  // i >= j

// A 4-value operand of a k = 16 MFMA as split bf16 (hi, lo).
struct Split4 {
  bf16x4 h, l;
};
__device__ __forceinline__ Split4 split_op(const f32x4 &x) {
  Split4 r;
  split4(x, r.h, r.l);
  return r;
}
// x (A layout) times y (B layout), k = 16, as split bf16 with the three
// partial products in separate accumulators (no product waits on the one
// before it).  Operands are split once and reused by every product they
// enter.
struct Acc3 {
  f32x4 a, b, c;
};
__device__ __forceinline__ void acc_split3(Acc3 &acc, const Split4 &x, const Split4 &y) {
  acc.a = mfma_bf16_k16(x.h, y.h, acc.a);
  acc.b = mfma_bf16_k16(x.h, y.l, acc.b);
  acc.c = mfma_bf16_k16(x.l, y.h, acc.c);
}
__device__ __forceinline__ Acc3 acc3_zero() { return Acc3{zero4(), zero4(), zero4()}; }
__device__ __forceinline__ f32x4 acc3_sum(const Acc3 &a) { return a.a + a.b + a.c; }

}  // namespace prep_detail

// The chunk's keys as MFMA fragments: kf[bt][m], lane (r, g) = (l & 15,
// l >> 4) holds key row 16 bt + r (rows past the chunk repeat its last row;
// they meet beta = 0 below), columns 32 m + 8 g .. + 7.  Plain loads, so a
// caller may issue them for its next chunk before working on this one.
template <int DK>
__device__ __forceinline__ void prep_load_keys(const bf16 *k, int H, int h, int t0, int Lc, bf16x8 (&kf)[4][DK / 32]) {
  const int l = lane_id(), g4 = l >> 4, jl = l & 15;
#pragma unroll
  for (int bt = 0; bt < 4; ++bt) {
    const int r = min(16 * bt + jl, Lc - 1);
    const bf16 *src = k + ((int64_t)(t0 + r) * H + h) * DK + 8 * g4;
#pragma unroll
    for (int m = 0; m < DK / 32; ++m) kf[bt][m] = *reinterpret_cast<const bf16x8 *>(src + 32 * m);
  }
}

// Offsets in the per-wave LDS scratch (floats): A / Tau blocks, cumulative
// log-gates, betas, reciprocal key norms.
constexpr int kPrepG = 10 * 256, kPrepB = kPrepG + 64, kPrepK = kPrepB + 64;

// The reciprocal norms of the diagonal blocks acc[blk(b, b)] of X X^T (C
// layout: lane (c, g) holds rows 4 g .. 4 g + 3 of column c, so the lanes
// with g = c >> 2 hold the diagonal) into dst[0 .. 63]; 0 for a zero row.
__device__ __forceinline__ void diag_rnorms(const f32x4 (&d)[4], float *dst) {
  const int l = lane_id(), g4 = l >> 4, jl = l & 15;
  if (g4 == (jl >> 2)) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const float n2 = d[b][jl & 3];
      dst[16 * b + jl] = n2 > 0.f ? rsqrtf(n2) : 0.f;
    }
  }
}

// Record of one (chunk, head) from its keys kf (prep_load_keys): tokens
// t0 .. t0 + Lc - 1 (1 <= Lc <= 64) of head h, gates alpha / beta [T, H]
// (bf16); rec receives kRecFloats * 4 bytes; scratch is this wave's
// kPrepWaveLds bytes of LDS; lds_rec (may be null) receives a second copy of
// the Tau fragments in LDS.  RAW: alpha and beta hold log-gates and logits,
// the keys are raw, and norms (kNormFloats floats) receives the reciprocal
// key norms.
template <int DK, bool RAW = false>
__device__ __forceinline__ void prep_chunk_wave_keys(const bf16x8 (&kf)[4][DK / 32], const bf16 *alpha,
                                                     const bf16 *beta, int H, int h, int t0, int Lc, char *rec,
                                                     float *scratch, char *lds_rec = nullptr,
                                                     float *norms = nullptr) {
  using namespace prep_detail;
  constexpr int NKS = DK / 32;
  float *sA = scratch;             // 10 blocks 16 x 16 row-major: A, then Tau
  float *sG = scratch + kPrepG, *sB = scratch + kPrepB, *sK = scratch + kPrepK;
  const int l = lane_id(), g4 = l >> 4, jl = l & 15;

  // ---- 1. gates (the keys are in kf) ----
  {
    float g = 0.f, b = 0.f;
    if (l < Lc) {
      const int64_t gi = (int64_t)(t0 + l) * H + h;
      if constexpr (RAW) {
        g = fmaxf((float)alpha[gi], kLogGateFloor);
        b = 1.f / (1.f + __expf(-(float)beta[gi]));
      } else {
        g = log_gate((float)alpha[gi]);
        b = (float)beta[gi];
      }
    }
    const float gs = wave_inclusive_scan(g);
    sG[l] = gs;
    sB[l] = b;
  }
  wave_lds_fence();

  // ---- 2. A = strictly-lower beta_r e^{g_r - g_s} K K^T, 10 blocks ----
  {
    f32x4 acc[10];
#pragma unroll
    for (int t = 0; t < 10; ++t) acc[t] = zero4();
#pragma unroll
    for (int m = 0; m < NKS; ++m)
#pragma unroll
      for (int bi = 0; bi < 4; ++bi)
#pragma unroll
        for (int bj = 0; bj <= bi; ++bj) acc[blk(bi, bj)] = mfma_bf16(kf[bi][m], kf[bj][m], acc[blk(bi, bj)]);
    if constexpr (RAW) {
      const f32x4 dg[4] = {acc[blk(0, 0)], acc[blk(1, 1)], acc[blk(2, 2)], acc[blk(3, 3)]};
      diag_rnorms(dg, sK);
      wave_lds_fence();
    }
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
      for (int bj = 0; bj <= bi; ++bj) {
        const int col = 16 * bj + jl, row0 = 16 * bi + 4 * g4;
        const float gc = sG[col];
        const f32x4 gr = *reinterpret_cast<const f32x4 *>(sG + row0);
        f32x4 br = *reinterpret_cast<const f32x4 *>(sB + row0);
        if constexpr (RAW) {   // beta_r / (|k_r| |k_s|)
          const float kc = sK[col];
          const f32x4 kr = *reinterpret_cast<const f32x4 *>(sK + row0);
#pragma unroll
          for (int e = 0; e < 4; ++e) br[e] *= kr[e] * kc;
        }
        float *dst = sA + blk(bi, bj) * 256 + 4 * g4 * 16 + jl;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          dst[e * 16] = (col < row0 + e) ? br[e] * __expf(gr[e] - gc) * acc[blk(bi, bj)][e] : 0.f;
      }
  }
  wave_lds_fence();

  // ---- 3. diagonal blocks: lane (b, c) solves (I + A_bb) x = e_c; the
  // result replaces A_bb (all reads of the block precede the writes) ----
  {
    const int b = g4, c = jl;
    float *ab = sA + blk(b, b) * 256;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float acc0 = (r == c) ? 1.f : 0.f, acc1 = 0.f;
#pragma unroll
      for (int s4 = 0; s4 < (r + 3) / 4; ++s4) {
        const f32x4 ar = *reinterpret_cast<const f32x4 *>(ab + r * 16 + 4 * s4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int s = 4 * s4 + e;
          if (s < r) {
            if (e & 1)
              acc1 -= ar[e] * x[s];
            else
              acc0 -= ar[e] * x[s];
          }
        }
      }
      x[r] = acc0 + acc1;
    }
    wave_lds_fence();
#pragma unroll
    for (int r = 0; r < 16; ++r) ab[r * 16 + c] = x[r];      // row-major: Tau_bb[r][c]
  }
  wave_lds_fence();

  // ---- 4. off-diagonal blocks (C layout: lane column jl, rows 4 g4 + e) ----
  {
    // operands: A_im and Tau_ii in A layout (row jl, columns 4 g4 ..), Tau_jj
    // in B layout (column jl, rows 4 g4 ..: four reads down a column)
    auto Aop = [&](int i, int m) {
      return split_op(*reinterpret_cast<const f32x4 *>(sA + blk(i, m) * 256 + jl * 16 + 4 * g4));
    };
    auto Tjj = [&](int i) {
      const float *t = sA + blk(i, i) * 256 + 4 * g4 * 16 + jl;
      return split_op(f32x4{t[0], t[16], t[32], t[48]});
    };
    auto neg_tau = [&](const Split4 &tii, const Acc3 &x) {       // -Tau_ii X
      Acc3 y = acc3_zero();
      acc_split3(y, tii, split_op(acc3_sum(x)));
      return -acc3_sum(y);
    };
    // every operand split once: Tau_jj (B layout), Tau_ii (A layout), A_im
    const Split4 T00 = Tjj(0), T11 = Tjj(1), T22 = Tjj(2);
    const Split4 D11 = Aop(1, 1), D22 = Aop(2, 2), D33 = Aop(3, 3);
    const Split4 A10 = Aop(1, 0), A21 = Aop(2, 1), A32 = Aop(3, 2), A20 = Aop(2, 0), A31 = Aop(3, 1), A30 = Aop(3, 0);
    // level 1: Tau_10, Tau_21, Tau_32
    Acc3 x10 = acc3_zero(), x21 = acc3_zero(), x32 = acc3_zero();
    acc_split3(x10, A10, T00);
    acc_split3(x21, A21, T11);
    acc_split3(x32, A32, T22);
    const f32x4 T10 = neg_tau(D11, x10), T21 = neg_tau(D22, x21), T32 = neg_tau(D33, x32);
    const Split4 T10s = split_op(T10), T21s = split_op(T21);
    // level 2: Tau_20, Tau_31
    Acc3 x20 = acc3_zero(), x31 = acc3_zero();
    acc_split3(x20, A20, T00);
    acc_split3(x31, A31, T11);
    acc_split3(x20, A21, T10s);
    acc_split3(x31, A32, T21s);
    const f32x4 T20 = neg_tau(D22, x20), T31 = neg_tau(D33, x31);
    // level 3: Tau_30
    Acc3 x30 = acc3_zero();
    acc_split3(x30, A30, T00);
    acc_split3(x30, A31, T10s);
    acc_split3(x30, A32, split_op(T20));
    const f32x4 T30 = neg_tau(D33, x30);
    // every A block has been read: the off-diagonal Tau blocks take their place
    wave_lds_fence();
    auto put = [&](int i, int jb, const f32x4 &t) {
      float *dst = sA + blk(i, jb) * 256 + 4 * g4 * 16 + jl;
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[e * 16] = t[e];
    };
    put(1, 0, T10);
    put(2, 1, T21);
    put(3, 2, T32);
    put(2, 0, T20);
    put(3, 1, T31);
    put(3, 0, T30);
  }
  wave_lds_fence();

  // ---- 5. Tau diag(beta) as split-bf16 A fragments: fragment f = (bt, m),
  // lane (r, g) = (l & 15, l >> 4) holds row 16 bt + r, columns
  // 32 m + 4 g + {0..3} then 32 m + 16 + 4 g + {0..3} (column scale: beta,
  // or none) ----
  auto write_frags = [&](char *dst, char *lds_dst, bool scale_beta) {
    bf16 *outh = reinterpret_cast<bf16 *>(dst), *outl = outh + kTauFragPlane;
#pragma unroll
    for (int f = 0; f < kTauFrags; ++f) {
      const int bt = f < 2 ? f : (f - 2) / 2 + 2;
      const int m = f < 2 ? 0 : (f - 2) % 2;
      float x[8];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int cb = 2 * m + half, c0 = 16 * cb + 4 * g4;
        f32x4 v = zero4();
        if (cb <= bt) v = *reinterpret_cast<const f32x4 *>(sA + blk(bt, cb) * 256 + jl * 16 + 4 * g4);
        if (scale_beta) {
          const f32x4 bc = *reinterpret_cast<const f32x4 *>(sB + c0);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] *= bc[e];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) x[4 * half + e] = v[e];
      }
      bf16x8 hi, lo;
      split8(x, hi, lo);
      *reinterpret_cast<bf16x8 *>(outh + 8 * (f * 64 + l)) = hi;
      *reinterpret_cast<bf16x8 *>(outl + 8 * (f * 64 + l)) = lo;
      if (lds_dst) {
        bf16 *lh = reinterpret_cast<bf16 *>(lds_dst), *ll = lh + kTauFragPlane;
        *reinterpret_cast<bf16x8 *>(lh + 8 * (f * 64 + l)) = hi;
        *reinterpret_cast<bf16x8 *>(ll + 8 * (f * 64 + l)) = lo;
      }
    }
  };
  write_frags(rec, lds_rec, true);

  if constexpr (RAW) {
    wave_lds_fence();
    norms[l] = sK[l];
  }
}

// Record of one (chunk, head), keys loaded here (see prep_chunk_wave_keys).
template <int DK, bool RAW = false>
__device__ __forceinline__ void prep_chunk_wave(const bf16 *k, const bf16 *alpha, const bf16 *beta, int H, int h,
                                                int t0, int Lc, char *rec, float *scratch, char *lds_rec = nullptr,
                                                float *norms = nullptr) {
  bf16x8 kf[4][DK / 32];
  prep_load_keys<DK>(k, H, h, t0, Lc, kf);
  prep_chunk_wave_keys<DK, RAW>(kf, alpha, beta, H, h, t0, Lc, rec, scratch, lds_rec, norms);
}

}  // namespace gdn
