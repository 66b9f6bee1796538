// gdn_device.h -- device-side building blocks for the gfx950 GDN kernels:
// MFMA fragment loaders over LDS-resident operands, split-bfloat16 products
// and small lane utilities.
//
// MFMA lane layouts used (gfx950, wave64; checked on the device):
//   v_mfma_f32_16x16x32_bf16:  A[16 x 32]: lane l holds row (l & 15),
//     k = 8*(l >> 4) .. +7;  B[32 x 16]: lane l holds column (l & 15), the
//     same 8 k;  C/D[16 x 16]: lane l holds column (l & 15), rows
//     4*(l >> 4) .. +3.
//   v_mfma_f32_16x16x16_bf16:  A: row (l & 15), k = 4*(l >> 4) .. +3;
//     B: column (l & 15), the same 4 k;  C/D as above.  The C/D layout of a
//     16 x 16 tile is therefore exactly its B-operand layout, which lets a
//     product result feed the next product without leaving registers.
//   v_mfma_f32_16x16x4_f32:    A: row (l & 15), k = l >> 4;  B: column
//     (l & 15), k = l >> 4;  C/D as above.
//
// Split bfloat16 (Henry, Tang and Heinecke, "Leveraging the bfloat16
// Artificial Intelligence Datatype For Higher-Precision Computations",
// ARITH 2019): an fp32 value x is carried as hi = bf16(x) and
// lo = bf16(x - hi); a product a*b is approximated by up to three bf16
// products a_hi b_hi + a_hi b_lo + a_lo b_hi accumulated in fp32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_bf16_k16(const bf16x4 &a, const bf16x4 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

__device__ __forceinline__ float ld_in(const float *p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ld_in(const bf16 *p, int64_t i) { return (float)p[i]; }

// Float offset of lower block row bi in a packed 64 x 64 Tau (block row bi
// holds 16 rows x 16 (bi + 1) columns): 256 * bi (bi + 1) / 2.
__device__ __forceinline__ int tau_off(int bi) { return 128 * bi * (bi + 1); }

// ---------------------------------------------------------------------------
// LDS operand views.  An operand of an MFMA tile is addressed as
// element(row, k): "row" runs over the 16 M (or N) positions of the tile and
// k over the contraction.
//   RowMajor<T>:  p[row * ld + k]           (k contiguous: 8-wide loads)
//   ColMajor<T>:  p[k * ld + row]           (only single-element loads)
//   RowScaled:    fp32 p[row * ld + k] * s[k]  (column scaling on load)
// ---------------------------------------------------------------------------
template <class T>
struct RowMajor {
  const T *p;
  int ld;
  __device__ float one(int row, int k) const { return to_f32(p[row * ld + k]); }
};

template <class T>
struct ColMajor {
  const T *p;
  int ld;
  __device__ float one(int row, int k) const { return to_f32(p[k * ld + row]); }
};

struct RowScaled {
  const float *p;
  int ld;
  const float *s;
  __device__ float one(int row, int k) const { return p[row * ld + k] * s[k]; }
};

struct RowNeg {  // -p[row * ld + k], fp32
  const float *p;
  int ld;
  __device__ float one(int row, int k) const { return -p[row * ld + k]; }
};

// 8 consecutive k of one row as split bf16 (hi, lo); defined below split2.
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8 &hi, bf16x8 &lo);

template <bool NEED_LO>
__device__ __forceinline__ void load8f(const float *src, const float *scale, float sign, bf16x8 &hi,
                                       bf16x8 &lo) {
  f32x4 x0 = *reinterpret_cast<const f32x4 *>(src);
  f32x4 x1 = *reinterpret_cast<const f32x4 *>(src + 4);
  float x[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
  if (scale) {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] *= scale[i];
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] *= sign;
  if (NEED_LO) {
    split8(x, hi, lo);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) hi[i] = (bf16)x[i];
  }
}

template <bool NEED_LO>
__device__ __forceinline__ void load8(const RowMajor<float> &a, int row, int k, bf16x8 &hi, bf16x8 &lo) {
  load8f<NEED_LO>(a.p + row * a.ld + k, nullptr, 1.f, hi, lo);
}
template <bool NEED_LO>
__device__ __forceinline__ void load8(const RowScaled &a, int row, int k, bf16x8 &hi, bf16x8 &lo) {
  load8f<NEED_LO>(a.p + row * a.ld + k, a.s + k, 1.f, hi, lo);
}
template <bool NEED_LO>
__device__ __forceinline__ void load8(const RowNeg &a, int row, int k, bf16x8 &hi, bf16x8 &lo) {
  load8f<NEED_LO>(a.p + row * a.ld + k, nullptr, -1.f, hi, lo);
}
template <bool NEED_LO>
__device__ __forceinline__ void load8(const RowMajor<bf16> &a, int row, int k, bf16x8 &hi, bf16x8 &lo) {
  hi = *reinterpret_cast<const bf16x8 *>(a.p + row * a.ld + k);
  (void)lo;
}

// A pre-split fp32 operand: hi = bf16(x), lo = bf16(x - hi), row-major planes.
struct Planes {
  const bf16 *hi;
  const bf16 *lo;
  int ld;
};
template <bool NEED_LO>
__device__ __forceinline__ void load8(const Planes &a, int row, int k, bf16x8 &hi, bf16x8 &lo) {
  hi = *reinterpret_cast<const bf16x8 *>(a.hi + row * a.ld + k);
  if (NEED_LO) lo = *reinterpret_cast<const bf16x8 *>(a.lo + row * a.ld + k);
}
// Column access of exact bf16 data: element (row, k) = p[k * ld + row].
template <bool NEED_LO>
__device__ __forceinline__ void load8(const ColMajor<bf16> &a, int row, int k, bf16x8 &hi, bf16x8 &lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) hi[e] = a.p[(k + e) * a.ld + row];
  (void)lo;
}

template <class Op>
struct IsExactBf16 {
  static constexpr bool value = false;
};
template <>
struct IsExactBf16<RowMajor<bf16>> {
  static constexpr bool value = true;
};
template <>
struct IsExactBf16<ColMajor<bf16>> {
  static constexpr bool value = true;
};

// C[16x16] += A[m0.., k] * B[k, n0..] for k in [k0, k1) (multiple of 32), with
// A given as opA(m, k) and B given through its transpose opB(n, k).
// PA / PB: 2 = split that operand into hi + lo (ignored for exact bf16 data).
// Products formed: hi*hi, plus hi_A*lo_B if PB == 2, plus lo_A*hi_B if PA == 2.
template <int PA, int PB, class OA, class OB>
__device__ __forceinline__ void mma_bf16(f32x4 &c, const OA &opA, const OB &opB, int m0, int n0, int k0,
                                         int k1) {
  constexpr bool LA = (PA == 2) && !IsExactBf16<OA>::value;
  constexpr bool LB = (PB == 2) && !IsExactBf16<OB>::value;
  const int l = lane_id();
  const int r = l & 15, kq = (l >> 4) * 8;
  for (int k = k0; k < k1; k += 32) {
    bf16x8 ah, al, bh, bl;
    load8<LA>(opA, m0 + r, k + kq, ah, al);
    load8<LB>(opB, n0 + r, k + kq, bh, bl);
    c = mfma_bf16(ah, bh, c);
    if (LB) c = mfma_bf16(ah, bl, c);
    if (LA) c = mfma_bf16(al, bh, c);
  }
}

// Same contract with fp32 operands on the fp32 MFMA (k step 4).
template <class OA, class OB>
__device__ __forceinline__ void mma_f32(f32x4 &c, const OA &opA, const OB &opB, int m0, int n0, int k0,
                                        int k1) {
  const int l = lane_id();
  const int r = l & 15, kk = l >> 4;
  for (int k = k0; k < k1; k += 4) c = mfma_f32(opA.one(m0 + r, k + kk), opB.one(n0 + r, k + kk), c);
}

__device__ __forceinline__ void split4(const f32x4 &x, bf16x4 &hi, bf16x4 &lo);  // defined below split2

// Store a C-layout tile into split planes (hi, lo) of a row-major bf16 array.
__device__ __forceinline__ void store_tile_planes(bf16 *hi, bf16 *lo, int ld, int m0, int n0, const f32x4 &c) {
  const int l = lane_id();
  const int col = n0 + (l & 15), row = m0 + 4 * (l >> 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16 h = (bf16)c[i];
    hi[(row + i) * ld + col] = h;
    lo[(row + i) * ld + col] = (bf16)(c[i] - (float)h);
  }
}

// ---------------------------------------------------------------------------
// Wave-wide inclusive prefix sum over the 64 lanes with DPP: row_shr 1, 2,
// 4, 8 scans each row of 16 lanes, then row_bcast:15 and row_bcast:31 carry
// the row totals upward (GFX9 wave64 DPP controls).  Lanes with no source
// keep the "old" operand, 0.
// ---------------------------------------------------------------------------
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_src(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xf, false));
}
__device__ __forceinline__ float wave_inclusive_scan(float x) {
  x += dpp_src<0x111, 0xf>(x);  // row_shr:1
  x += dpp_src<0x112, 0xf>(x);  // row_shr:2
  x += dpp_src<0x114, 0xf>(x);  // row_shr:4
  x += dpp_src<0x118, 0xf>(x);  // row_shr:8
  x += dpp_src<0x142, 0xa>(x);  // row_bcast:15 into rows 1 and 3
  x += dpp_src<0x143, 0xc>(x);  // row_bcast:31 into rows 2 and 3
  return x;
}
// Sum over the 16 lanes of a DPP row (lanes 16 r .. 16 r + 15): the quad
// pairs (lane ^ 1), the quads' halves (lane ^ 2), the two quads of each
// half-row (mirror in 8), the two half-rows (mirror in 16).  Every step adds
// the same two partial sums in both lanes of a pair, so all 16 lanes end
// with the same bits.  (DPP moves stay in the VALU; a shuffle by
// ds_bpermute is an LDS round trip per step.)
template <int CTRL>
__device__ __forceinline__ float dpp_row(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_row<0xB1>(x);    // quad_perm [1, 0, 3, 2]
  x += dpp_row<0x4E>(x);    // quad_perm [2, 3, 0, 1]
  x += dpp_row<0x141>(x);   // row_half_mirror
  x += dpp_row<0x140>(x);   // row_mirror
  return x;
}
__device__ __forceinline__ float lane_value(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

// log(alpha) of a gate with a finite floor.  Decays are formed as
// exp(g_r - g_s) from cumulative sums g of these values; a gate of 0 (or one
// below e^kLogGateFloor, including subnormals) would make g = -inf and
// (-inf) - (-inf) = NaN.  With the floor such a gate scales the carried
// state by e^-60 (about 8.8e-27) instead of 0: far below any tolerance,
// while 64 floored gates in one chunk keep |g| <= 3840, where the fp32
// rounding of the sums stays near 1e-4 absolute.
constexpr float kLogGateFloor = -60.f;
__device__ __forceinline__ float log_gate(float alpha) { return fmaxf(logf(alpha), kLogGateFloor); }

// ---------------------------------------------------------------------------
// Fragments with a permuted contraction index.  A C-layout 16 x 16 result
// (lane l holds rows 4 (l >> 4) .. + 3 of column l & 15) is used directly as
// the B operand of a k = 32 MFMA by pairing two such tiles: lane group
// g = l >> 4 then supplies the rows {4g .. 4g+3} of the first tile and
// {4g .. 4g+3} of the second, i.e. the physical k indices
// {4g + e, 16 + 4g + e} (e < 4) of the 32-wide step.  Any A operand of the
// same product must be read with the same k order; a sum over k does not
// depend on the order.
// ---------------------------------------------------------------------------
typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 cat_bf16x8(uint2 a, uint2 b) {
  union { uint4 u; bf16x8 v; } x;
  x.u = uint4{a.x, a.y, b.x, b.y};
  return x.v;
}

// Transposing LDS read (gfx950 ds_read_b64_tr_b16): within each group of 16
// lanes, output lane i element e is element (i mod 4) of the 8 bytes read by
// source lane 4e + i/4.  Pointing source lane q of group g at
// M[r0 + 4g + q/4][c0 + 4 (q mod 4)] of a row-major bf16 matrix M therefore
// gives lane i the column c0 + i, rows r0 + 4g + e (e < 4): a k = 16 A
// fragment of M^T.  Issue it with every lane of the wave on: under a partial
// or empty EXEC mask the destination is still written, with unusable data.
// It carries no alias information either, so while a load-to-LDS copy is in
// flight the compiler makes it wait for that copy.
__device__ __forceinline__ uint2 ds_read_tr16(const bf16 *p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(p));
  union { s16x4 s; uint2 u; } x;
  x.s = v;
  return x.u;
}

// Two fp32 values as packed bf16 (round to nearest even, v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), bf16x2));
}
// Split-bf16 of a pair with one rounding per part: hi = bf16(x), read back
// exactly by shifting the packed bits, lo = bf16(x - hi).
__device__ __forceinline__ void split2(float a, float b, uint32_t &hi, uint32_t &lo) {
  hi = pack_bf16x2(a, b);
  const float ha = __uint_as_float(hi << 16), hb = __uint_as_float(hi & 0xffff0000u);
  lo = pack_bf16x2(a - ha, b - hb);
}

// Split two C-layout tiles into a k = 32 B fragment (hi, lo).
__device__ __forceinline__ void b_frag_split(const f32x4 &t0, const f32x4 &t1, bf16x8 &hi, bf16x8 &lo) {
  uint4 h, o;
  split2(t0[0], t0[1], h.x, o.x);
  split2(t0[2], t0[3], h.y, o.y);
  split2(t1[0], t1[1], h.z, o.z);
  split2(t1[2], t1[3], h.w, o.w);
  hi = __builtin_bit_cast(bf16x8, h);
  lo = __builtin_bit_cast(bf16x8, o);
}

__device__ __forceinline__ void split8(const float (&x)[8], bf16x8 &hi, bf16x8 &lo) {
  uint4 h, o;
  split2(x[0], x[1], h.x, o.x);
  split2(x[2], x[3], h.y, o.y);
  split2(x[4], x[5], h.z, o.z);
  split2(x[6], x[7], h.w, o.w);
  hi = __builtin_bit_cast(bf16x8, h);
  lo = __builtin_bit_cast(bf16x8, o);
}

__device__ __forceinline__ void split4(const f32x4 &x, bf16x4 &hi, bf16x4 &lo) {
  uint2 h, o;
  split2(x[0], x[1], h.x, o.x);
  split2(x[2], x[3], h.y, o.y);
  hi = __builtin_bit_cast(bf16x4, h);
  lo = __builtin_bit_cast(bf16x4, o);
}

// ---------------------------------------------------------------------------
// Load-to-LDS DMA (gfx950 buffer_load_dwordx4 ... lds / global_load_lds_dwordx4):
// lane l of the wave copies 16 bytes from its own source address to
// dst + 16 l; completion is counted by vmcnt.  The buffer form reads through
// a raw descriptor covering nbytes from base: lanes past the range write
// zeros.  (The builtins exist only for the device pass; the host pass of a
// kernel template must not see them.)
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void dma16_buffer(const void *base, uint32_t nbytes, lds_void *dst, uint32_t voff,
                                             uint32_t soff = 0) {
#if defined(__HIP_DEVICE_COMPILE__)
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, nbytes, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, soff, 0, 0);
#endif
}
__device__ __forceinline__ void dma16_global(const void *src, lds_void *dst) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
#endif
}
// 4 bytes per lane through a raw descriptor: lane l copies the dword at
// base + voff (4-byte aligned) to dst + 4 l.
__device__ __forceinline__ void dma4_buffer(const void *base, uint32_t nbytes, lds_void *dst, uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, nbytes, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 4, voff, 0, 0, 0);
#endif
}

// Wait until at most N vector-memory operations of this wave are
// outstanding (vmcnt is split across bits 3:0 and 15:14 of the immediate).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}
// Wait for all outstanding vector-memory loads of this wave (vmcnt(0)).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Workgroup barrier for LDS hand-offs only: waits for this wave's LDS
// operations, not for its outstanding global loads (which stay in flight
// across the barrier; their consumers wait for them as usual).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Make prior LDS writes of this wave visible to its later LDS reads.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Store a C-layout tile into a row-major fp32 LDS array (optionally scaled per column).
__device__ __forceinline__ void store_tile(float *dst, int ld, int m0, int n0, const f32x4 &c) {
  const int l = lane_id();
  const int col = n0 + (l & 15), row = m0 + 4 * (l >> 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[(row + i) * ld + col] = c[i];
}

}  // namespace gdn
