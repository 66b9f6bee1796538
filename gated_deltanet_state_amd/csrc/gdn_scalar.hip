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
// bf16 at dk = dv = 128 runs scalar_op_dma_kernel instead: the same
// arithmetic with every input copied to LDS by load-to-LDS DMA, three steps
// in flight (0.173 -> 0.157 ms on 64 x 512 tokens x 32 heads).
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
// gamma of a chunk, in wave 0: lane l multiplies the alphas of tokens l,
// l + 64, l + 128, ... in that order, then the lanes are combined by xor
// shuffles.  The loads go out eight at a time (indices clamped into the
// chunk, the surplus multiplied as 1): a load per iteration, each waited
// for before the next was issued, made the rest of the workgroup wait at
// its first barrier for eight memory round trips per 512 tokens.
template <typename TI>
__device__ __forceinline__ float chunk_gate_product(const TI *alpha, int64_t t0, int L, int H, int h) {
  const int l = lane_id();
  float g = 1.f;
  for (int j0 = 0; j0 < L; j0 += 8 * 64) {
    float x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = to_f32(alpha[(t0 + min(j0 + 64 * u + l, L - 1)) * H + h]);
#pragma unroll
    for (int u = 0; u < 8; ++u) g *= j0 + 64 * u + l < L ? x[u] : 1.f;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) g *= __shfl_xor(g, m, 64);
  return g;
}

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
    const float g = chunk_gate_product(alpha, t0, L, p.H, h);
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
    lds_barrier();   // (LDS only: __syncthreads' fence would also wait for the loads in flight)
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
    lds_barrier();
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

// Transposing reads of one step's key fragments: block j from the 8-byte
// reads at addr[j] (rows 0..15) and addr[j] + 4096 (rows 16..31), all in one
// inline-assembly group with its own lgkmcnt wait (as a compiler builtin the
// read carries no alias information and would be made to wait for every
// load-to-LDS copy in flight); early-clobber results, so no result shares a
// register with an address.
__device__ __forceinline__ void key_frags_tr(const uint32_t (&addr)[8], bf16x8 (&b)[8]) {
  uint2 r[16];
  asm volatile(
      "ds_read_b64_tr_b16 %0, %16 offset:0\n\t"
      "ds_read_b64_tr_b16 %1, %16 offset:4096\n\t"
      "ds_read_b64_tr_b16 %2, %17 offset:0\n\t"
      "ds_read_b64_tr_b16 %3, %17 offset:4096\n\t"
      "ds_read_b64_tr_b16 %4, %18 offset:0\n\t"
      "ds_read_b64_tr_b16 %5, %18 offset:4096\n\t"
      "ds_read_b64_tr_b16 %6, %19 offset:0\n\t"
      "ds_read_b64_tr_b16 %7, %19 offset:4096\n\t"
      "ds_read_b64_tr_b16 %8, %20 offset:0\n\t"
      "ds_read_b64_tr_b16 %9, %20 offset:4096\n\t"
      "ds_read_b64_tr_b16 %10, %21 offset:0\n\t"
      "ds_read_b64_tr_b16 %11, %21 offset:4096\n\t"
      "ds_read_b64_tr_b16 %12, %22 offset:0\n\t"
      "ds_read_b64_tr_b16 %13, %22 offset:4096\n\t"
      "ds_read_b64_tr_b16 %14, %23 offset:0\n\t"
      "ds_read_b64_tr_b16 %15, %23 offset:4096\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7]),
        "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]), "=&v"(r[12]), "=&v"(r[13]), "=&v"(r[14]),
        "=&v"(r[15])
      : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]), "v"(addr[4]), "v"(addr[5]), "v"(addr[6]),
        "v"(addr[7]));
#pragma unroll
  for (int j = 0; j < 8; ++j) b[j] = cat_bf16x8(r[2 * j], r[2 * j + 1]);
}
// The value fragment of the same step (one block, two reads, one wait).
__device__ __forceinline__ bf16x8 value_frag_tr(uint32_t addr) {
  uint2 r0, r1;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %2 offset:0\n\t"
      "ds_read_b64_tr_b16 %1, %2 offset:4096\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1)
      : "v"(addr));
  return cat_bf16x8(r0, r1);
}

// scalar_op_kernel for bf16 at dk = dv = 128, with every input copied
// global -> LDS by load-to-LDS DMA instead of through registers: the same
// contraction, step order and weights, but no register is a load
// destination, so none of the compiler's waits can drain the copies in
// flight (waits for loaded registers across the loop are conservative, and
// __syncthreads' fence waits for all of them).  NS LDS stages, each one
// step's 32 key and 32 value rows (16 KiB) and the next step's gates; at the
// top of step i every wave issues its share of stage i + NS - 1's copies
// (indices clamped into the chunk, so every wave issues the same four
// operations every step and the wait for stage i is a fixed count).  Wave 0
// turns the gates into the next step's weights after its products (two
// weight sets), so a step needs two barriers.  Rows are 256 bytes without
// padding: the 32-byte groups of row r sit at group index g ^ (r & 7), so
// the transposing reads of eight rows at one column group meet eight
// distinct bank groups.  The copies go through raw buffer descriptors
// (tensor start, tensor bytes < 2^31).  Rows past the chunk's end repeat its
// last (finite) row with weight zero.  The gates are copied as the aligned
// dwords that hold them (the other half is discarded; an aligned dword
// never crosses a page).
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4))) scalar_op_dma_kernel(ScalarOpLaunch p) {
  constexpr int D = 128, NB = D / 16, ROWB = 2 * D;   // row bytes
  constexpr int TB = SB * ROWB;                        // one tensor's rows in a stage
  constexpr int STB = 2 * TB + 512;                    // a stage: keys, values, 64 alpha + 64 beta dwords
  constexpr int NS = 3;                                // stages (copies run NS - 1 steps ahead; 4: 4% slower)
  // one LDS object (stages, then the weights)
  __shared__ __align__(16) char sBuf[NS * STB + 2 * SB * 4];
  float *const sU = reinterpret_cast<float *>(sBuf + NS * STB);   // two sets of weights
  const int c = blockIdx.x / p.H, h = blockIdx.x % p.H;
  const int t0 = p.cu[c], L = p.cu[c + 1] - t0;
  const int w = __builtin_amdgcn_readfirstlane(wave_id()), l = lane_id();   // (descriptors need w uniform)
  const bf16 *alpha = reinterpret_cast<const bf16 *>(p.alpha), *beta = reinterpret_cast<const bf16 *>(p.beta);

  if (w == 0) {   // gamma = the product of the chunk's alphas
    const float g = chunk_gate_product(alpha, t0, L, p.H, h);
    if (l == 0) p.gamma[(int64_t)c * p.H + h] = g;
  }
  if (!p.S_local) return;

  f32x4 acc[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) acc[j] = zero4();
  if (L > 0) {
    const int first = (L - 1) / SB * SB, nsteps = first / SB + 1;   // steps run from the chunk's end backwards
    auto tok = [&](int s0, int r) { return t0 + min(s0 + r, L - 1); };
    const uint32_t row_bytes = (uint32_t)(p.n_tokens * p.H * D * 2);
    const uint32_t gate_bytes = (uint32_t)((p.n_tokens * p.H * 2 + 3) & ~int64_t(3));
    const int isv = w >> 2;   // waves 0..3 copy keys, 4..7 values
    const bf16 *rows = reinterpret_cast<const bf16 *>(isv ? p.v : p.k);
    auto s0_of = [&](int i) { return first - SB * min(i, nsteps - 1); };
    // gates of step j into the gate area at g (every wave alike; lanes
    // 32..63 repeat 0..31)
    auto copy_gates = [&](int j, char *g) {
      const int64_t e = (int64_t)tok(s0_of(j), l & (SB - 1)) * p.H + h;
      dma4_buffer(alpha, gate_bytes, (lds_void *)g, (uint32_t)(4 * (e >> 1)));
      dma4_buffer(beta, gate_bytes, (lds_void *)(g + 256), (uint32_t)(4 * (e >> 1)));
    };
    // stage i % NS: the rows of step i (wave w copies 4-row pieces 2w and
    // 2w + 1; lane l: row 4 (piece & 7) + (l >> 4), its 16-byte slot l & 15
    // holding piece-of-row (slot ^ 2 (row & 7))) and the gates of step i + 1
    auto copy = [&](int i) {
      const int s0 = s0_of(i);
      char *st = sBuf + (i % NS) * STB;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int n = 2 * w + u, row = 4 * (n & 7) + (l >> 4), slot = l & 15;
        const int piece = ((((slot >> 1) ^ (row & 7)) << 1) | (slot & 1));
        const uint32_t off = (uint32_t)((((int64_t)tok(s0, row) * p.H + h) * D + 8 * piece) * 2);
        dma16_buffer(rows, row_bytes, (lds_void *)(st + isv * TB + (n & 7) * 1024), off);
      }
      copy_gates(i + 1, st + 2 * TB);
    };
    float later = 1.f;   // product of the alphas of the steps already done (wave 0)
    // wave 0: the weights of step j from its gates at g into sU set j & 1
    auto weights = [&](int j, const char *g) {
      const int s0 = s0_of(j);
      const int64_t e = (int64_t)tok(s0, l & (SB - 1)) * p.H + h;
      const uint32_t ad = reinterpret_cast<const uint32_t *>(g)[l & (SB - 1)];
      const uint32_t bd = reinterpret_cast<const uint32_t *>(g + 256)[l & (SB - 1)];
      const bool in = l < SB && s0 + l < L;
      const float pa = in ? __uint_as_float((e & 1) ? (ad & 0xffff0000u) : (ad << 16)) : 1.f;
      const float pb = in ? __uint_as_float((e & 1) ? (bd & 0xffff0000u) : (bd << 16)) : 0.f;
      const float P = wave_inclusive_scan(log_gate(pa));
      const float tot = lane_value(P, 63);
      if (l < SB) sU[(j & 1) * SB + l] = pb * later * expf(tot - P);
      later *= expf(tot);
    };
    // the gates of step 0 (in the last stage's gate area, free until step 0
    // issues that stage's copies), then stages 0 .. NS - 2; the weights of step 0
    copy_gates(0, sBuf + (NS - 1) * STB + 2 * TB);
#pragma unroll
    for (int j = 0; j < NS - 1; ++j) copy(j);
    wait_vmcnt<4 * (NS - 1)>();
    if (w == 0) weights(0, sBuf + (NS - 1) * STB + 2 * TB);
    const int g4 = l >> 4, q = l & 15, row0 = 4 * g4 + (q >> 2);
    // this lane's transposing reads: row row0 (and row0 + 16), 8 bytes at
    // 8 (q & 3) in column group j, which sits at group j ^ (row0 & 7)
    uint32_t ka[NB];
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void *)(sBuf) + row0 * ROWB + 8 * (q & 3);   // LDS offset
#pragma unroll
    for (int j = 0; j < NB; ++j) ka[j] = lds0 + 32 * (j ^ (row0 & 7));
    const uint32_t va = lds0 + TB + 32 * (w ^ (row0 & 7));
    for (int i = 0; i < nsteps; ++i) {
      lds_barrier();   // step i - 1 is done with its stage and weight set
      copy(i + NS - 1);
      wait_vmcnt<4 * (NS - 1)>();   // stage i: issued before those of steps i + 1 .. i + NS - 1 (4 operations each)
      lds_barrier();   // (barriers wait for LDS operations only: a fence would wait for every copy)
      const uint32_t so = (uint32_t)((i % NS) * STB);
      uint32_t kas[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j) kas[j] = ka[j] + so;
      bf16x8 bh[NB];
      key_frags_tr(kas, bh);
      const bf16x8 vv = value_frag_tr(va + so);
      const float *su = sU + (i & 1) * SB;   // written during step i - 1 (or before step 0)
      const f32x4 u0 = *reinterpret_cast<const f32x4 *>(su + 4 * g4);
      const f32x4 u1 = *reinterpret_cast<const f32x4 *>(su + 16 + 4 * g4);
      float a[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a[e] = (float)vv[e] * u0[e];
        a[4 + e] = (float)vv[4 + e] * u1[e];
      }
      bf16x8 ah, al;
      split8(a, ah, al);
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        acc[j] = mfma_bf16(ah, bh[j], acc[j]);
        acc[j] = mfma_bf16(al, bh[j], acc[j]);
      }
      // wave 0: the next step's weights (its gates came with stage i), into
      // the other set, read after the next step's barriers
      if (w == 0) weights(i + 1, sBuf + so + 2 * TB);
    }
    wait_vmem();   // the copies issued past the last step have landed before the workgroup ends
  }
  // S_local[c, h] row-major [D][D]: lane holds rows 4 (l >> 4) + i, column l & 15
  float *out = p.S_local + ((int64_t)c * p.H + h) * D * D;
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) out[(16 * w + 4 * (l >> 4) + e) * D + 16 * j + (l & 15)] = acc[j][e];
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
  if (p.in_bf16 && DK == 128 && DV == 128 && p.n_tokens * p.H * DK * 2 < (int64_t(1) << 31))
    return launch_kernel(scalar_op_dma_kernel, dim3((unsigned)items), dim3(512), 0, stream, p);
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
