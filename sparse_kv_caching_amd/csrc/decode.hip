// K4: one decode token for every unit (LoLA notes §2.4, the per-token update,
// read first as in the chunk schedule with C = 1).
//
// Per unit (b, KV head), with n tokens already seen and the new pair at n:
//   read   y = (H^T phi(q) + sum_V a v) / (phi(q)^T s + sum_V a) over the cache
//          G and positions max(0, n - eta) .. n (Eq. (14));
//   update the pair at n - eta leaves the window; E = G u {it}: if |E| <=
//          lam it is cached, else every candidate is scored by SRE against
//          (H, s) and the lowest (ties: the newer position) is folded into H,
//          s; if that was a cache entry, the leaving pair takes its slot
//          (Eqs. (10)-(13)).  The new pair enters the ring slot n % eta.
//
// The step is bound by HBM traffic (H and s read and written once, the window
// and cache K / V read once), so the kernel is shaped for every unit to be
// resident at once, with the reads issued up front in two waves:
//
//   * One workgroup of 4 waves per unit.  For bf16 state it needs at most
//     80 KB of LDS and 256 registers per lane, so two workgroups share a CU.
//   * The keys a query sees (cache 0..gs-1, window oldest first; the new pair
//     apart) come in chunks of 128, 32 per wave (wave w: keys 16 w .. and
//     64 + 16 w ..), loaded straight into the registers of the wave's MFMA
//     operands; the wave also loads its keys' V rows.  W^T, the queries, s and the leaving and new pairs go to LDS.
//     Only when those reads have arrived does the wave issue its slab of H,
//     so that across the GPU the keys and values come back first and the
//     logits and phi work overlaps the stream of H.
//   * Per wave: logits S^T = K Q^T of its keys (MFMA, 16 x 16 x 32), a
//     softmax with a wave-local running max, and P V on the VALU.  The
//     partials of the four waves are merged once; the linear read enters as
//     the term with logit 0; the new pair's logits are dot products.
//   * SRE candidates are keys 0..gs (the leaving pair is key gs).  phi of
//     the candidate rows (and of the queries) is computed once, by the wave
//     holding the rows, and stored in LDS as 16-bit hi / lo operands with
//     the row's normalisers and phi^T s.  Wave w owns the 32-column slab w
//     of H (H lives on the device as H^T [d][D], so the slab arrives in
//     operand layout) and multiplies it by every phi tile: its columns of
//     the SRE parts and of H^T phi(q).
//   * Wave 0 picks the argmin and takes phi of the folded row from its
//     tile; every slab wave adds the rank-1 term to its registers and writes
//     the slab back once.
#include "internal.h"

namespace lola {

namespace {
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int WP = 8;   // row padding (elements) of W^T and q in LDS (bank spread)
constexpr size_t kLdsPair = 80 * 1024;    // two workgroups per CU
constexpr size_t kLdsOne = 160 * 1024;

constexpr int kKC = 32 * kWaves;   // keys per chunk: a 32-key tile per wave
static_assert(kKC == kDecodeOneChunkKeys, "the host's view of the one-chunk instance");

// phi tiles of 16 rows per chunk: the candidate rows of the chunk, then (last
// chunk) the new pair when it is a candidate and the g <= 4 query rows
__host__ __device__ inline int dec_phi_tiles(int lam, int eta) {
  const int rows = (lam + eta <= kKC ? lam + 1 : kKC + 1) + 4;
  return (rows + 15) / 16;
}

// Byte offsets of the LDS arrays.
struct DecLayout {
  uint32_t wt, q, lk, lv, nk, nv, ve, s, cpos, spart, logit, nlin, pv, phe, wst, zq, red, slot,
      meta, pend, total;
  int ntile;
};

inline __host__ __device__ uint32_t al16(uint32_t x) { return (x + 15u) & ~15u; }

__host__ __device__ inline DecLayout dec_layout(int lam, int eta, int d, int esz) {
  DecLayout L;
  uint32_t off = 0;
  auto take = [&](uint32_t b) { const uint32_t o = off; off = al16(off + b); return o; };
  const uint32_t row = (uint32_t)(d + WP) * esz;
  L.ntile = dec_phi_tiles(lam, eta);
  L.wt = take(kM * row);                               // [kM][d + WP] W^T of this KV head
  L.q = take(4 * row);                                 // [g][d + WP] queries
  L.lk = take((uint32_t)d * esz);                      // leaving pair
  L.lv = take((uint32_t)d * esz);
  L.nk = take((uint32_t)d * esz);                      // new pair
  L.nv = take((uint32_t)d * esz);
  L.ve = take((uint32_t)d * 4);                        // value of the folded row
  L.s = take(kD * 4);                                  // s
  L.cpos = take((uint32_t)lam * 4);                    // cache positions
  L.spart = take((uint32_t)(d / 32) * (lam + 1) * 4);  // [slab][candidate] SRE parts
  L.logit = take(kKC * 16);                            // [key][4] softmax weights
  L.nlin = take((uint32_t)4 * d * 4);                  // [g][d] H^T phi(q)
  L.pv = take((uint32_t)kWaves * 4 * d * 4);           // [wave][4][d] P V partials
  L.phe = take(kD * 4);                                // phi of the folded row
  L.wst = take(kWaves * 8 * 4);                        // [wave][max 4, sum 4]
  L.zq = take(4 * 4);                                  // [g] phi(q)^T s
  L.red = take(16);                                    // the folded row
  L.slot = take((uint32_t)L.ntile * 8 * 64 * 16);      // [tile][kb][hi, lo][lane] phi operands
  L.meta = take((uint32_t)L.ntile * 16 * 16);          // [tile][row] 1/S+, 1/S-, phi^T s
  // held-back fold terms [k][phi, v] (the one-chunk instance only)
  L.pend = take(lam + eta <= kKC ? (uint32_t)kPend * (kD + d) * 4 : 0u);
  L.total = off;
  return L;
}

// 8 consecutive input elements as a 16-bit MFMA operand (hi; lo for split types)
__device__ __forceinline__ void xop(const BF16&, const uint16_t* p, u32x4& hi, u32x4& lo) {
  hi = ld16(p);
  lo = u32x4{0, 0, 0, 0};
}
__device__ __forceinline__ void xop(const F32&, const float* p, u32x4& hi, u32x4& lo) {
  float x[8];
  load8_f32(p, x);
  splitop<F32>(x, hi, lo);
}

// v_mfma_f32_16x16x32_{bf16,f16}: A is 16 x 32 (M x K), B is 32 x 16 (K x N).
// Lane l supplies row / column (l % 16) and the 8 K-values 8 (l / 16) + j;
// the output lane l holds column (l % 16), rows 4 (l / 16) + i, i = 0..3.
// Because a contraction may permute its K index freely (A and B agreeing), a
// C-layout result feeds the next product directly; within a 32-wide K-block
// kb the lane group q = l / 16 then holds the K-slots
//     sigma(kb, q, j) = 32 kb + 16 (j / 4) + 4 q + (j % 4),  j = 0..7.
__device__ __forceinline__ f32x4 mma16(const BF16&, u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(const F32&, u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
// a b with the split passes of the type (hi hi + hi lo + lo hi for fp32 inputs)
template <class DT>
__device__ __forceinline__ f32x4 mma16x(u32x4 ah, u32x4 al, u32x4 bh, u32x4 bl, f32x4 c) {
  const DT dt{};
  c = mma16(dt, ah, bh, c);
  if constexpr (DT::kSplit) {
    c = mma16(dt, ah, bl, c);
    c = mma16(dt, al, bh, c);
  }
  return c;
}

__device__ __forceinline__ float ldf(const uint16_t* p) { return bf16_bits_to_f32(*p); }
__device__ __forceinline__ float ldf(const float* p) { return *p; }
// Sum / max / min over the four lane groups q of a 16-lane column, on the
// VALU: v_permlane16_swap of x with itself gives the lanes of rows 2i and
// 2i + 1 the pair (x in row 2i, x in row 2i + 1) of their column, and
// v_permlane32_swap the pair of halves; every lane of the column combines the
// same operands in the same order ((x0 o x1) o (x2 o x3)).  The four lanes
// of a column are always active together.
template <class Op>
__device__ __forceinline__ float qreduce(float x, Op op) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = op(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return op(__uint_as_float(t[0]), __uint_as_float(t[1]));
}
__device__ __forceinline__ float qsum(float x) { return qreduce(x, [](float a, float b) { return a + b; }); }
__device__ __forceinline__ float qmax(float x) { return qreduce(x, [](float a, float b) { return fmaxf(a, b); }); }
__device__ __forceinline__ float qmin(float x) { return qreduce(x, [](float a, float b) { return fminf(a, b); }); }

constexpr float kL2E = 1.4426950408889634f;

// Pre-activations of phi for 16 rows: U^T = W x^T; bop(kb, hi, lo) gives the
// lane's x operand of k-block kb (row n, k = 32 kb + 8 q ..); W^T rows
// f = 16 mt + n, row stride HD + WP elements (LDS).  U[mt][i] is feature
// 16 mt + 4 q + i of row n.  The operands of k-block kb + 1 are read while
// kb's products run; the scheduling barriers keep the compiler from
// hoisting every block's reads.
template <class DT, int HD, class BOp>
__device__ __forceinline__ void pre16(BOp bop, const typename DT::T* WT, int n, int q,
                                      f32x4 (&U)[4]) {
  constexpr int KB = HD / 32;
  const DT dt{};
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) U[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 bh, bl, ah[4], al[4];
  auto ops = [&](int kb) {
    bop(kb, bh, bl);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) xop(dt, WT + (16 * mt + n) * (HD + WP) + 32 * kb + 8 * q, ah[mt], al[mt]);
  };
  ops(0);
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    u32x4 cah[4], cal[4];
    const u32x4 cbh = bh, cbl = bl;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) { cah[mt] = ah[mt]; cal[mt] = al[mt]; }
    if (kb + 1 < KB) ops(kb + 1);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) U[mt] = mma16x<DT>(cah[mt], cal[mt], cbh, cbl, U[mt]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// phi from the pre-activations: ph[half][mt][i] = phi[64 half + 16 mt + 4 q + i]
// of the lane's row.
__device__ __forceinline__ void phi16(const f32x4 (&U)[4], float (&ph)[2][4][4]) {
  float mx = -INFINITY, mn = INFINITY;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) { mx = fmaxf(mx, U[mt][i]); mn = fminf(mn, U[mt][i]); }
  mx = qmax(mx);
  mn = qmin(mn);
  // e^(u - max) = 2^(u log2 e - max log2 e)
  const float mxl = mx * kL2E, mnl = mn * kL2E;
  float sp = 0.f, sn = 0.f;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ph[0][mt][i] = __builtin_amdgcn_exp2f(fmaf(U[mt][i], kL2E, -mxl));
      ph[1][mt][i] = __builtin_amdgcn_exp2f(fmaf(-U[mt][i], kL2E, mnl));
      sp += ph[0][mt][i];
      sn += ph[1][mt][i];
    }
  const float ip = 1.f / qsum(sp), in_ = 1.f / qsum(sn);
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) { ph[0][mt][i] *= ip; ph[1][mt][i] *= in_; }
}

// The wave's slab of H in the lane's operand positions: lane (n, q) holds
// H[sigma(kb, q, j)][16 mb + n].  For bf16 state the products use the 16-bit
// pair of the three-pass scheme, hi = bf16(x) and mid = bf16(x - hi), split
// once; the fold needs the fp32 values, which the one-chunk instance keeps
// as they are (fewer instructions) and the chunked one, short of registers,
// as a third bf16 part lo = bf16(x - hi - mid) (hi + mid + lo is exactly x).
// fp32 state keeps fp32 and splits on use.
template <class DT, bool KEEP> struct HSlab;
template <> struct HSlab<BF16, true> {
  float v[2][4][8];
  u32x4 hi[2][4], mid[2][4];
  __device__ __forceinline__ void set(int mb, int kb, const float (&x)[8]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a0 = x[2 * j], a1 = x[2 * j + 1];
      const uint32_t h = cvt_pk_bf16(a0, a1);
      hi[mb][kb][j] = h;
      mid[mb][kb][j] = cvt_pk_bf16(a0 - __uint_as_float(h << 16), a1 - __uint_as_float(h & 0xFFFF0000u));
      v[mb][kb][2 * j] = a0;
      v[mb][kb][2 * j + 1] = a1;
    }
  }
  __device__ __forceinline__ void ops(int mb, int kb, u32x4& Ah, u32x4& Al) const {
    Ah = hi[mb][kb];
    Al = mid[mb][kb];
  }
  __device__ __forceinline__ void get(int mb, int kb, float (&x)[8]) const {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = v[mb][kb][j];
  }
};
template <> struct HSlab<BF16, false> {
  u32x4 hi[2][4], mid[2][4], lo[2][4];
  __device__ __forceinline__ void set(int mb, int kb, const float (&x)[8]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a0 = x[2 * j], a1 = x[2 * j + 1];
      const uint32_t h = cvt_pk_bf16(a0, a1);
      const float r0 = a0 - __uint_as_float(h << 16), r1 = a1 - __uint_as_float(h & 0xFFFF0000u);
      const uint32_t m = cvt_pk_bf16(r0, r1);
      hi[mb][kb][j] = h;
      mid[mb][kb][j] = m;
      lo[mb][kb][j] = cvt_pk_bf16(r0 - __uint_as_float(m << 16), r1 - __uint_as_float(m & 0xFFFF0000u));
    }
  }
  __device__ __forceinline__ void ops(int mb, int kb, u32x4& Ah, u32x4& Al) const {
    Ah = hi[mb][kb];
    Al = mid[mb][kb];
  }
  __device__ __forceinline__ void get(int mb, int kb, float (&x)[8]) const {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t h = hi[mb][kb][j], m = mid[mb][kb][j], l = lo[mb][kb][j];
      x[2 * j] = (__uint_as_float(h << 16) + __uint_as_float(m << 16)) + __uint_as_float(l << 16);
      x[2 * j + 1] = (__uint_as_float(h & 0xFFFF0000u) + __uint_as_float(m & 0xFFFF0000u)) +
                     __uint_as_float(l & 0xFFFF0000u);
    }
  }
};
template <bool KEEP> struct HSlab<F32, KEEP> {
  float v[2][4][8];
  __device__ __forceinline__ void set(int mb, int kb, const float (&x)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[mb][kb][j] = x[j];
  }
  __device__ __forceinline__ void ops(int mb, int kb, u32x4& Ah, u32x4& Al) const {
    splitop<F32>(v[mb][kb], Ah, Al);
  }
  __device__ __forceinline__ void get(int mb, int kb, float (&x)[8]) const {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = v[mb][kb][j];
  }
};

// phi of a 16-row tile into its LDS slot.  phi = [e+ / S+, e- / S-] with
// e+- the exponentials of +-u less their max and S+- their sums: the slot
// holds the unnormalised e as 16-bit hi / lo operands in the B layout of the
// H product (k-block kb: features sigma(kb, q, j), half kb / 2; lane (n, q)
// keeps its own 16 bytes), meta[n] = (1 / S+, 1 / S-, phi^T s).
template <class DT>
__device__ __forceinline__ void phi_to_slot(const f32x4 (&U)[4], const float* s, int lane, int n,
                                            int q, u32x4* slot, float* meta) {
  float mx = -INFINITY, mn = INFINITY;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) { mx = fmaxf(mx, U[mt][i]); mn = fminf(mn, U[mt][i]); }
  mx = qmax(mx);
  mn = qmin(mn);
  const float mxl = mx * kL2E, mnl = mn * kL2E;
  float sum[2] = {0.f, 0.f}, zs[2] = {0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const int half = kb >> 1, mt0 = 2 * (kb & 1);
    const f32x4 s0 = *reinterpret_cast<const f32x4*>(s + 32 * kb + 4 * q);
    const f32x4 s1 = *reinterpret_cast<const f32x4*>(s + 32 * kb + 16 + 4 * q);
    float e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float uu = U[mt0 + (j >> 2)][j & 3];
      e[j] = __builtin_amdgcn_exp2f(half ? fmaf(-uu, kL2E, mnl) : fmaf(uu, kL2E, -mxl));
      sum[half] += e[j];
      zs[half] = fmaf(e[j], j < 4 ? s0[j] : s1[j - 4], zs[half]);
    }
    u32x4 Bh, Bl;
    splitop<DT>(e, Bh, Bl);
    slot[(2 * kb) * 64 + lane] = Bh;
    slot[(2 * kb + 1) * 64 + lane] = Bl;
  }
  const float ip = 1.f / qsum(sum[0]), in_ = 1.f / qsum(sum[1]);
  const float z = qsum(zs[0]) * ip + qsum(zs[1]) * in_;
  if (q == 0) *reinterpret_cast<f32x4*>(meta + 4 * n) = f32x4{ip, in_, z, 0.f};
}

// P^T = H_slab^T phi^T for the 16 rows of a slot: three passes per k-block
// (H hi / lo from the slab, phi hi / lo from the slot) into the products of
// the two halves, normalised by the row's meta.
// Lane (n, q) gets P[mb][i] = P^T[16 mb + 4 q + i][row n] and z of row n.
template <class DT, class Slab>
__device__ __forceinline__ void slab_prod(const u32x4* slot, const float* meta, const Slab& Hs,
                                          int lane, int n, f32x4 (&P)[2], float& z) {
  const DT dt{};
  f32x4 Pp[2], Pn[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) { Pp[mb] = f32x4{0.f, 0.f, 0.f, 0.f}; Pn[mb] = Pp[mb]; }
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const u32x4 Bh = slot[(2 * kb) * 64 + lane], Bl = slot[(2 * kb + 1) * 64 + lane];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      u32x4 Ah, Al;
      Hs.ops(mb, kb, Ah, Al);
      f32x4& A = (kb >> 1) ? Pn[mb] : Pp[mb];
      A = mma16(dt, Ah, Bh, A);
      A = mma16(dt, Ah, Bl, A);
      A = mma16(dt, Al, Bh, A);
    }
  }
  const f32x4 m = *reinterpret_cast<const f32x4*>(meta + 4 * n);
  z = m[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) P[mb][i] = Pp[mb][i] * m[0] + Pn[mb][i] * m[1];
}

// The lane's 8 key elements of one k-block in registers (row n, k = 32 kb + 8 q ..)
template <class DT> struct KOp;
template <> struct KOp<BF16> {
  u32x4 w;
  __device__ __forceinline__ void load(const uint16_t* p) { w = ld16(p); }
  // y if c else x, register by register (no indexed copy)
  __device__ static __forceinline__ KOp pick(bool c, const KOp& x, const KOp& y) {
    KOp r;
#pragma unroll
    for (int j = 0; j < 4; ++j) r.w[j] = c ? y.w[j] : x.w[j];
    return r;
  }
  // the operand: these registers if use, else the 8 elements at p (LDS)
  __device__ __forceinline__ void op(bool use, const uint16_t* p, u32x4& hi, u32x4& lo) const {
    const u32x4 x = ld16(p);
#pragma unroll
    for (int j = 0; j < 4; ++j) hi[j] = use ? w[j] : x[j];
    lo = u32x4{0, 0, 0, 0};
  }
};
template <> struct KOp<F32> {
  f32x4 a, b;
  __device__ static __forceinline__ KOp pick(bool c, const KOp& x, const KOp& y) {
    KOp r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      r.a[j] = c ? y.a[j] : x.a[j];
      r.b[j] = c ? y.b[j] : x.b[j];
    }
    return r;
  }
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const f32x4*>(p);
    b = *reinterpret_cast<const f32x4*>(p + 4);
  }
  __device__ __forceinline__ void op(bool use, const float* p, u32x4& hi, u32x4& lo) const {
    float x[8];
    load8_f32(p, x);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[j] = use ? a[j] : x[j];
      x[4 + j] = use ? b[j] : x[4 + j];
    }
    splitop<F32>(x, hi, lo);
  }
};

// 16 bytes of input elements as floats
__device__ __forceinline__ void cvt_piece(const BF16&, u32x4 w, float* o) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    o[2 * e] = __uint_as_float(w[e] << 16);
    o[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void cvt_piece(const F32&, u32x4 w, float* o) {
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = __uint_as_float(w[e]);
}

// four consecutive values of a V row (the SRE operand of one lane and block)
template <class DT> struct VQuad;
template <> struct VQuad<BF16> {
  u32x2 w;
  __device__ __forceinline__ void load(const uint16_t* p) { w = *reinterpret_cast<const u32x2*>(p); }
  __device__ __forceinline__ float get(int i) const {
    const uint32_t x = w[i >> 1];
    return __uint_as_float((i & 1) ? (x & 0xFFFF0000u) : (x << 16));
  }
};
template <> struct VQuad<F32> {
  f32x4 w;
  __device__ __forceinline__ void load(const float* p) { w = *reinterpret_cast<const f32x4*>(p); }
  __device__ __forceinline__ float get(int i) const { return w[i]; }
};

// CPL consecutive elements of a V row (the lane's P V columns) in registers
template <class DT, int CPL> struct VCols;
template <> struct VCols<BF16, 2> {
  using W = uint32_t;
  __device__ static __forceinline__ W load(const uint16_t* p) { return *reinterpret_cast<const uint32_t*>(p); }
  __device__ static __forceinline__ void cvt(W w, float* o) {
    o[0] = __uint_as_float(w << 16);
    o[1] = __uint_as_float(w & 0xFFFF0000u);
  }
};
template <> struct VCols<BF16, 1> {
  using W = uint32_t;
  __device__ static __forceinline__ W load(const uint16_t* p) { return *p; }
  __device__ static __forceinline__ void cvt(W w, float* o) { o[0] = __uint_as_float(w << 16); }
};
template <> struct VCols<F32, 2> {
  using W = u32x2;
  __device__ static __forceinline__ W load(const float* p) { return *reinterpret_cast<const u32x2*>(p); }
  __device__ static __forceinline__ void cvt(W w, float* o) {
    o[0] = __uint_as_float(w[0]);
    o[1] = __uint_as_float(w[1]);
  }
};
template <> struct VCols<F32, 1> {
  using W = uint32_t;
  __device__ static __forceinline__ W load(const float* p) { return __float_as_uint(*p); }
  __device__ static __forceinline__ void cvt(W w, float* o) { o[0] = __uint_as_float(w); }
};

}  // namespace

// Keys per chunk (kKC = 128); kc = 0 when the layout exceeds the LDS of a CU.
// Two workgroups share a CU whenever the layout fits 80 KB.
void decode_plan(int lam, int eta, int d, int g, bool f32, int* kc_out) {
  (void)g;
  *kc_out = dec_layout(lam, eta, d, f32 ? 4 : 2).total <= kLdsOne ? kKC : 0;
}

size_t decode_lds_bytes(int lam, int eta, int d, int g, bool f32) {
  (void)g;
  return dec_layout(lam, eta, d, f32 ? 4 : 2).total;
}

// MULTI: more than one key chunk (lam + eta > 128); the one-chunk instance
// has no chunk loop at all.
template <class DT, int HD, bool MULTI>
__global__ __launch_bounds__(kThreads, DT::kSplit ? 1 : 2) void decode_kernel(DecodeArgs a) {
  using T = typename DT::T;
  constexpr int NS = HD / 32;                // column slabs of H (one per wave)
  constexpr int KB = HD / 32;                // 32-wide k-blocks of a d-long contraction
  constexpr int PER = 16 / (int)sizeof(T);   // elements per 16-byte piece
  constexpr int PPR = HD / PER;              // pieces per row
  constexpr int RS = HD + WP;                // LDS row stride (elements)
  constexpr int CPL = HD / 64;               // P V columns per lane
  constexpr int WPT = kM * PPR / kThreads;   // W^T pieces per thread
  constexpr int MISC = 8 * PPR + kD / 4;     // queries (4 rows), leaving and new pair, s
  constexpr int MPT = (MISC + kThreads - 1) / kThreads;
  constexpr int NVS = 5;                     // phi tiles whose SRE values are loaded up front
  const DT dt{};
  const int u = blockIdx.x, lam = a.lam, eta = a.eta, g = a.g;
  // (the wave index is uniform: scalar registers and scalar address math)
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15, q4 = lane >> 4;       // 16 x 16 MFMA layout: row / column, K group
  const int kg = lane / PPR, cp = lane % PPR;      // a lane's piece of a row: row group, piece
  const int kvh = u % a.Hkv;
  const long long n = a.npos ? a.npos[u / a.Hkv] : a.n;   // this sequence's position
  const bool up = a.phase != 2, rd = a.phase != 1; // update the state / write the outputs
  if (a.npos_next && threadIdx.x == 0 && u % a.Hkv == 0) a.npos_next[u / a.Hkv] = n + 1;
  const int gs = (int)min((long long)lam, max(0LL, n - eta));
  const bool has_leave = up && n >= eta;           // eta == 0: the new pair leaves at once
  const bool full = has_leave && gs + 1 > lam;     // score and fold
  const int ncand = full ? gs + 1 : 0;             // candidate rows = keys 0..gs
  const int w_len = (int)min((long long)eta, n);   // window positions n - w_len .. n - 1
  const int nko = gs + w_len;                      // cache and window keys; the new pair is key nko
  const int ring0 = eta > 0 ? (int)((n - w_len) % eta) : 0;   // ring slot of the oldest window row
  const int ringn = eta > 0 ? (int)(n % eta) : 0;             // ring slot of position n (and n - eta)
  const bool has_slab = wave < NS;
  const int nch = MULTI ? max(1, (nko + kKC - 1) / kKC) : 1;  // key chunks (at least one)

  extern __shared__ __align__(16) unsigned char smem[];
  const DecLayout L = dec_layout(lam, eta, HD, (int)sizeof(T));
  T* sm_wt = (T*)(smem + L.wt);
  T* sm_q = (T*)(smem + L.q);
  T* sm_lk = (T*)(smem + L.lk);
  T* sm_lv = (T*)(smem + L.lv);
  T* sm_nk = (T*)(smem + L.nk);
  T* sm_nv = (T*)(smem + L.nv);
  float* sm_ve = (float*)(smem + L.ve);
  float* sm_s = (float*)(smem + L.s);
  int32_t* sm_cpos = (int32_t*)(smem + L.cpos);
  float* sm_spart = (float*)(smem + L.spart);
  float* sm_logit = (float*)(smem + L.logit);
  float* sm_nlin = (float*)(smem + L.nlin);
  float* sm_pv = (float*)(smem + L.pv);
  float* sm_phe = (float*)(smem + L.phe);
  float* sm_wst = (float*)(smem + L.wst);
  float* sm_zq = (float*)(smem + L.zq);
  int32_t* sm_red = (int32_t*)(smem + L.red);
  u32x4* sm_slot = (u32x4*)(smem + L.slot);
  float* sm_meta = (float*)(smem + L.meta);
  float* sm_pend = (float*)(smem + L.pend);

  const T* qg = reinterpret_cast<const T*>(a.q) + (size_t)u * a.q_su;
  const T* kin = reinterpret_cast<const T*>(a.k) + (size_t)u * a.kv_su;
  const T* vin = reinterpret_cast<const T*>(a.v) + (size_t)u * a.kv_su;
  T* ringk = reinterpret_cast<T*>(a.ring_k) + (size_t)u * eta * HD;
  T* ringv = reinterpret_cast<T*>(a.ring_v) + (size_t)u * eta * HD;
  T* ck = reinterpret_cast<T*>(a.cache_k) + (size_t)u * lam * HD;
  T* cv = reinterpret_cast<T*>(a.cache_v) + (size_t)u * lam * HD;
  const T* WT = reinterpret_cast<const T*>(a.WT) + (size_t)kvh * kM * HD;
  const float* sg = a.s + (size_t)u * kD;
  float* HT = a.H + (size_t)u * kD * HD;          // H^T [HD][kD] of this unit
  // the leaving pair (position n - eta): ring slot n % eta, or the new pair
  const T* leave_k = eta > 0 ? ringk + (size_t)ringn * HD : kin;
  const T* leave_v = eta > 0 ? ringv + (size_t)ringn * HD : vin;
  // global row of key kk (kk == nko: the new pair)
  auto key_row = [&](int kk, bool val) -> const T* {
    if (kk < gs) return (val ? cv : ck) + (size_t)kk * HD;
    if (kk < nko) {
      int slot = ring0 + (kk - gs);
      if (slot >= eta) slot -= eta;
      return (val ? ringv : ringk) + (size_t)slot * HD;
    }
    return val ? vin : kin;
  };
  // The wave's keys of chunk k0 (two 16-key blocks: keys k0 + kkey(kt, n16),
  // clamped to the chunk) as MFMA operands, and their V rows for P V: lane l
  // takes the columns CPL l .. of every key (the weights of absent keys are 0).
  // Block kt of wave w is the chunk's keys 16 (4 kt + w) .. + 15, so that each
  // wave holds one of the first four 16-row phi tiles (the cache rows).
  auto kkey = [&](int kt, int r) { return 16 * (kWaves * kt + wave) + r; };
  KOp<DT> Kr[2][KB];
  typename VCols<DT, CPL>::W Vpv[32];
  auto load_keys = [&](int k0, int kn, int ln) {
    if (16 * wave < kn) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const T* kr = key_row(k0 + min(kkey(kt, ln & 15), kn - 1), false) + 8 * (ln >> 4);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) Kr[kt][kb].load(kr + 32 * kb);
      }
    }
  };
  auto load_vals = [&](int k0, int kn, int ln) {
    if (16 * wave < kn) {
      // lane j (< 32) finds the V row of the wave's key j once; load j takes that
      // address from lane j (a scalar base plus the lane's column offset)
      // (as a byte offset from the cache's V rows, so that the loads stay
      // global-memory loads)
      const char* vb = reinterpret_cast<const char*>(cv);
      const uint64_t ra = reinterpret_cast<uintptr_t>(key_row(k0 + min(kkey((ln >> 4) & 1, ln & 15), kn - 1), true)) -
                          reinterpret_cast<uintptr_t>(vb);
      const uint32_t rlo = (uint32_t)ra, rhi = (uint32_t)(ra >> 32);
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const uint64_t rj = ((uint64_t)__builtin_amdgcn_readlane(rhi, j) << 32) | __builtin_amdgcn_readlane(rlo, j);
        Vpv[j] = VCols<DT, CPL>::load(reinterpret_cast<const T*>(vb + rj) + CPL * ln);
      }
    }
  };
  // V values of candidate row row0 + rr at the lane's SRE columns
  // 32 wave + 16 mb + 4 q4 + (0..3)
  auto load_vs = [&](VQuad<DT> (&v)[2], int row0, int rr) {
    const T* p = key_row(min(row0 + rr, ncand - 1), true) + 32 * wave + 4 * q4;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) v[mb].load(p + 16 * mb);
  };
  // the small pieces: queries, leaving pair, new pair, s
  auto misc_src = [&](int i) -> const u32x4* {
    if (i < 4 * PPR) return i / PPR < g ? reinterpret_cast<const u32x4*>(qg + (size_t)(i / PPR) * a.q_sh + (i % PPR) * PER) : nullptr;
    if (i < 6 * PPR) return has_leave ? reinterpret_cast<const u32x4*>((i < 5 * PPR ? leave_k : leave_v) + (i % PPR) * PER) : nullptr;
    if (i < 8 * PPR) return reinterpret_cast<const u32x4*>((i < 7 * PPR ? kin : vin) + (i % PPR) * PER);
    if (i < MISC) return reinterpret_cast<const u32x4*>(sg + 4 * (i - 8 * PPR));
    return nullptr;
  };
  auto misc_dst = [&](int i) -> u32x4* {
    if (i < 4 * PPR) return reinterpret_cast<u32x4*>(sm_q + (i / PPR) * RS + (i % PPR) * PER);
    if (i < 6 * PPR) return reinterpret_cast<u32x4*>((i < 5 * PPR ? sm_lk : sm_lv) + (i % PPR) * PER);
    if (i < 8 * PPR) return reinterpret_cast<u32x4*>((i < 7 * PPR ? sm_nk : sm_nv) + (i % PPR) * PER);
    return reinterpret_cast<u32x4*>(sm_s + 4 * (i - 8 * PPR));
  };

  // ---- first wave of reads: the wave's keys, W^T and the small pieces (to
  // LDS), the first kThreads cache positions (no load here waits for another)
  const int kn0 = min(kKC, nko);
  load_keys(0, kn0, lane);
  u32x4 wbuf[WPT], mbuf[MPT];
#pragma unroll
  for (int j = 0; j < WPT; ++j) {
    const int i = j * kThreads + tid;
    wbuf[j] = *reinterpret_cast<const u32x4*>(WT + (size_t)(i / PPR) * HD + (i % PPR) * PER);
  }
#pragma unroll
  for (int j = 0; j < MPT; ++j) {
    const u32x4* p = misc_src(j * kThreads + tid);
    if (p) mbuf[j] = *p;
  }
  int32_t cpos0 = 0;
  if (tid < gs) cpos0 = a.cache_pos[(size_t)u * lam + tid];
  // the unit's held-back fold terms (phi, v: PQ 16-byte pieces each)
  constexpr int PQ = (kD + HD) / 4;
  static_assert(kPend * PQ <= kThreads, "one piece of the held-back terms per thread");
  // (the chunked instance writes every fold at once and never holds one back)
  const int np = !MULTI && a.npend ? max(0, min((int)a.npend[u], kPend)) : 0;
  u32x4 pbuf = u32x4{0, 0, 0, 0};
  if (tid < np * PQ)
    pbuf = *reinterpret_cast<const u32x4*>(a.pend + (size_t)u * kPend * (kD + HD) + 4 * tid);
#pragma unroll
  for (int j = 0; j < WPT; ++j) {
    const int i = j * kThreads + tid;
    *reinterpret_cast<u32x4*>(sm_wt + (i / PPR) * RS + (i % PPR) * PER) = wbuf[j];
  }
#pragma unroll
  for (int j = 0; j < MPT; ++j) {
    const int i = j * kThreads + tid;
    if (misc_src(i)) *misc_dst(i) = mbuf[j];
  }
  if (tid < gs) sm_cpos[tid] = cpos0;
  if (tid < np * PQ) *reinterpret_cast<u32x4*>(sm_pend + 4 * tid) = pbuf;
  for (int i = tid + kThreads; i < gs; i += kThreads) sm_cpos[i] = a.cache_pos[(size_t)u * lam + i];
  __syncthreads();
  // The last phi tile of a one-chunk step holds at most one key row, the
  // leaving pair's, which LDS holds too; its other rows are the new pair and
  // the queries.  Its wave computes it here, from LDS, before issuing its
  // second wave of reads, so that no wave has more than one tile in the phi
  // phase (four tiles of cache rows and this one in the decode shapes).
  int early = -1;
  if constexpr (!MULTI) {
    const int cno = max(0, min(kn0, ncand));        // as in the chunk loop (one chunk)
    const int cn = cno + (ncand > nko ? 1 : 0);
    const int t = (cn + g + 15) / 16 - 1;
    // (cno <= gs + 1: the tile's only key row is gs, the leaving pair)
    if (t >= 0 && 16 * t >= min(cno, gs)) early = t;
    if (early >= 0 && (early & (kWaves - 1)) == wave) {
      const int row = 16 * early + n16;
      const T* xr = row < cno ? sm_lk : row < cn ? sm_nk : sm_q + min(max(row - cn, 0), g - 1) * RS;
      f32x4 U[4];
      pre16<DT, HD>([&](int kb, u32x4& hi, u32x4& lo) { xop(dt, xr + 32 * kb + 8 * q4, hi, lo); },
                    sm_wt, n16, q4, U);
      phi_to_slot<DT>(U, sm_s, lane, n16, q4, sm_slot + early * (8 * 64), sm_meta + early * 64);
    }
  }
  // ---- second wave, issued once every wave's first-wave LDS data has
  // arrived: the values of the wave's keys, the SRE values of the first phi
  // tiles, the H slab (lane (n16, q4) holds H[sigma(kb, q4, j)][32 wave +
  // 16 mb + n16]: two 16-byte pieces of an H^T row per block).  Logits and
  // phi run while these stream in.
  __builtin_amdgcn_sched_barrier(0);
  load_vals(0, kn0, lane);
  VQuad<DT> vs[NVS][2];
#pragma unroll
  for (int t = 0; t < NVS; ++t)
    if (has_slab && 16 * t < ncand) load_vs(vs[t], 16 * t, n16);
  f32x4 Hraw[2][4][2];
  if (has_slab) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const float* hrow = HT + (size_t)(32 * wave + 16 * mb + n16) * kD + 4 * q4;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        Hraw[mb][kb][0] = *reinterpret_cast<const f32x4*>(hrow + 32 * kb);
        Hraw[mb][kb][1] = *reinterpret_cast<const f32x4*>(hrow + 32 * kb + 16);
      }
    }
  }

  const float scale2 = kL2E / sqrtf((float)HD);   // logits in the log2 domain
  // the wave's running max and sum per head (the same in every lane); its
  // P V partials live in sm_pv[wave], rescaled when the max moves
  float mrun[4], lrun[4];
#pragma unroll
  for (int hd = 0; hd < 4; ++hd) { mrun[hd] = -INFINITY; lrun[hd] = 0.f; }
  HSlab<DT, !MULTI> Hs;

  // ---- key chunks (one for the decode shapes here)
  for (int c = 0; c < nch; ++c) {
    const int k0 = c * kKC;
    const int kn = max(0, min(kKC, nko - k0));
    const bool last = c == nch - 1;
    if (MULTI && c > 0) {
      __syncthreads();                             // the previous chunk's phi tiles are consumed
      // (the lane index made opaque here: the addresses of a later chunk's
      // reads are not hoisted out of the chunk loop, where they would stay
      // live through the whole kernel)
      int t = lane;
      __asm__ volatile("" : "+v"(t));
      load_keys(k0, kn, t);
      load_vals(k0, kn, t);
#pragma unroll
      for (int tt = 0; tt < NVS; ++tt)
        if (has_slab && k0 + 16 * tt < ncand) load_vs(vs[tt], k0 + 16 * tt, t & 15);
    }
    float alpha[4] = {1.f, 1.f, 1.f, 1.f};         // rescale of the earlier chunks' partials
    {
      // logits of the wave's keys: S^T = K Q^T in two 16-key blocks, lane
      // (n16, q4) = query n16, keys kkey(kt, 4 q4 + i); softmax weights with
      // the running max
      if (16 * wave < kn) {
        // (queries past g read a valid row; never read back)
        const T* qrow = sm_q + min(n16, g - 1) * RS + 8 * q4;
        f32x4 St[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) St[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          u32x4 qh, ql;
          xop(dt, qrow + 32 * kb, qh, ql);
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) {
            u32x4 kh, kl;
            Kr[kt][kb].op(true, qrow, kh, kl);
            St[kt] = mma16x<DT>(kh, kl, qh, ql, St[kt]);
          }
        }
        float S[2][4], mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int j = kkey(kt, 4 * q4 + i);
            const bool vis = j < kn && (k0 + j >= gs || (a.branches & LOLA_READ_CACHE));   // cache keys unless hidden
            S[kt][i] = vis ? St[kt][i] * scale2 : -INFINITY;
            mx = fmaxf(mx, S[kt][i]);
          }
        mx = qmax(mx);
        // (a maximum still at -inf means no visible key so far in this wave,
        // e.g. cache keys hidden from the read: nothing to rescale, and the
        // weights exp2(-inf - 0) are 0)
#pragma unroll
        for (int hd = 0; hd < 4; ++hd) {
          const float mn = fmaxf(mrun[hd], __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mx), hd)));
          alpha[hd] = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(mrun[hd] - mn);
          mrun[hd] = mn;
        }
        const float mr0 = n16 == 0 ? mrun[0] : (n16 == 1 ? mrun[1] : (n16 == 2 ? mrun[2] : mrun[3]));
        const float mr = mr0 == -INFINITY ? 0.f : mr0;
        float ls = 0.f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p = __builtin_amdgcn_exp2f(S[kt][i] - mr);
            ls += p;
            if (n16 < 4) sm_logit[4 * kkey(kt, 4 * q4 + i) + n16] = n16 < g ? p : 0.f;
          }
        ls = qsum(ls);
#pragma unroll
        for (int hd = 0; hd < 4; ++hd)
          lrun[hd] = fmaf(lrun[hd], alpha[hd], __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ls), hd)));
      }
    }

    // phi rows of the chunk: its candidate keys (cno), the new pair when it is
    // a candidate (eta = 0), then (last chunk) the queries.  Tile t (rows
    // 16 t ..) is computed by wave t % 4, whose key block t / 4 holds its key
    // rows (tiles past the keys: rows from LDS).
    const int cno = max(0, min(kn, ncand - k0));
    const int cn = cno + (last && ncand > nko ? 1 : 0);
    const int nr = cn + (last ? g : 0);
    const int nt = (nr + 15) / 16;
    for (int t = 0; t < nt; ++t) {
      if ((t & (kWaves - 1)) != wave || t == early) continue;
      const int row = 16 * t + n16;
      // rows past the keys: the new pair, a query, else a copy of a query (never read back)
      const T* xr = row < cn ? sm_nk : sm_q + min(max(row - cn, 0), g - 1) * RS;
      const bool use = row < cno;
      const bool odd = ((t / kWaves) & 1) != 0;    // key block t / 4 (selected, not indexed)
      f32x4 U[4];
      pre16<DT, HD>([&](int kb, u32x4& hi, u32x4& lo) {
                      const KOp<DT> kr = KOp<DT>::pick(odd, Kr[0][kb], Kr[1][kb]);
                      kr.op(use, xr + 32 * kb + 8 * q4, hi, lo);
                    },
                    sm_wt, n16, q4, U);
      phi_to_slot<DT>(U, sm_s, lane, n16, q4, sm_slot + t * (8 * 64), sm_meta + t * 64);
    }
    // P V of the wave's keys (their values arrive while the logits and phi
    // tiles run), the new pair, into the wave's partials
    {
      float acc[4][CPL];
#pragma unroll
      for (int hd = 0; hd < 4; ++hd)
#pragma unroll
        for (int e = 0; e < CPL; ++e) acc[hd][e] = 0.f;
      if (16 * wave < kn) {
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");   // weights written above
        // lane l over the 32 keys, its CPL columns, four heads
#pragma unroll
        for (int j = 0; j < 32; ++j) {
          const f32x4 p4 = *reinterpret_cast<const f32x4*>(sm_logit + 4 * kkey(j >> 4, j & 15));
          float v[CPL];
          VCols<DT, CPL>::cvt(Vpv[j], v);
#pragma unroll
          for (int hd = 0; hd < 4; ++hd)
#pragma unroll
            for (int e = 0; e < CPL; ++e) acc[hd][e] = fmaf(p4[hd], v[e], acc[hd][e]);
        }
      }
      if (up && last && wave == kWaves - 1) {
        // the new pair (key nko): logits q . k on the VALU, lane (kg, cp) a
        // piece of head hd0 + kg (RG row groups of PPR lanes)
        constexpr int RG = 64 / PPR;
        float snew[4];
#pragma unroll
        for (int hd0 = 0; hd0 < 4; hd0 += RG) {
          const int hd = hd0 + kg;
          float part = 0.f;
          if (hd < g) {
            float qv[PER], kv[PER];
            cvt_piece(dt, *reinterpret_cast<const u32x4*>(sm_q + hd * RS + cp * PER), qv);
            cvt_piece(dt, *reinterpret_cast<const u32x4*>(sm_nk + cp * PER), kv);
#pragma unroll
            for (int e = 0; e < PER; ++e) part = fmaf(qv[e], kv[e], part);
          }
#pragma unroll
          for (int o = 1; o < PPR; o <<= 1) part += __shfl_xor(part, o, 64);
#pragma unroll
          for (int hh = 0; hh < RG; ++hh)
            if (hd0 + hh < 4)
              snew[hd0 + hh] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(part), hh * PPR)) * scale2;
        }
        float v[CPL];
#pragma unroll
        for (int e = 0; e < CPL; ++e) v[e] = DT::to_f32(sm_nv[CPL * lane + e]);
#pragma unroll
        for (int hd = 0; hd < 4; ++hd) {
          const float mn = fmaxf(mrun[hd], snew[hd]);      // finite: the new pair is visible
          const float al = __builtin_amdgcn_exp2f(mrun[hd] - mn);
          const float p = __builtin_amdgcn_exp2f(snew[hd] - mn);
          lrun[hd] = fmaf(lrun[hd], al, p);
          mrun[hd] = mn;
          alpha[hd] *= al;
#pragma unroll
          for (int e = 0; e < CPL; ++e) acc[hd][e] = fmaf(acc[hd][e], al, p * v[e]);
        }
      }
      // into the wave's partials, rescaling the earlier chunks'
#pragma unroll
      for (int hd = 0; hd < 4; ++hd) {
        float* dst = sm_pv + (wave * 4 + hd) * HD + CPL * lane;
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
          float x = acc[hd][e];
          if (MULTI && c > 0) x = fmaf(dst[e], alpha[hd], x);
          dst[e] = x;
        }
      }
      if (last) {
#pragma unroll
        for (int hd = 0; hd < 4; ++hd)
          if (lane == hd) {
            sm_wst[wave * 8 + hd] = mrun[hd];
            sm_wst[wave * 8 + 4 + hd] = lrun[hd];
          }
      }
    }

    __syncthreads();                               // phi tiles

    // per slab wave: its columns of the SRE parts and of H^T phi(q)
    if (has_slab) {
      if (c == 0) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            float x[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) { x[j] = Hraw[mb][kb][0][j]; x[4 + j] = Hraw[mb][kb][1][j]; }
            // the held-back folds, oldest first: the fma of the step that
            // made each term (so H is bitwise the one written at once)
            for (int k = 0; k < np; ++k) {
              const float* pk = sm_pend + k * (kD + HD);
              const f32x4 f0 = *reinterpret_cast<const f32x4*>(pk + 32 * kb + 4 * q4);
              const f32x4 f1 = *reinterpret_cast<const f32x4*>(pk + 32 * kb + 16 + 4 * q4);
              const float vk = pk[kD + 32 * wave + 16 * mb + n16];
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                x[j] = fmaf(f0[j], vk, x[j]);
                x[4 + j] = fmaf(f1[j], vk, x[4 + j]);
              }
            }
            Hs.set(mb, kb, x);
          }
      }
      auto tile = [&](int t, const VQuad<DT> (&v)[2]) {
        const int row = 16 * t + n16;
        f32x4 P[2];
        float z;
        slab_prod<DT>(sm_slot + t * (8 * 64), sm_meta + t * 64, Hs, lane, n16, P, z);
        if (row < cn) {
          const float iz = z > 0.f ? 1.f / z : 0.f;
          float part = 0.f;
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float e = fmaf(P[mb][i], iz, -v[mb].get(i));
              part = fmaf(e, e, part);
            }
          part = qsum(part);
          if (q4 == 0) sm_spart[wave * (lam + 1) + k0 + row] = part;
        } else if (row < nr) {
          const int hd = row - cn;
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
            *reinterpret_cast<f32x4*>(sm_nlin + hd * HD + 32 * wave + 16 * mb + 4 * q4) = P[mb];
          if (wave == 0 && q4 == 0) sm_zq[hd] = z;
        }
      };
#pragma unroll
      for (int t = 0; t < NVS; ++t)
        if (t < nt) tile(t, vs[t]);
      for (int t = NVS; t < nt; ++t) {
        VQuad<DT> v[2];
        if (16 * t < cn) load_vs(v, k0 + 16 * t, n16);
        tile(t, v);
      }
    }
  }
  __syncthreads();                                 // SRE parts, partials, linear read

  if (wave == 0) {
    if (full) {
      // ---- the candidate to fold: lowest SRE, ties to the newer position,
      // as the smallest 64-bit key (SRE bits, then the position complemented;
      // SRE >= 0, so its bits order as the values); the wave minimum by DPP
      // moves (lane 63), the winner's lane by a ballot
      uint64_t key = ~0ull;
      int bi = 0;
      for (int e = lane; e < ncand; e += 64) {
        float sre = 0.f;
#pragma unroll
        for (int w = 0; w < NS; ++w) sre += sm_spart[w * (lam + 1) + e];
        const int pos = e < gs ? sm_cpos[e] : (int)(n - eta);
        const uint64_t k = ((uint64_t)__float_as_uint(sre) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)pos);
        if (k < key) { key = k; bi = e; }
      }
      uint64_t m = key;
      {
        auto mn = [&](uint64_t y) { m = y < m ? y : m; };
        mn(dpp_u64<0x111, 0xf>(m, ~0ull));
        mn(dpp_u64<0x112, 0xf>(m, ~0ull));
        mn(dpp_u64<0x114, 0xf>(m, ~0ull));
        mn(dpp_u64<0x118, 0xf>(m, ~0ull));
        mn(dpp_u64<0x142, 0xa>(m, ~0ull));
        mn(dpp_u64<0x143, 0xc>(m, ~0ull));
      }
      const uint64_t mk = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(m >> 32), 63) << 32) |
                          (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)m, 63);
      bi = __builtin_amdgcn_readlane(bi, (int)__builtin_ctzll(__ballot(key == mk)));
      if (lane == 0) sm_red[0] = bi;
      const T* vrow = bi == gs ? sm_lv : cv + (size_t)bi * HD;
      for (int e = lane; e < HD; e += 64) sm_ve[e] = ldf(vrow + e);
      if constexpr (!MULTI) {
        // phi of the folded row from its tile (hi + lo, normalised)
        const int t = bi >> 4;
        if (n16 == (bi & 15)) {
          const u32x4* sl = sm_slot + t * (8 * 64);
          const f32x4 mt = *reinterpret_cast<const f32x4*>(sm_meta + t * 64 + 4 * n16);
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            const u32x4 bh = sl[(2 * kb) * 64 + lane], bl = sl[(2 * kb + 1) * 64 + lane];
            const float sc = kb < 2 ? mt[0] : mt[1];
            f32x4 o0, o1;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const uint32_t hw = (bh[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
              const uint32_t lw = (bl[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
              const float x = (DT::from_bits(hw) + DT::from_bits(lw)) * sc;
              if (j < 4) o0[j] = x; else o1[j - 4] = x;
            }
            *reinterpret_cast<f32x4*>(sm_phe + 32 * kb + 4 * q4) = o0;
            *reinterpret_cast<f32x4*>(sm_phe + 32 * kb + 16 + 4 * q4) = o1;
          }
        }
      } else {
        // (chunks of earlier keys are gone) phi of the folded row again, every
        // lane supplying the same row
        const T* xrow = bi == gs ? sm_lk : ck + (size_t)bi * HD;
        f32x4 U[4];
        pre16<DT, HD>([&](int kb, u32x4& hi, u32x4& lo) { xop(dt, xrow + 32 * kb + 8 * q4, hi, lo); },
                      sm_wt, n16, q4, U);
        float ph[2][4][4];
        phi16(U, ph);
        if (n16 == 0) {
#pragma unroll
          for (int half = 0; half < 2; ++half)
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
              *reinterpret_cast<f32x4*>(sm_phe + 64 * half + 16 * mt + 4 * q4) =
                  f32x4{ph[half][mt][0], ph[half][mt][1], ph[half][mt][2], ph[half][mt][3]};
        }
      }
    }
  } else {
    // ---- the outputs: the four waves' partials and the linear read (logit 0)
    for (int i = tid - 64; i < g * HD; i += kThreads - 64) {
      const int hd = i / HD, e = i % HD;
      // the linear read enters with logit 0 unless the state is hidden or
      // empty (z = 0); without it the maximum is the waves' alone, so that
      // the weights of very negative logits do not all underflow
      const bool lin = (a.branches & LOLA_READ_STATE) && sm_zq[hd] > 0.f;
      float m = lin ? 0.f : -INFINITY;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) m = fmaxf(m, sm_wst[w * 8 + hd]);
      const float em = lin ? __builtin_amdgcn_exp2f(-m) : 0.f;
      float num = em * sm_nlin[hd * HD + e], den = em * sm_zq[hd];
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = __builtin_amdgcn_exp2f(sm_wst[w * 8 + hd] - m);
        num = fmaf(f, sm_pv[(w * 4 + hd) * HD + e], num);
        den = fmaf(f, sm_wst[w * 8 + 4 + hd], den);
      }
      if (rd) a.out[(size_t)u * a.o_su + (size_t)hd * a.o_sh + e] = num / den;
    }
    // ---- the new pair enters the ring slot n % eta (every read of the ring is done)
    if (eta > 0 && up) {
      T* dk = ringk + (size_t)ringn * HD;
      T* dv = ringv + (size_t)ringn * HD;
      for (int i = tid - 64; i < 2 * PPR; i += kThreads - 64) {
        const int k = (i % PPR) * PER;
        if (i < PPR) *reinterpret_cast<u32x4*>(dk + k) = *reinterpret_cast<const u32x4*>(sm_nk + k);
        else *reinterpret_cast<u32x4*>(dv + k) = *reinterpret_cast<const u32x4*>(sm_nv + k);
      }
    }
  }
  __syncthreads();                                 // the folded row, its phi and value

  // ---- update: fold into the slab and s, cache slot
  const int fold_row = full ? sm_red[0] : -1;      // < gs: cache slot; == gs: the leaving pair
  if (fold_row >= 0) {
    // H is written every kPend + 1 positions (the same steps for every unit
    // of a uniform batch, so that the other steps write no H at all) or when the
    // held-back list is full; otherwise the step's term joins the list
    static_assert(((kPend + 1) & kPend) == 0, "the write period is a power of two");
    const bool wr = MULTI || !a.pend || np >= kPend || ((uint32_t)n & (uint32_t)kPend) == 0;
    if (!wr) {
      float* dst = a.pend + ((size_t)u * kPend + np) * (kD + HD);
      for (int i = tid; i < kD + HD; i += kThreads) dst[i] = i < kD ? sm_phe[i] : sm_ve[i - kD];
    }
    if (a.npend && tid == 0) a.npend[u] = wr ? 0 : np + 1;
    if (has_slab && wr) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const float ve = sm_ve[32 * wave + 16 * mb + n16];
        float* hrow = HT + (size_t)(32 * wave + 16 * mb + n16) * kD + 4 * q4;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const f32x4 p0 = *reinterpret_cast<const f32x4*>(sm_phe + 32 * kb + 4 * q4);
          const f32x4 p1 = *reinterpret_cast<const f32x4*>(sm_phe + 32 * kb + 16 + 4 * q4);
          float hv[8];
          Hs.get(mb, kb, hv);
          f32x4 x0, x1;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            x0[j] = fmaf(p0[j], ve, hv[j]);
            x1[j] = fmaf(p1[j], ve, hv[4 + j]);
          }
          *reinterpret_cast<f32x4*>(hrow + 32 * kb) = x0;
          *reinterpret_cast<f32x4*>(hrow + 32 * kb + 16) = x1;
        }
      }
    }
    for (int F = tid; F < kD; F += kThreads) a.s[(size_t)u * kD + F] = sm_s[F] + sm_phe[F];
  }
  if (has_leave) {
    const int slot_in = !full ? gs : (fold_row < gs ? fold_row : -1);
    if (slot_in >= 0) {
      for (int i = tid; i < 2 * PPR; i += kThreads) {
        const int k = (i % PPR) * PER;
        if (i < PPR) *reinterpret_cast<u32x4*>(ck + (size_t)slot_in * HD + k) = *reinterpret_cast<const u32x4*>(sm_lk + k);
        else *reinterpret_cast<u32x4*>(cv + (size_t)slot_in * HD + k) = *reinterpret_cast<const u32x4*>(sm_lv + k);
      }
      if (tid == 0) a.cache_pos[(size_t)u * lam + slot_in] = (int32_t)(n - eta);
    }
  }
}

// H += the held-back fold terms of each unit, npend = 0 (before anything
// other than the decode step reads or replaces H).  One workgroup per unit.
__global__ __launch_bounds__(256) void flush_pending_kernel(float* H, const float* pend,
                                                            int32_t* npend, int d) {
  const int u = blockIdx.x;
  const int np = max(0, min((int)npend[u], kPend));
  if (np == 0) return;
  const float* pu = pend + (size_t)u * kPend * (kD + d);
  float* Hu = H + (size_t)u * d * kD;                // H^T [d][kD]
  for (int e = threadIdx.x; e < d * kD; e += blockDim.x) {
    const int c = e / kD, F = e % kD;
    float x = Hu[e];
    for (int k = 0; k < np; ++k) x = fmaf(pu[k * (kD + d) + F], pu[k * (kD + d) + kD + c], x);
    Hu[e] = x;
  }
  __syncthreads();                                   // every thread has read npend[u]
  if (threadIdx.x == 0) npend[u] = 0;
}

hipError_t launch_flush_pending(float* H, const float* pend, int32_t* npend, int U, int d,
                                hipStream_t st) {
  if (U <= 0) return hipSuccess;
  hipLaunchKernelGGL(flush_pending_kernel, dim3(U), dim3(256), 0, st, H, pend, npend, d);
  return hipGetLastError();
}

// W [Hkv, d, kM] -> W^T [Hkv, kM, d] (once, at state creation)
template <class T>
__global__ void transpose_w_kernel(const T* W, T* WT, int d, int total) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int hk = i / (kM * d), rem = i % (kM * d);
  const int f = rem / d, k = rem % d;
  WT[i] = W[(size_t)hk * d * kM + (size_t)k * kM + f];
}

hipError_t launch_transpose_w(const void* W, void* WT, int Hkv, int d, bool f32, hipStream_t st) {
  const int total = Hkv * kM * d;
  const int blocks = (total + 255) / 256;
  if (f32)
    hipLaunchKernelGGL(transpose_w_kernel<float>, dim3(blocks), dim3(256), 0, st,
                       (const float*)W, (float*)WT, d, total);
  else
    hipLaunchKernelGGL(transpose_w_kernel<uint16_t>, dim3(blocks), dim3(256), 0, st,
                       (const uint16_t*)W, (uint16_t*)WT, d, total);
  return hipGetLastError();
}

template <class DT, int HD>
static hipError_t launch_decode_t(const DecodeArgs& a, int U, hipStream_t st) {
  if (a.kc != kKC || a.g < 1 || a.g > 4) return hipErrorInvalidValue;
  const size_t lds = dec_layout(a.lam, a.eta, HD, (int)sizeof(typename DT::T)).total;
  if (lds > kLdsOne) return hipErrorInvalidValue;
  const bool multi = a.lam + a.eta > kKC;
  const void* fn = multi ? (const void*)decode_kernel<DT, HD, true> : (const void*)decode_kernel<DT, HD, false>;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  if (multi)
    hipLaunchKernelGGL((decode_kernel<DT, HD, true>), dim3(U), dim3(kThreads), lds, st, a);
  else
    hipLaunchKernelGGL((decode_kernel<DT, HD, false>), dim3(U), dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int U, bool f32, hipStream_t st) {
  if (U <= 0) return hipSuccess;
  if (a.d == 128) return f32 ? launch_decode_t<F32, 128>(a, U, st) : launch_decode_t<BF16, 128>(a, U, st);
  return f32 ? launch_decode_t<F32, 64>(a, U, st) : launch_decode_t<BF16, 64>(a, U, st);
}

}  // namespace lola
