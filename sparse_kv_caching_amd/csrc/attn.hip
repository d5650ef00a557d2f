// K3: the read of every chunk, LoLA notes §2.5, Eq. (14):
//
//   y_t = (H_j^T phi(q_t) + sum_{i in V(t)} a_ti v_i)
//         / (phi(q_t)^T s_j + sum_{i in V(t)} a_ti),   a_ti = exp(q_t.k_i / sqrt(d)),
//
// V(t) = G_j (cache at chunk start) plus the local positions
// max(0, n_j - eta) .. t (window and the causal prefix of the chunk).  All
// chunks run in parallel: they only need the per-chunk snapshots (H_j, s_j,
// G_j) written by the chain kernel.
//
// One workgroup = one unit, one chunk, one tile of up to 256 / g positions,
// and 8 waves; wave = one q-head x 32 positions, so the GQA heads of a unit
// share every staged K/V tile.  Keys are staged 64 at a time, double-buffered:
// the global loads of tile t + 1 are in flight while tile t is multiplied,
// and one barrier per tile separates the buffers.  Scores are computed
// transposed, S^T = K Q^T (32 keys x 32 queries per MFMA), so each lane owns
// one query and softmax statistics need a single cross-half exchange; P then
// feeds O^T += V^T P^T straight from registers (the K index of that MFMA is
// permuted to match the result layout, see common.h), with V staged
// transposed (key pairs packed per dword).
//
// Exponentials are unshifted in Eq. (14); here they are shifted by a running
// maximum m >= 0 (log2 domain) and the linear terms are scaled by the same
// 2^{-m}:  y = (2^-m N_lin + sum 2^{x-m} v) / (2^-m z_lin + sum 2^{x-m}),
// which is the same quantity.  The linear read is done first with m = 0.
//
// Precision: q.k is exact-product bf16 MFMA with fp32 accumulation; P and V
// go through fp16 MFMA (11-bit significand, P in [0, 1]); the linear read
// uses the hi/lo bf16 split on both phi(q) and H.  fp32 inputs split every
// operand into hi/lo fp16 (three passes, ~2^-22 per product).
#include "internal.h"

namespace lola {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int KT = 64;        // keys per staged tile
constexpr float kSlack = 8.f; // log2 headroom of the softmax weights over the running maximum
constexpr int HTS = kD + 4;   // LDS row of H^T (16-bit elements): 66 dwords, so that the 32
                              // rows of a 64-bit operand read fall on distinct bank pairs
constexpr int VTS = KT + 4;   // LDS row of the V^T tile (keys): 34 dwords, so that the 32 rows of a
                              // 64-bit operand read fall on distinct bank pairs

// Byte offsets of the LDS arrays; the key phase reuses the region of the
// linear-read phase.
struct AttnLayout {
  uint32_t G;                                  // both phases
  uint32_t WT, HT_hi, HT_lo, s;                // linear-read phase
  uint32_t K[2], KL[2], VT[2], VTL[2];         // key phase, two buffers
  uint32_t total;
};

inline __host__ __device__ uint32_t al16(uint32_t x) { return (x + 15u) & ~15u; }

// max / sum of a lane's value and the value 32 lanes away, in every lane, on
// the VALU: v_permlane32_swap of x with itself gives r0 = x[l % 32] and
// r1 = x[l % 32 + 32] in lane l (the same two operands, in the same order,
// in both halves)
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__host__ __device__ inline AttnLayout attn_layout(int d, int lam, bool f32) {
  AttnLayout L;
  uint32_t off = 0;
  auto take = [&](uint32_t b) { const uint32_t o = off; off = al16(off + b); return o; };
  const uint32_t esz = f32 ? 4 : 2;
  L.G = take((uint32_t)(lam > 0 ? lam : 1) * 4);      // cache at chunk start (virtual indices)
  const uint32_t base = off;
  L.WT = take((uint32_t)kM * (d + 8) * esz);          // [kM][d + 8] W^T, input dtype
  L.HT_hi = take((uint32_t)d * HTS * 2);               // [d][HTS]
  L.HT_lo = take((uint32_t)d * HTS * 2);
  L.s = take(kD * 4);
  const uint32_t phaseA = off;
  off = base;
  for (int b = 0; b < 2; ++b) {
    L.K[b] = take((uint32_t)KT * (d + 8) * 2);         // [KT][d + 8] bf16 (fp32 inputs: fp16 hi)
    L.KL[b] = take(f32 ? (uint32_t)KT * (d + 8) * 2 : 16);   //                  fp16 lo
    L.VT[b] = take((uint32_t)d * VTS * 2);             // [d][VTS] fp16 (fp32 inputs: hi)
    L.VTL[b] = take(f32 ? (uint32_t)d * VTS * 2 : 16); //                       lo
  }
  L.total = phaseA > off ? phaseA : off;
  return L;
}

__device__ __forceinline__ u32x2 ld8(const uint16_t* p) { return *reinterpret_cast<const u32x2*>(p); }

// operand with K-slots sigma_h: elements [4h, 4h+4) and [8+4h, 8+4h+4) of a 16-block
__device__ __forceinline__ u32x4 sigma_load(const uint16_t* row16, int h) {
  u32x2 a = ld8(row16 + 4 * h), b = ld8(row16 + 8 + 4 * h);
  return u32x4{a[0], a[1], b[0], b[1]};
}

// First V column (of 8) of thread tid's item in the V^T staging: the two
// half-waves take column groups 2 apart (V^T rows 16 apart, 544 dwords:
// 32 banks apart), so that their 4-byte writes to one key-pair column fall on
// all 64 banks
__device__ __forceinline__ int vt_cols(int tid) {
  const int w = tid >> 6, hh = (tid >> 5) & 1;
  return 8 * (4 * (w >> 1) + (w & 1) + 2 * hh);
}

__device__ __forceinline__ uint32_t f16_bits(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
}

}  // namespace

size_t attn_lds_bytes(int d, int lam, bool f32) { return attn_layout(d, lam, f32).total; }

template <class DT, int HD>
__global__ __launch_bounds__(kThreads) void attn_kernel(AttnArgs a) {
  using T = typename DT::T;
  constexpr int KB = HD / 16;     // 16-wide K blocks over the head dim
  constexpr int NMT = HD / 32;    // 32-row tiles of the output
  constexpr int KRS = HD + 8;     // LDS row of a staged key (elements)
  constexpr int PER = 16 / (int)sizeof(T);       // input elements per 16-byte piece
  constexpr int KPT = KT * HD / PER / kThreads;  // key pieces per thread and tile
  constexpr int VITEMS = (KT / 2) * (HD / 8);    // (key pair, 8 columns) items per tile
  const VirtRows vr = a.vr;
  const int lam = vr.lam, eta = vr.eta;
  // unit fastest: with the unit count a multiple of 8, a unit's chunks share
  // an XCD (blocks are dealt to the 8 XCDs round-robin) and its K/V rows,
  // re-read by every chunk, stay in that XCD's L2
  const int u = blockIdx.x, j = a.ch0 + blockIdx.y, pt = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, r = lane & 31;
  const int kvh = u % a.Hkv;
  const long long n0 = vr.n0;
  const long long nj = n0 + (long long)j * a.C;
  const int cj = min(a.C, vr.T - j * a.C);
  const long long pbase = nj + (long long)pt * a.ptile;
  const long long pend = min(pbase + a.ptile, nj + cj);     // exclusive
  if (pbase >= pend) return;                                // whole block idle (uniform)
  const int hd = wave / a.nblk, pblk = wave % a.nblk;
  const long long p0 = pbase + 32LL * pblk;
  const bool wactive = hd < a.g && p0 < pend;
  const long long qpos = p0 + r;
  const bool qvalid = wactive && qpos < pend;
  const int gsj = (int)min((long long)lam, max(0LL, nj - eta));
  const long long lo_j = max(0LL, nj - eta);
  const int nkeys = gsj + (int)(pend - lo_j);
  // last key any query of this wave sees (wave-uniform)
  const int wlast = gsj + (int)(min(p0 + 31, pend - 1) - lo_j);
  // keys 0 .. vis_end - 1 are visible to the lane's query (cache, window and
  // the causal prefix of the chunk up to and including the query)
  const int vis_end = (int)min((long long)nkeys, gsj + (qpos - lo_j) + 1);
  const int n0e = eta > 0 ? (int)(n0 % eta) : 0;            // ring slot of position n0 - eta

  extern __shared__ __align__(16) unsigned char smem[];
  const AttnLayout L = attn_layout(HD, lam, DT::kSplit);
  int32_t* sm_G = (int32_t*)(smem + L.G);
  T* sm_WT = (T*)(smem + L.WT);
  uint16_t* sm_HT_hi = (uint16_t*)(smem + L.HT_hi);
  uint16_t* sm_HT_lo = (uint16_t*)(smem + L.HT_lo);
  float* sm_s = (float*)(smem + L.s);

  // row of virtual index vi (cache slot, ring slot or input row), 32-bit math
  const T* ck = reinterpret_cast<const T*>(vr.cache_k) + (size_t)u * lam * HD;
  const T* cv = reinterpret_cast<const T*>(vr.cache_v) + (size_t)u * lam * HD;
  const T* rk = reinterpret_cast<const T*>(vr.ring_k) + (size_t)u * eta * HD;
  const T* rv = reinterpret_cast<const T*>(vr.ring_v) + (size_t)u * eta * HD;
  const T* ik = reinterpret_cast<const T*>(vr.in_k) + (size_t)u * vr.T * HD;
  const T* iv = reinterpret_cast<const T*>(vr.in_v) + (size_t)u * vr.T * HD;
  auto vrow = [&](int vi, bool val) -> const T* {
    if (vi < lam) return (val ? cv : ck) + (size_t)vi * HD;
    const int off = vi - lam;                       // position n0 - eta + off
    if (off < eta) {
      int slot = n0e + off;
      if (slot >= eta) slot -= eta;
      return (val ? rv : rk) + (size_t)slot * HD;
    }
    return (val ? iv : ik) + (size_t)(off - eta) * HD;
  };
  // virtual index of key kk: cache G_j, then local positions lo_j ..
  const int vi_loc0 = lam + eta + (int)(lo_j - n0);
  auto key_vi = [&](int kk) -> int { return kk < gsj ? sm_G[kk] : vi_loc0 + (kk - gsj); };

  // ---- stage W^T (this KV head), H_j^T hi / lo, s_j and G_j
  {
    const T* WT = reinterpret_cast<const T*>(a.WT) + (size_t)kvh * kM * HD;
    constexpr int WPIECES = kM * HD / PER;
    for (int i = tid; i < WPIECES; i += kThreads) {
      const int f = i / (HD / PER), c = (i % (HD / PER)) * PER;
      *reinterpret_cast<u32x4*>(sm_WT + f * KRS + c) = *reinterpret_cast<const u32x4*>(WT + (size_t)f * HD + c);
    }
    const uint16_t* snap = a.snapHT + ((size_t)u * a.nch + j) * 2 * HD * kD;
    constexpr int HPIECES = HD * (kD / 8);
    for (int i = tid; i < 2 * HPIECES; i += kThreads) {
      const int pl = i / HPIECES, rem = i % HPIECES;
      const int row = rem / (kD / 8), col = (rem % (kD / 8)) * 8;
      // (rows are 8-byte aligned: two 8-byte stores)
      const u32x4 x = *reinterpret_cast<const u32x4*>(snap + (size_t)pl * HD * kD + (size_t)row * kD + col);
      uint16_t* dst = (pl ? sm_HT_lo : sm_HT_hi) + row * HTS + col;
      *reinterpret_cast<u32x2*>(dst) = u32x2{x[0], x[1]};
      *reinterpret_cast<u32x2*>(dst + 4) = u32x2{x[2], x[3]};
    }
    const float* sj = a.snaps + ((size_t)u * a.nch + j) * kD;
    for (int F = tid; F < kD; F += kThreads) sm_s[F] = sj[F];
    const int32_t* Gj = a.snapG + ((size_t)u * a.nch + j) * lam;
    for (int i = tid; i < gsj; i += kThreads) sm_G[i] = Gj[i];
  }

  // ---- Q operands (B of S^T = K Q^T): lane = query r, K-slots 8h .. 8h+7
  u32x4 qh[KB], ql[KB];
  {
    const T* qrow = reinterpret_cast<const T*>(a.q) +
                    (((size_t)u * a.g + (wactive ? hd : 0)) * vr.T + (size_t)(qvalid ? qpos - n0 : 0)) * HD;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int k0 = 16 * kb + 8 * h;
      if constexpr (DT::kSplit) {
        float x[8];
        if (qvalid) load8_f32(qrow + k0, x);
        else for (int q = 0; q < 8; ++q) x[q] = 0.f;
        splitop<DT>(x, qh[kb], ql[kb]);
      } else {
        qh[kb] = qvalid ? ld16(reinterpret_cast<const uint16_t*>(qrow) + k0) : u32x4{0, 0, 0, 0};
        ql[kb] = u32x4{0, 0, 0, 0};
      }
    }
    // the operands are used here on every path: otherwise their loads would
    // count as pending in the key loop, which would then wait for all of its
    // own prefetches before the first product of every tile
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) __asm__ volatile("" :: "v"(qh[kb]), "v"(ql[kb]));
  }
  __syncthreads();

  // ---- phi(q): u^T = W^T q^T (64 features x 32 queries), softmax halves
  float ph[2][2][16];   // [half pos/neg][mt][i]: feature 64*half + 32*mt + 8(i/4) + 4h + (i%4)
  float zlin = 0.f;
  {
    f32x16 acc[2];
    for (int mt = 0; mt < 2; ++mt) for (int i = 0; i < 16; ++i) acc[mt][i] = 0.f;
    if (wactive) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int k0 = 16 * kb + 8 * h;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const T* wrow = sm_WT + (32 * mt + r) * KRS + k0;
          if constexpr (DT::kSplit) {
            float x[8];
            load8_f32(wrow, x);
            u32x4 ah, al;
            splitop<DT>(x, ah, al);
            acc[mt] = DT::mma(ah, qh[kb], acc[mt]);
            acc[mt] = DT::mma(ah, ql[kb], acc[mt]);
            acc[mt] = DT::mma(al, qh[kb], acc[mt]);
          } else {
            acc[mt] = DT::mma(ld16(reinterpret_cast<const uint16_t*>(wrow)), qh[kb], acc[mt]);
          }
        }
      }
    }
    float mx = -INFINITY, mn = INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
      for (int i = 0; i < 16; ++i) { mx = fmaxf(mx, acc[mt][i]); mn = fminf(mn, acc[mt][i]); }
    mx = fmaxf(mx, xor32(mx));
    mn = fminf(mn, xor32(mn));
    constexpr float kL2E = 1.4426950408889634f;
    const float mxl = mx * kL2E, mnl = mn * kL2E;
    float sp = 0.f, sn = 0.f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
      for (int i = 0; i < 16; ++i) {
        ph[0][mt][i] = __builtin_amdgcn_exp2f(fmaf(acc[mt][i], kL2E, -mxl));
        ph[1][mt][i] = __builtin_amdgcn_exp2f(fmaf(-acc[mt][i], kL2E, mnl));
        sp += ph[0][mt][i];
        sn += ph[1][mt][i];
      }
    sp += xor32(sp);
    sn += xor32(sn);
    const float ip = 1.f / sp, in_ = 1.f / sn;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
      for (int i = 0; i < 16; ++i) {
        ph[0][mt][i] *= ip;
        ph[1][mt][i] *= in_;
        const int f = 32 * mt + 8 * (i >> 2) + 4 * h + (i & 3);
        zlin = fmaf(ph[0][mt][i], sm_s[f], zlin);
        zlin = fmaf(ph[1][mt][i], sm_s[kM + f], zlin);
      }
    zlin += xor32(zlin);
    if (!(a.branches & LOLA_READ_STATE)) zlin = 0.f;   // state hidden from the read
  }

  // ---- linear read N_lin^T = H_j^T phi^T into the output accumulator
  f32x16 O[NMT];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) O[mt][i] = 0.f;
  if (wactive && (a.branches & LOLA_READ_STATE)) {
#pragma unroll
    for (int kb = 0; kb < kD / 16; ++kb) {
      const int half = kb >> 2, mt = (kb >> 1) & 1, i0 = 8 * (kb & 1);
      u32x4 bh, bl;
      splitop<DT>(&ph[half][mt][i0], bh, bl);
#pragma unroll
      for (int mo = 0; mo < NMT; ++mo) {
        const int row = 32 * mo + r;
        const u32x4 ah = sigma_load(sm_HT_hi + row * HTS + 16 * kb, h);
        const u32x4 al = sigma_load(sm_HT_lo + row * HTS + 16 * kb, h);
        O[mo] = DT::mma(ah, bh, O[mo]);
        O[mo] = DT::mma(ah, bl, O[mo]);
        O[mo] = DT::mma(al, bh, O[mo]);
      }
    }
  }
  __syncthreads();   // the key tiles reuse the linear-read region

  // ---- explicit branch: key tiles of KT, double-buffered
  float m2 = 0.f, l = zlin;
  const float scale2 = 1.4426950408889634f / sqrtf((float)HD);
  // cache keys hidden from the read: the key loop starts past them
  const int kbase = (a.branches & LOLA_READ_CACHE) ? 0 : gsj;
  const int ntiles = (nkeys - kbase + KT - 1) / KT;
  // one tile's pieces in registers: keys (KPT pieces of 16 bytes) and one
  // (key pair, 8 columns) item of V, kept as loaded: converting inside the
  // load's branch would make the wave wait for the load right there, before
  // the current tile's products
  constexpr int VPC = (int)sizeof(T) / 2;        // 16-byte pieces per 8 V columns
  u32x4 kreg[KPT];
  u32x4 vreg[2][VPC];
  auto load_tile = [&](int t0) {
#pragma unroll
    for (int q = 0; q < KPT; ++q) {
      const int pc = q * kThreads + tid, kl = pc / (HD / PER), c = (pc % (HD / PER)) * PER;
      const int kk = t0 + kl;
      kreg[q] = kk < nkeys ? *reinterpret_cast<const u32x4*>(vrow(key_vi(kk), false) + c)
                           : u32x4{0, 0, 0, 0};
    }
    if (tid < VITEMS) {
      const int pr = tid % (KT / 2), c = vt_cols(tid);
#pragma unroll
      for (int kq = 0; kq < 2; ++kq) {
        const int kk = t0 + 2 * pr + kq;
#pragma unroll
        for (int w = 0; w < VPC; ++w) vreg[kq][w] = u32x4{0, 0, 0, 0};
        if (kk < nkeys) {
          const u32x4* src = reinterpret_cast<const u32x4*>(vrow(key_vi(kk), true) + c);
#pragma unroll
          for (int w = 0; w < VPC; ++w) vreg[kq][w] = src[w];
        }
      }
    }
  };
  // buffer b's arrays (selects, so that the offsets stay in registers)
  auto buf_off = [&](const uint32_t (&o)[2], int b) -> uint32_t { return b ? o[1] : o[0]; };
  auto store_tile = [&](int b) {
    uint16_t* Kb = (uint16_t*)(smem + buf_off(L.K, b));
    uint16_t* KLb = (uint16_t*)(smem + buf_off(L.KL, b));
#pragma unroll
    for (int q = 0; q < KPT; ++q) {
      const int pc = q * kThreads + tid, kl = pc / (HD / PER), c = (pc % (HD / PER)) * PER;
      if constexpr (DT::kSplit) {
        float x[4] = {__uint_as_float(kreg[q][0]), __uint_as_float(kreg[q][1]),
                      __uint_as_float(kreg[q][2]), __uint_as_float(kreg[q][3])};
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) DT::split(x[e], hi[e], lo[e]);
        *reinterpret_cast<u32x2*>(Kb + kl * KRS + c) = u32x2{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16)};
        *reinterpret_cast<u32x2*>(KLb + kl * KRS + c) = u32x2{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)};
      } else {
        *reinterpret_cast<u32x4*>(Kb + kl * KRS + c) = kreg[q];
      }
    }
    if (tid < VITEMS) {
      const int pr = tid % (KT / 2), c = vt_cols(tid);
      uint16_t* VTb = (uint16_t*)(smem + buf_off(L.VT, b));
      uint16_t* VTLb = (uint16_t*)(smem + buf_off(L.VTL, b));
      float vf[2][8];
#pragma unroll
      for (int kq = 0; kq < 2; ++kq)
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          if constexpr (VPC == 1) {   // 8 bf16 in one piece
            const uint32_t w = vreg[kq][0][q >> 1];
            vf[kq][q] = __uint_as_float((q & 1) ? (w & 0xFFFF0000u) : (w << 16));
          } else {                    // 8 fp32 in two pieces
            vf[kq][q] = __uint_as_float(vreg[kq][q >> 2][q & 3]);
          }
        }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        uint32_t* row = reinterpret_cast<uint32_t*>(VTb + (c + q) * VTS) + pr;
        if constexpr (DT::kSplit) {
          uint32_t h0, l0, h1, l1;
          DT::split(vf[0][q], h0, l0);
          DT::split(vf[1][q], h1, l1);
          *row = h0 | (h1 << 16);
          *(reinterpret_cast<uint32_t*>(VTLb + (c + q) * VTS) + pr) = l0 | (l1 << 16);
        } else {
          *row = f16_bits(vf[0][q]) | (f16_bits(vf[1][q]) << 16);
        }
      }
    }
  };
  if (ntiles > 0) {
    load_tile(kbase);
    store_tile(0);
  }
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int t0 = kbase + t * KT, b = t & 1;
    if (t + 1 < ntiles) load_tile(t0 + KT);       // in flight during this tile's products
    if (wactive && t0 <= wlast) {
      const uint16_t* Kb = (const uint16_t*)(smem + buf_off(L.K, b));
      const uint16_t* KLb = (const uint16_t*)(smem + buf_off(L.KL, b));
      const uint16_t* VTb = (const uint16_t*)(smem + buf_off(L.VT, b));
      const uint16_t* VTLb = (const uint16_t*)(smem + buf_off(L.VTL, b));
      f32x16 S[2];
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
        for (int i = 0; i < 16; ++i) S[kh][i] = 0.f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const int k0 = 16 * kb + 8 * h;
          const u32x4 ah = ld16(Kb + (32 * kh + r) * KRS + k0);
          S[kh] = DT::mma(ah, qh[kb], S[kh]);
          if constexpr (DT::kSplit) {
            const u32x4 al = ld16(KLb + (32 * kh + r) * KRS + k0);
            S[kh] = DT::mma(ah, ql[kb], S[kh]);
            S[kh] = DT::mma(al, qh[kb], S[kh]);
          }
        }
      }
      // masks only where the tile has keys past the end or past the wave's
      // first query position (every query of the wave sees a full tile);
      // the scale goes into the exponent's fma.  Key kk is visible to the
      // lane's query iff kk < vis_end (cache keys precede the local ones, a
      // local key is visible up to the query's own position).
      const int klast = t0 + KT - 1;
      const bool full = klast < nkeys && (klast < gsj || lo_j + (klast - gsj) <= p0);
      if (!full) {
        const int dl = vis_end - t0 - 4 * h;      // the lane's offsets below dl are visible
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (32 * kh + 8 * (i >> 2) + (i & 3) >= dl) S[kh][i] = -INFINITY;
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, S[kh][i]);
      tmax = half_max(tmax) * scale2;   // (the scale is positive)
      // the running maximum moves only when a score would exceed it by more
      // than kSlack (weights up to 2^kSlack, well inside fp16 and fp32), so
      // that the accumulators are rarely rescaled
      if (tmax > m2 + kSlack) {
        const float mnew = tmax;
        const float alpha = __builtin_amdgcn_exp2f(m2 - mnew);
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
          for (int i = 0; i < 16; ++i) O[mt][i] *= alpha;
        l *= alpha;
        m2 = mnew;
      }
      float rs = 0.f;
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          S[kh][i] = __builtin_amdgcn_exp2f(fmaf(S[kh][i], scale2, -m2));
          rs += S[kh][i];
        }
      rs = half_sum(rs);
      l += rs;
#pragma unroll
      for (int kb = 0; kb < KT / 16; ++kb) {
        const int kh = kb >> 1, i0 = 8 * (kb & 1);
        if constexpr (DT::kSplit) {
          u32x4 ph8, pl8;
          float pv[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) pv[q] = S[kh][i0 + q];
          splitop<DT>(pv, ph8, pl8);
#pragma unroll
          for (int mo = 0; mo < NMT; ++mo) {
            const int row = 32 * mo + r;
            const u32x4 vh = sigma_load(VTb + row * VTS + 16 * kb, h);
            const u32x4 vl = sigma_load(VTLb + row * VTS + 16 * kb, h);
            O[mo] = DT::mma(vh, ph8, O[mo]);
            O[mo] = DT::mma(vh, pl8, O[mo]);
            O[mo] = DT::mma(vl, ph8, O[mo]);
          }
        } else {
          f16x8 p8;
#pragma unroll
          for (int q = 0; q < 8; ++q) p8[q] = (_Float16)S[kh][i0 + q];
#pragma unroll
          for (int mo = 0; mo < NMT; ++mo) {
            const int row = 32 * mo + r;
            const f16x8 vh = __builtin_bit_cast(f16x8, sigma_load(VTb + row * VTS + 16 * kb, h));
            O[mo] = mfma_f16(vh, p8, O[mo]);
          }
        }
      }
    }
    if (t + 1 < ntiles) store_tile(b ^ 1);
    __syncthreads();
  }

  // ---- y = O / l
  if (!qvalid) return;
  const float il = 1.f / l;
  float* orow = a.out + (((size_t)u * a.g + hd) * vr.T + (size_t)(qpos - n0)) * HD;
#pragma unroll
  for (int mo = 0; mo < NMT; ++mo)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int cc = 32 * mo + 8 * g4 + 4 * h;
      f32x4 y;
      for (int q = 0; q < 4; ++q) y[q] = O[mo][4 * g4 + q] * il;
      *reinterpret_cast<f32x4*>(orow + cc) = y;
    }
}

template <class DT, int HD>
static hipError_t launch_attn_t(const AttnArgs& a, int U, hipStream_t st) {
  const int nptile = (a.C + a.ptile - 1) / a.ptile;
  dim3 grid(U, a.nch_launch, nptile);
  const size_t lds = attn_lds_bytes(HD, a.vr.lam, DT::kSplit);
  const void* fn = (const void*)attn_kernel<DT, HD>;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_kernel<DT, HD>), grid, dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

int attn_positions_per_block(int C, int g) {
  const int p = 32 * kWaves / g;
  return C < p ? (C + 31) / 32 * 32 : p;
}

hipError_t launch_attn(const AttnArgs& a, int U, bool f32, hipStream_t st) {
  if (U <= 0 || a.nch_launch <= 0) return hipSuccess;
  if (a.ch0 < 0 || a.ch0 + a.nch_launch > a.nch) return hipErrorInvalidValue;
  if (a.vr.d == 64)
    return f32 ? launch_attn_t<F32, 64>(a, U, st) : launch_attn_t<BF16, 64>(a, U, st);
  return f32 ? launch_attn_t<F32, 128>(a, U, st) : launch_attn_t<BF16, 128>(a, U, st);
}

}  // namespace lola
