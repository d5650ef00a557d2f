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
// One workgroup = one unit, one chunk, and up to 4 waves; wave = one q-head
// x 32 positions (the GQA heads of a unit share every K/V tile).  Scores are
// computed transposed, S^T = K Q^T (32 keys x 32 queries), so each lane owns
// one query and softmax statistics need a single cross-half exchange; P then
// feeds O^T += V^T P^T straight from registers (the K index of that MFMA is
// permuted to match the result layout, see common.h).
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

constexpr int kThreads = 256;
constexpr int HTH = kM + 8;  // padded row of one half of H^T in LDS
constexpr int KTP = 36;      // row of the V^T tile: 32 keys + 4 (conflict-free pitch)

// Byte offsets of the LDS arrays; the key phase reuses the region of the
// linear-read phase.
struct AttnLayout {
  uint32_t WT_hi, WT_lo, HT_hi, HT_lo, s;      // linear-read phase
  uint32_t K_hi, K_lo, VT_a, VT_b;             // key phase
  uint32_t total;
};

inline __host__ __device__ uint32_t al16(uint32_t x) { return (x + 15u) & ~15u; }

__host__ __device__ inline AttnLayout attn_layout(int d, bool f32) {
  AttnLayout L;
  uint32_t off = 0;
  auto take = [&](uint32_t b) { const uint32_t o = off; off = al16(off + b); return o; };
  L.WT_hi = take((uint32_t)kM * (d + 8) * 2);          // [kM][d + 8]
  L.WT_lo = take(f32 ? (uint32_t)kM * (d + 8) * 2 : 16);
  L.HT_hi = take((uint32_t)d * HTH * 2);               // [d][HTH], one feature half
  L.HT_lo = take((uint32_t)d * HTH * 2);
  L.s = take(kD * 4);
  const uint32_t phaseA = off;
  off = 0;
  L.K_hi = take((uint32_t)32 * (d + 8) * 2);           // [32][d + 8]
  L.K_lo = take(f32 ? (uint32_t)32 * (d + 8) * 2 : 16);
  L.VT_a = take((uint32_t)d * KTP * 2);                // [d][KTP] fp16 (bf16 inputs) or hi
  L.VT_b = take(f32 ? (uint32_t)d * KTP * 2 : 16);     //          lo (fp32 inputs)
  L.total = phaseA > off ? phaseA : off;
  return L;
}

__device__ __forceinline__ u32x2 ld8(const uint16_t* p) { return *reinterpret_cast<const u32x2*>(p); }

// operand with K-slots sigma_h: elements [4h, 4h+4) and [8+4h, 8+4h+4) of a 16-block
__device__ __forceinline__ u32x4 sigma_load(const uint16_t* row16, int h) {
  u32x2 a = ld8(row16 + 4 * h), b = ld8(row16 + 8 + 4 * h);
  return u32x4{a[0], a[1], b[0], b[1]};
}

}  // namespace

size_t attn_lds_bytes(int d, bool f32) { return attn_layout(d, f32).total; }

template <class DT, int HD>
__global__ __launch_bounds__(kThreads) void attn_kernel(AttnArgs a) {
  using T = typename DT::T;
  constexpr int d = HD;
  constexpr int KB = HD / 16;     // 16-wide K blocks over the head dim
  constexpr int nmt = HD / 32;    // 32-row tiles of the output
  const VirtRows vr = a.vr;
  const int lam = vr.lam, eta = vr.eta;
  const int pt = blockIdx.x, j = blockIdx.y, u = blockIdx.z;
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

  extern __shared__ __align__(16) unsigned char smem[];
  const AttnLayout L = attn_layout(d, DT::kSplit);
  struct {
    uint16_t *WT_hi, *WT_lo, *HT_hi, *HT_lo;
    float* s;
    uint16_t *K_hi, *K_lo, *VT_a, *VT_b;
  } sm = {(uint16_t*)(smem + L.WT_hi), (uint16_t*)(smem + L.WT_lo), (uint16_t*)(smem + L.HT_hi),
          (uint16_t*)(smem + L.HT_lo), (float*)(smem + L.s), (uint16_t*)(smem + L.K_hi),
          (uint16_t*)(smem + L.K_lo), (uint16_t*)(smem + L.VT_a), (uint16_t*)(smem + L.VT_b)};

  // ---- W^T of this KV head and s_j into LDS
  const T* W = reinterpret_cast<const T*>(a.W) + (size_t)kvh * d * kM;
  for (int i = tid; i < d * kM; i += kThreads) {
    const int k = i / kM, f = i % kM;
    uint32_t hi, lo;
    DT::split(DT::to_f32(W[i]), hi, lo);
    sm.WT_hi[f * (d + 8) + k] = (uint16_t)hi;
    if (DT::kSplit) sm.WT_lo[f * (d + 8) + k] = (uint16_t)lo;
  }
  const float* sj = a.snaps + ((size_t)u * a.nch + j) * kD;
  for (int F = tid; F < kD; F += kThreads) sm.s[F] = sj[F];

  // ---- Q operands (B of S^T = K Q^T): lane = query r, K-slots 8h .. 8h+7
  u32x4 qh[KB], ql[KB];
  {
    const T* qrow = reinterpret_cast<const T*>(a.q) +
                    (((size_t)u * a.g + (wactive ? hd : 0)) * vr.T + (size_t)(qvalid ? qpos - n0 : 0)) * d;
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
      }
    }
  }
  __syncthreads();

  // ---- phi(q): u^T = W^T q^T (64 features x 32 queries)
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
          const int f = 32 * mt + r;
          const u32x4 ah = ld16(sm.WT_hi + f * (d + 8) + k0);
          acc[mt] = DT::mma(ah, qh[kb], acc[mt]);
          if constexpr (DT::kSplit) {
            const u32x4 al = ld16(sm.WT_lo + f * (d + 8) + k0);
            acc[mt] = DT::mma(ah, ql[kb], acc[mt]);
            acc[mt] = DT::mma(al, qh[kb], acc[mt]);
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
    float sp = 0.f, sn = 0.f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
      for (int i = 0; i < 16; ++i) {
        ph[0][mt][i] = expf(acc[mt][i] - mx);
        ph[1][mt][i] = expf(mn - acc[mt][i]);
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
        zlin = fmaf(ph[0][mt][i], sm.s[f], zlin);
        zlin = fmaf(ph[1][mt][i], sm.s[kM + f], zlin);
      }
    zlin += xor32(zlin);
  }

  // ---- linear read N_lin^T = H_j^T phi^T into the output accumulator
  f32x16 O[nmt];
#pragma unroll
  for (int mt = 0; mt < nmt; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) O[mt][i] = 0.f;
  const uint16_t* snap = a.snapHT + ((size_t)u * a.nch + j) * 2 * d * kD;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    __syncthreads();
    for (int i = tid; i < 2 * d * (kM / 8); i += kThreads) {
      const int pl = i / (d * (kM / 8)), rem = i % (d * (kM / 8));
      const int row = rem / (kM / 8), col = (rem % (kM / 8)) * 8;
      *reinterpret_cast<u32x4*>((pl ? sm.HT_lo : sm.HT_hi) + row * HTH + col) =
          *reinterpret_cast<const u32x4*>(snap + (size_t)pl * d * kD + (size_t)row * kD + kM * half + col);
    }
    __syncthreads();
    if (wactive) {
#pragma unroll
      for (int kb = 0; kb < kM / 16; ++kb) {
        const int mt = kb >> 1, i0 = 8 * (kb & 1);
        u32x4 bh, bl;
        splitop<DT>(&ph[half][mt][i0], bh, bl);
#pragma unroll
        for (int mo = 0; mo < nmt; ++mo) {
          const int row = 32 * mo + r;
          const u32x4 ah = sigma_load(sm.HT_hi + row * HTH + 16 * kb, h);
          const u32x4 al = sigma_load(sm.HT_lo + row * HTH + 16 * kb, h);
          O[mo] = DT::mma(ah, bh, O[mo]);
          O[mo] = DT::mma(ah, bl, O[mo]);
          O[mo] = DT::mma(al, bh, O[mo]);
        }
      }
    }
  }

  // ---- explicit branch: cache G_j, then local positions lo_j .. pend-1
  float m2 = 0.f, l = zlin;
  const float scale2 = 1.4426950408889634f / sqrtf((float)d);
  const int gsj = (int)min((long long)lam, max(0LL, nj - eta));
  const long long lo_j = max(0LL, nj - eta);
  const int nkeys = gsj + (int)(pend - lo_j);
  const int32_t* Gj = a.snapG + ((size_t)u * a.nch + j) * lam;
  for (int t0 = 0; t0 < nkeys; t0 += 32) {
    __syncthreads();
    // K tile, row-major [key][d]: 16-byte pieces (raw copy for bf16)
    for (int i = tid; i < 32 * (d / 8); i += kThreads) {
      const int kl = i / (d / 8), cc = (i % (d / 8)) * 8;
      const int kk = t0 + kl;
      const int vi = kk < nkeys ? (kk < gsj ? Gj[kk] : lam + eta + (int)(lo_j + (kk - gsj) - n0)) : -1;
      if constexpr (DT::kSplit) {
        float kv[8];
        if (vi >= 0) load8_f32(reinterpret_cast<const T*>(vr.krow(u, vi, sizeof(T))) + cc, kv);
        else for (int q = 0; q < 8; ++q) kv[q] = 0.f;
        u32x4 kh, kl8;
        splitop<DT>(kv, kh, kl8);
        *reinterpret_cast<u32x4*>(sm.K_hi + kl * (d + 8) + cc) = kh;
        *reinterpret_cast<u32x4*>(sm.K_lo + kl * (d + 8) + cc) = kl8;
      } else {
        *reinterpret_cast<u32x4*>(sm.K_hi + kl * (d + 8) + cc) =
            vi >= 0 ? *reinterpret_cast<const u32x4*>(vr.krow(u, vi, sizeof(T)) + cc * sizeof(T))
                    : u32x4{0, 0, 0, 0};
      }
    }
    // V^T tile [d][KTP]: a thread takes two consecutive keys x 8 columns and
    // writes 8 dwords (the key pair) -- 16 threads fill 16 consecutive dwords
    // of one row, and the row pitch puts the four row groups of a wave on
    // disjoint banks.
    for (int i = tid; i < 16 * (d / 8); i += kThreads) {
      const int pr = i % 16, cc = (i / 16) * 8;
      float v0[8], v1[8];
#pragma unroll
      for (int kq = 0; kq < 2; ++kq) {
        const int kk = t0 + 2 * pr + kq;
        float* dst = kq ? v1 : v0;
        if (kk < nkeys) {
          const int vi = kk < gsj ? Gj[kk] : lam + eta + (int)(lo_j + (kk - gsj) - n0);
          load8_f32(reinterpret_cast<const T*>(vr.vrow(u, vi, sizeof(T))) + cc, dst);
        } else {
          for (int q = 0; q < 8; ++q) dst[q] = 0.f;
        }
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        uint32_t* row = reinterpret_cast<uint32_t*>(sm.VT_a + (cc + q) * KTP) + pr;
        if constexpr (DT::kSplit) {
          uint32_t h0, l0, h1, l1;
          DT::split(v0[q], h0, l0);
          DT::split(v1[q], h1, l1);
          *row = h0 | (h1 << 16);
          *(reinterpret_cast<uint32_t*>(sm.VT_b + (cc + q) * KTP) + pr) = l0 | (l1 << 16);
        } else {
          *row = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v0[q]) |
                 ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v1[q]) << 16);
        }
      }
    }
    __syncthreads();
    if (!wactive) continue;
    f32x16 S;
#pragma unroll
    for (int i = 0; i < 16; ++i) S[i] = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int k0 = 16 * kb + 8 * h;
      const u32x4 ah = ld16(sm.K_hi + r * (d + 8) + k0);
      S = DT::mma(ah, qh[kb], S);
      if constexpr (DT::kSplit) {
        const u32x4 al = ld16(sm.K_lo + r * (d + 8) + k0);
        S = DT::mma(ah, ql[kb], S);
        S = DT::mma(al, qh[kb], S);
      }
    }
    float tmax = -INFINITY;
    for (int i = 0; i < 16; ++i) {
      const int kk = t0 + 8 * (i >> 2) + 4 * h + (i & 3);
      bool ok = kk < nkeys;
      if (ok && kk >= gsj) ok = lo_j + (kk - gsj) <= qpos;   // causal (diagonal included)
      S[i] = ok ? S[i] * scale2 : -INFINITY;
      tmax = fmaxf(tmax, S[i]);
    }
    tmax = fmaxf(tmax, xor32(tmax));
    const float mnew = fmaxf(m2, tmax);
    if (mnew > m2) {
      const float alpha = exp2f(m2 - mnew);
#pragma unroll
      for (int mt = 0; mt < nmt; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) O[mt][i] *= alpha;
      l *= alpha;
      m2 = mnew;
    }
    float rs = 0.f;
    for (int i = 0; i < 16; ++i) { S[i] = exp2f(S[i] - m2); rs += S[i]; }
    rs += xor32(rs);
    l += rs;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if constexpr (DT::kSplit) {
        u32x4 ph8, pl8;
        float pv[8];
        for (int q = 0; q < 8; ++q) pv[q] = S[8 * kb + q];
        splitop<DT>(pv, ph8, pl8);
#pragma unroll
        for (int mo = 0; mo < nmt; ++mo) {
          const int row = 32 * mo + r;
          const u32x4 vh = sigma_load(sm.VT_a + row * KTP + 16 * kb, h);
          const u32x4 vl = sigma_load(sm.VT_b + row * KTP + 16 * kb, h);
          O[mo] = DT::mma(vh, ph8, O[mo]);
          O[mo] = DT::mma(vh, pl8, O[mo]);
          O[mo] = DT::mma(vl, ph8, O[mo]);
        }
      } else {
        f16x8 p8;
#pragma unroll
        for (int q = 0; q < 8; ++q) p8[q] = (_Float16)S[8 * kb + q];
#pragma unroll
        for (int mo = 0; mo < nmt; ++mo) {
          const int row = 32 * mo + r;
          f16x8 vh = __builtin_bit_cast(f16x8, sigma_load(sm.VT_a + row * KTP + 16 * kb, h));
          O[mo] = mfma_f16(vh, p8, O[mo]);
        }
      }
    }
  }

  // ---- y = O / l
  if (!qvalid) return;
  const float il = 1.f / l;
  float* orow = a.out + (((size_t)u * a.g + hd) * vr.T + (size_t)(qpos - n0)) * d;
#pragma unroll
  for (int mo = 0; mo < nmt; ++mo)
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
  dim3 grid(nptile, a.nch, U);
  const size_t lds = attn_lds_bytes(HD, DT::kSplit);
  (void)hipFuncSetAttribute((const void*)attn_kernel<DT, HD>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  hipLaunchKernelGGL((attn_kernel<DT, HD>), grid, dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

hipError_t launch_attn(const AttnArgs& a, int U, bool f32, hipStream_t st) {
  if (U <= 0 || a.nch <= 0) return hipSuccess;
  if (a.vr.d == 64)
    return f32 ? launch_attn_t<F32, 64>(a, U, st) : launch_attn_t<BF16, 64>(a, U, st);
  return f32 ? launch_attn_t<F32, 128>(a, U, st) : launch_attn_t<BF16, 128>(a, U, st);
}

}  // namespace lola
