// K1: feature map phi(x) = [softmax(x W_h), softmax(-x W_h)] for every row a
// prefill call may score or fold (cache at call start, window ring, input).
//
// LoLA notes §2.1 (phi: R^{d_k} -> R^D, D = 2 d_k) with the fixed softmax form
// of the workloads; one W_h (d x 64) per KV head.  x W_h is a dense
// contraction and runs on MFMA: bf16 inputs are exact in one pass with fp32
// accumulation; fp32 inputs use the hi/lo fp16 split (three passes).  The
// 64-wide softmaxes run on the VALU in fp32.  The result is stored as two
// 16-bit planes (hi, lo = x - hi; bf16 for bf16 inputs, fp16 for fp32 inputs),
// ready to be MFMA operands of the SRE GEMM and the fold.
//
// Work split: one wave = 32 rows.  It computes u^T = W^T x^T (64 features x
// 32 rows), so lane l owns row l % 32 and 32 of its 64 features; the other 32
// sit in lane l ^ 32, and each softmax needs one cross-half exchange.
#include "internal.h"

namespace lola {

template <class DT, int HD>
__global__ __launch_bounds__(256) void phi_kernel(PhiArgs a) {
  using T = typename DT::T;
  constexpr int WPAD = 8;
  constexpr int d = HD;
  const int u = blockIdx.y;
  const int kvh = u % a.Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, r = lane & 31;

  const int vi = blockIdx.x * 128 + wave * 32 + r;
  bool valid = vi < a.NV;
  if (valid) {
    if (vi < a.vr.lam) valid = vi < a.gs0;
    else valid = (a.vr.n0 - a.vr.eta + (vi - a.vr.lam)) >= 0;
  }
  const T* xrow = valid ? reinterpret_cast<const T*>(a.vr.krow(u, vi, sizeof(T))) : nullptr;
  // 16-bit inputs: the row's operands are loaded first, in flight with the
  // staging of W below (fixed trip counts: every load of the wave is issued
  // before any is used)
  u32x4 bx[HD / 16];
  if constexpr (!DT::kSplit) {
#pragma unroll
    for (int kb = 0; kb < HD / 16; ++kb)
      bx[kb] = valid ? ld16(reinterpret_cast<const uint16_t*>(xrow) + kb * 16 + 8 * h)
                     : u32x4{0, 0, 0, 0};
  }

  // W^T for this KV head: wT[f][k] (hi and, for fp32 inputs, lo planes);
  // 8 consecutive features of one k per piece, all pieces loaded first
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* wT_hi = reinterpret_cast<uint16_t*>(smem);
  uint16_t* wT_lo = wT_hi + kM * (d + WPAD);
  const T* W = reinterpret_cast<const T*>(a.W) + (size_t)kvh * d * kM;
  {
    constexpr int PIECES = d * kM / 8;
    static_assert(PIECES % 256 == 0, "fixed trip count");
    constexpr int PT = PIECES / 256;
    float wv[PT][8];
#pragma unroll
    for (int q = 0; q < PT; ++q) {
      const int i = threadIdx.x + 256 * q;
      const int k = i / (kM / 8), f0 = (i % (kM / 8)) * 8;
      if constexpr (sizeof(T) == 2) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(W + (size_t)k * kM + f0);
#pragma unroll
        for (int j = 0; j < 8; ++j) wv[q][j] = DT::from_bits((x[j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
      } else {
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(W + (size_t)k * kM + f0);
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(W + (size_t)k * kM + f0 + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) { wv[q][j] = x0[j]; wv[q][4 + j] = x1[j]; }
      }
    }
#pragma unroll
    for (int q = 0; q < PT; ++q) {
      const int i = threadIdx.x + 256 * q;
      const int k = i / (kM / 8), f0 = (i % (kM / 8)) * 8;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t hi, lo;
        DT::split(wv[q][j], hi, lo);
        wT_hi[(f0 + j) * (d + WPAD) + k] = (uint16_t)hi;
        if (DT::kSplit) wT_lo[(f0 + j) * (d + WPAD) + k] = (uint16_t)lo;
      }
    }
  }
  __syncthreads();

  f32x16 acc[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[mt][i] = 0.f;
#pragma unroll
  for (int kb = 0; kb < d / 16; ++kb) {
    const int k0 = kb * 16 + 8 * h;
    u32x4 bx_hi, bx_lo;
    if constexpr (DT::kSplit) {
      float xv[8];
      if (valid) load8_f32(xrow + k0, xv);
      else for (int j = 0; j < 8; ++j) xv[j] = 0.f;
      splitop<DT>(xv, bx_hi, bx_lo);
    } else {
      bx_hi = bx[kb];
    }
    for (int mt = 0; mt < 2; ++mt) {
      const int f = mt * 32 + r;
      const u32x4 aw_hi = ld16(wT_hi + f * (d + WPAD) + k0);
      acc[mt] = DT::mma(aw_hi, bx_hi, acc[mt]);
      if constexpr (DT::kSplit) {
        const u32x4 aw_lo = ld16(wT_lo + f * (d + WPAD) + k0);
        acc[mt] = DT::mma(aw_hi, bx_lo, acc[mt]);
        acc[mt] = DT::mma(aw_lo, bx_hi, acc[mt]);
      }
    }
  }
  // lane holds u[f] for f = 32mt + 8(i/4) + 4h + (i%4), row r
  float mx = -INFINITY, mn = INFINITY;
  for (int mt = 0; mt < 2; ++mt)
    for (int i = 0; i < 16; ++i) { mx = fmaxf(mx, acc[mt][i]); mn = fminf(mn, acc[mt][i]); }
  mx = fmaxf(mx, xor32(mx));
  mn = fminf(mn, xor32(mn));
  float ep[2][16], en[2][16], sp = 0.f, sn = 0.f;
  for (int mt = 0; mt < 2; ++mt)
    for (int i = 0; i < 16; ++i) {
      ep[mt][i] = expf(acc[mt][i] - mx);
      en[mt][i] = expf(mn - acc[mt][i]);
      sp += ep[mt][i];
      sn += en[mt][i];
    }
  sp += xor32(sp);
  sn += xor32(sn);
  if (!valid) return;
  const float ip = 1.f / sp, in_ = 1.f / sn;
  const size_t rowoff = ((size_t)u * a.NV + vi) * kD;
  for (int mt = 0; mt < 2; ++mt)
    for (int g4 = 0; g4 < 4; ++g4) {
      const int f = mt * 32 + 8 * g4 + 4 * h;
      uint32_t hp[4], lp[4], hn[4], ln[4];
      for (int j = 0; j < 4; ++j) {
        DT::split(ep[mt][4 * g4 + j] * ip, hp[j], lp[j]);
        DT::split(en[mt][4 * g4 + j] * in_, hn[j], ln[j]);
      }
      u32x2 w;
      w[0] = hp[0] | (hp[1] << 16); w[1] = hp[2] | (hp[3] << 16);
      *reinterpret_cast<u32x2*>(a.phi_hi + rowoff + f) = w;
      w[0] = lp[0] | (lp[1] << 16); w[1] = lp[2] | (lp[3] << 16);
      *reinterpret_cast<u32x2*>(a.phi_lo + rowoff + f) = w;
      w[0] = hn[0] | (hn[1] << 16); w[1] = hn[2] | (hn[3] << 16);
      *reinterpret_cast<u32x2*>(a.phi_hi + rowoff + kM + f) = w;
      w[0] = ln[0] | (ln[1] << 16); w[1] = ln[2] | (ln[3] << 16);
      *reinterpret_cast<u32x2*>(a.phi_lo + rowoff + kM + f) = w;
    }
}

hipError_t launch_phi(const PhiArgs& a, int U, bool f32, hipStream_t st) {
  if (a.NV <= 0 || U <= 0) return hipSuccess;
  dim3 grid((a.NV + 127) / 128, U);
  size_t lds = (size_t)2 * kM * (a.vr.d + 8) * sizeof(uint16_t);
  if (a.vr.d == 64) {
    if (f32) hipLaunchKernelGGL((phi_kernel<F32, 64>), grid, dim3(256), lds, st, a);
    else hipLaunchKernelGGL((phi_kernel<BF16, 64>), grid, dim3(256), lds, st, a);
  } else {
    if (f32) hipLaunchKernelGGL((phi_kernel<F32, 128>), grid, dim3(256), lds, st, a);
    else hipLaunchKernelGGL((phi_kernel<BF16, 128>), grid, dim3(256), lds, st, a);
  }
  return hipGetLastError();
}

}  // namespace lola
