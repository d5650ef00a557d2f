// K2: LoLA's serial memory-allocation chain, one step per chunk, one
// workgroup (8 waves) per unit (b, KV head).
//
// Per chunk j (LoLA notes §2.6, Eq. (15); §2.4, Eqs. (11)-(13)):
//   1. snapshot (H_j, s_j, G_j): the state the chunk's queries read;
//   2. candidates E = G_j ++ L_j, L_j = positions leaving the window;
//   3. if |E| <= lam: G_{j+1} = E (keep all);
//   4. else SRE of every candidate against (H_j, s_j) (notes §2.3, Eq. (10),
//      squared), exact top-lam by (SRE desc, position asc), stable compaction,
//      and the fold H += Phi_S^T V_S, s += sum phi over the rest.
//
// Precision.  SRE decides an integer (cache membership), so its GEMM
// p = H^T phi runs as a three-pass 16-bit split (hi*hi + hi*lo + lo*hi, fp32
// accumulation; bf16 halves for bf16 inputs, fp16 for fp32 inputs): relative
// error ~1e-8 on these data, far inside the 1e-5 ranking band.  z = phi^T s is
// an fp32 dot product of (hi + lo) with s on the VALU, overlapping the MFMAs.
// The fold multiplies phi (hi + lo) by V (exact in one bf16 operand, or split
// for fp32 inputs) and accumulates into fp32 H.
//
// Layout.  H (D x d, fp32) lives in registers for the whole call in MFMA
// result layout: 32 x 32 tiles (feature block mt, column slab cs), two tiles
// per wave; folds accumulate into them in place.  After each fold H^T is
// rebuilt in LDS as hi/lo planes, the A operand of the next step's SRE GEMM,
// whose 32-candidate row tiles are spread over the eight waves.
#include "internal.h"

namespace lola {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int HTP = kD + 8;   // padded LDS row of H^T (16-bit elements)
constexpr int STP = 32 + 8;   // padded LDS row of fold staging tiles

// Byte offsets of the LDS arrays (computed by value so that the kernel's
// pointers stay plain LDS pointers).
struct ChainLayout {
  uint32_t HT_hi, HT_lo, s32, spart, G, E, S, keys, hist, misc, phT_hi, phT_lo, VT_hi, VT_lo;
  uint32_t total;
};

__host__ __device__ inline uint32_t align16(uint32_t x) { return (x + 15u) & ~15u; }

__host__ __device__ inline ChainLayout chain_layout(int lam, int C, int d, bool f32) {
  ChainLayout L;
  uint32_t off = 0;
  auto take = [&](uint32_t bytes) { const uint32_t o = off; off = align16(off + bytes); return o; };
  L.HT_hi = take((uint32_t)d * HTP * 2);   // [d][HTP]
  L.HT_lo = take((uint32_t)d * HTP * 2);
  L.s32 = take(kD * 4);                    // [kD]
  L.spart = take(4 * kD * 4);              // [4][kD]
  L.G = take((uint32_t)(lam > 0 ? lam : 1) * 4);   // [lam]
  L.E = take((uint32_t)(lam + C) * 4);     // [lam + C]
  L.S = take((uint32_t)(lam + C) * 4);     // [lam + C] folded list
  L.keys = take((uint32_t)(lam + C) * 8);  // [lam + C]
  L.hist = take(256 * 4);
  L.misc = take(16 * 4);
  L.phT_hi = take(kD * STP * 2);           // [kD][STP]
  L.phT_lo = take(kD * STP * 2);
  L.VT_hi = take((uint32_t)d * STP * 2);   // [d][STP]
  L.VT_lo = take(f32 ? (uint32_t)d * STP * 2 : 16);
  L.total = off;
  return L;
}

// exclusive scan of one int per thread over the block
__device__ __forceinline__ int block_excl_scan(int x, int32_t* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_incl_scan(x);
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int off = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w)
    if (w < wave) off += wsum[w];
  __syncthreads();
  return off + incl - x;
}

}  // namespace

size_t chain_lds_bytes(int lam, int C, int d, bool f32) {
  return chain_layout(lam, C, d, f32).total;
}

template <class DT, int HD>
__global__ __launch_bounds__(kThreads) void chain_kernel(ChainArgs a) {
  using T = typename DT::T;
  constexpr int NSLAB = HD / 32;                  // column slabs of H
  constexpr int NPW = NSLAB * 4 / kWaves;         // H tiles per wave (1 or 2)
  const VirtRows vr = a.vr;
  const int lam = vr.lam, eta = vr.eta;
  const int u = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, r = lane & 31;

  extern __shared__ __align__(16) unsigned char smem[];
  const ChainLayout L = chain_layout(lam, a.C, HD, DT::kSplit);
  struct {
    uint16_t *HT_hi, *HT_lo;
    float *s32, *spart;
    int32_t *G, *E, *S;
    uint64_t* keys;
    int32_t *hist, *misc;
    uint16_t *phT_hi, *phT_lo, *VT_hi, *VT_lo;
  } sm = {(uint16_t*)(smem + L.HT_hi), (uint16_t*)(smem + L.HT_lo), (float*)(smem + L.s32),
          (float*)(smem + L.spart), (int32_t*)(smem + L.G), (int32_t*)(smem + L.E),
          (int32_t*)(smem + L.S), (uint64_t*)(smem + L.keys), (int32_t*)(smem + L.hist),
          (int32_t*)(smem + L.misc), (uint16_t*)(smem + L.phT_hi), (uint16_t*)(smem + L.phT_lo),
          (uint16_t*)(smem + L.VT_hi), (uint16_t*)(smem + L.VT_lo)};

  // ---- H tiles of this wave: pair p = wave + kWaves * i -> (slab p / 4, mt p % 4)
  f32x16 Hreg[NPW];
  const float* Hg = a.H + (size_t)u * kD * HD;
#pragma unroll
  for (int i = 0; i < NPW; ++i) {
    const int p = wave + kWaves * i, cs = p >> 2, mt = p & 3;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int F = 32 * mt + 8 * (q >> 2) + 4 * h + (q & 3);
      Hreg[i][q] = Hg[(size_t)F * HD + 32 * cs + r];
    }
  }
  for (int F = tid; F < kD; F += kThreads) sm.s32[F] = a.s[(size_t)u * kD + F];
  const long long n0 = vr.n0;
  const int gs0 = (int)min((long long)lam, max(0LL, n0 - eta));
  for (int i = tid; i < gs0; i += kThreads) sm.G[i] = i;

  auto rebuild_HT = [&]() {
#pragma unroll
    for (int i = 0; i < NPW; ++i) {
      const int p = wave + kWaves * i, cs = p >> 2, mt = p & 3;
      const int c = 32 * cs + r;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int F = 32 * mt + 8 * g4 + 4 * h;
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) DT::split(Hreg[i][4 * g4 + q], hi[q], lo[q]);
        *reinterpret_cast<u32x2*>(sm.HT_hi + c * HTP + F) =
            u32x2{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16)};
        *reinterpret_cast<u32x2*>(sm.HT_lo + c * HTP + F) =
            u32x2{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)};
      }
    }
  };
  rebuild_HT();
  __syncthreads();

  int gs = gs0;
  const size_t phi_unit = (size_t)u * a.NV * kD;
  for (int j = 0; j < a.nch; ++j) {
    const long long nj = n0 + (long long)j * a.C;
    const int c = min(a.C, vr.T - j * a.C);

    // ---- 1. snapshot (H_j^T hi/lo, s_j, G_j)
    {
      uint16_t* dst = a.snapHT + ((size_t)u * a.nch + j) * 2 * HD * kD;
      constexpr int chunks = HD * (kD / 8);  // 16-byte pieces per plane
      for (int i = tid; i < 2 * chunks; i += kThreads) {
        const int pl = i / chunks, rem = i % chunks;
        const int row = rem / (kD / 8), col = (rem % (kD / 8)) * 8;
        const uint16_t* src = (pl ? sm.HT_lo : sm.HT_hi) + row * HTP + col;
        *reinterpret_cast<u32x4*>(dst + (size_t)pl * HD * kD + row * kD + col) =
            *reinterpret_cast<const u32x4*>(src);
      }
      float* sdst = a.snaps + ((size_t)u * a.nch + j) * kD;
      for (int F = tid; F < kD; F += kThreads) sdst[F] = sm.s32[F];
      int32_t* gdst = a.snapG + ((size_t)u * a.nch + j) * lam;
      for (int i = tid; i < gs; i += kThreads) gdst[i] = sm.G[i];
    }

    // ---- 2. candidates
    const long long lo_p = max(0LL, nj - eta), hi_p = max(0LL, nj + c - eta);
    const int nL = (int)(hi_p - lo_p);
    const int nE = gs + nL;
    const int vi_L0 = lam + eta + (int)(lo_p - n0);
    if (nE <= lam) {                       // 3. keep all
      for (int i = tid; i < nL; i += kThreads) sm.G[gs + i] = vi_L0 + i;
      gs = nE;
      __syncthreads();
      continue;
    }
    for (int i = tid; i < nE; i += kThreads) sm.E[i] = i < gs ? sm.G[i] : vi_L0 + (i - gs);
    __syncthreads();

    // ---- 4a. SRE of every candidate, 32-row tiles over the waves
    for (int t = wave; lam > 0 && t * 32 < nE; t += kWaves) {
      const int e = t * 32 + r;
      const bool ev = e < nE;
      const int vi = ev ? sm.E[e] : sm.E[0];
      const uint16_t* ph = a.phi_hi + phi_unit + (size_t)vi * kD;
      const uint16_t* pl = a.phi_lo + phi_unit + (size_t)vi * kD;
      f32x16 P[NSLAB];
#pragma unroll
      for (int mt = 0; mt < NSLAB; ++mt)
#pragma unroll
        for (int q = 0; q < 16; ++q) P[mt][q] = 0.f;
      float z = 0.f;
#pragma unroll 2
      for (int kb = 0; kb < 8; ++kb) {
        const int k0 = kb * 16 + 8 * h;
        const u32x4 bh = ld16(ph + k0), bl = ld16(pl + k0);
#pragma unroll
        for (int mt = 0; mt < NSLAB; ++mt) {
          const int row = 32 * mt + r;
          const u32x4 ah = ld16(sm.HT_hi + row * HTP + k0);
          const u32x4 al = ld16(sm.HT_lo + row * HTP + k0);
          P[mt] = DT::mma(ah, bh, P[mt]);
          P[mt] = DT::mma(al, bh, P[mt]);
          P[mt] = DT::mma(ah, bl, P[mt]);
        }
        // z = phi^T s on the VALU from the same operand registers
        const f32x4 s0 = *reinterpret_cast<const f32x4*>(sm.s32 + k0);
        const f32x4 s1 = *reinterpret_cast<const f32x4*>(sm.s32 + k0 + 4);
        const float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t wh = bh[q], wl = bl[q];
          z = fmaf(DT::from_bits(wh & 0xFFFFu) + DT::from_bits(wl & 0xFFFFu), sv[2 * q], z);
          z = fmaf(DT::from_bits(wh >> 16) + DT::from_bits(wl >> 16), sv[2 * q + 1], z);
        }
      }
      z += xor32(z);
      const float iz = z > 0.f ? 1.f / z : 0.f;   // z == 0: prediction 0
      float acc = 0.f;
      const T* vrow = reinterpret_cast<const T*>(vr.vrow(u, vi, sizeof(T)));
#pragma unroll
      for (int mt = 0; mt < NSLAB; ++mt)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int cc = 32 * mt + 8 * g4 + 4 * h;
          float vv[4];
          if constexpr (DT::kSplit) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(vrow + cc);
#pragma unroll
            for (int q = 0; q < 4; ++q) vv[q] = x[q];
          } else {
            const u32x2 x = *reinterpret_cast<const u32x2*>(vrow + cc);
            vv[0] = __uint_as_float(x[0] << 16);
            vv[1] = __uint_as_float(x[0] & 0xFFFF0000u);
            vv[2] = __uint_as_float(x[1] << 16);
            vv[3] = __uint_as_float(x[1] & 0xFFFF0000u);
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float df = P[mt][4 * g4 + q] * iz - vv[q];
            acc = fmaf(df, df, acc);
          }
        }
      acc += xor32(acc);
      if (ev && h == 0) {
        const uint32_t pos = (uint32_t)vr.pos_of(u, vi);
        sm.keys[e] = ((uint64_t)__float_as_uint(acc) << 32) | (uint64_t)(0xFFFFFFFFu - pos);
      }
    }
    __syncthreads();
    if (a.dbg_keys) {
      uint64_t* dk = a.dbg_keys + ((size_t)u * a.nch + j) * (lam + a.C);
      for (int e = tid; e < nE; e += kThreads) dk[e] = sm.keys[e];
    }

    // ---- 4b. exact top-lam: radix select of the lam-th largest key
    // (lam == 0: nothing is kept, every candidate is folded)
    uint64_t prefix = 0, mask = 0;
    int need = lam;
    for (int shift = 56; shift >= 0 && lam > 0; shift -= 8) {
      for (int i = tid; i < 256; i += kThreads) sm.hist[i] = 0;
      __syncthreads();
      for (int e = tid; e < nE; e += kThreads) {
        const uint64_t k = sm.keys[e];
        if ((k & mask) == prefix) atomicAdd(&sm.hist[(k >> shift) & 255], 1);
      }
      __syncthreads();
      if (wave == 0) {
        int cnt[4], tot = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) { cnt[b] = sm.hist[4 * lane + b]; tot += cnt[b]; }
        const int incl = wave_incl_scan(tot);
        const int all = __shfl(incl, 63, 64);
        int above = all - incl;            // elements in bins above this lane's four
#pragma unroll
        for (int b = 3; b >= 0; --b) {
          if (above < need && need <= above + cnt[b]) {
            sm.misc[0] = 4 * lane + b;
            sm.misc[1] = need - above;
            sm.misc[2] = cnt[b];
          }
          above += cnt[b];
        }
      }
      __syncthreads();
      const int b = sm.misc[0];
      need = sm.misc[1];
      const int cb = sm.misc[2];
      prefix |= (uint64_t)b << shift;
      mask |= (uint64_t)255 << shift;
      if (cb == need) break;
    }

    // ---- 4c. stable compaction: kept -> G (E order), rest -> S
    {
      const int seg = (nE + kThreads - 1) / kThreads;
      const int e0 = min(nE, tid * seg), e1 = min(nE, e0 + seg);
      int kept = 0;
      for (int e = e0; e < e1; ++e) kept += lam > 0 && (sm.keys[e] & mask) >= prefix;
      int kb = block_excl_scan(kept, sm.misc + 4);
      for (int e = e0; e < e1; ++e) {
        if (lam > 0 && (sm.keys[e] & mask) >= prefix) {
          if (kb < lam) sm.G[kb] = sm.E[e];
          ++kb;
        } else if (e - kb < nE - lam) {
          sm.S[e - kb] = sm.E[e];
        }
      }
    }
    gs = lam;
    __syncthreads();

    // ---- 4d. fold the rest into H (MFMA) and s
    const int nS = nE - lam;
    float sacc = 0.f;
    {
      const int F = tid % kD, tg = tid / kD;   // tg in [0, 4): 8 tokens each
      for (int sb = 0; sb < nS; sb += 32) {
        {
          uint32_t hb[8], lb[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const int tok = sb + 8 * tg + q;
            if (tok < nS) {
              const size_t o = phi_unit + (size_t)sm.S[tok] * kD + F;
              hb[q] = a.phi_hi[o];
              lb[q] = a.phi_lo[o];
              sacc += DT::from_bits(hb[q]) + DT::from_bits(lb[q]);
            } else {
              hb[q] = 0; lb[q] = 0;
            }
          }
          *reinterpret_cast<u32x4*>(sm.phT_hi + F * STP + 8 * tg) = pack8(hb);
          *reinterpret_cast<u32x4*>(sm.phT_lo + F * STP + 8 * tg) = pack8(lb);
        }
        for (int it = tid; it < HD * 4; it += kThreads) {
          const int cc = it % HD, grp = it / HD;
          uint32_t vh[8], vl[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const int tok = sb + 8 * grp + q;
            float x = 0.f;
            if (tok < nS) {
              const T* vrow = reinterpret_cast<const T*>(vr.vrow(u, sm.S[tok], sizeof(T)));
              x = DT::to_f32(vrow[cc]);
            }
            DT::split(x, vh[q], vl[q]);
          }
          *reinterpret_cast<u32x4*>(sm.VT_hi + cc * STP + 8 * grp) = pack8(vh);
          if constexpr (DT::kSplit)
            *reinterpret_cast<u32x4*>(sm.VT_lo + cc * STP + 8 * grp) = pack8(vl);
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < NPW; ++i) {
          const int p = wave + kWaves * i, cs = p >> 2, mt = p & 3;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            const int k0 = 16 * kb + 8 * h;
            const u32x4 bv = ld16(sm.VT_hi + (32 * cs + r) * STP + k0);
            const u32x4 ah = ld16(sm.phT_hi + (32 * mt + r) * STP + k0);
            const u32x4 al = ld16(sm.phT_lo + (32 * mt + r) * STP + k0);
            Hreg[i] = DT::mma(ah, bv, Hreg[i]);
            Hreg[i] = DT::mma(al, bv, Hreg[i]);
            if constexpr (DT::kSplit) {
              const u32x4 bvl = ld16(sm.VT_lo + (32 * cs + r) * STP + k0);
              Hreg[i] = DT::mma(ah, bvl, Hreg[i]);
            }
          }
        }
        __syncthreads();
      }
      sm.spart[tg * kD + F] = sacc;
    }
    __syncthreads();
    for (int F = tid; F < kD; F += kThreads)
      sm.s32[F] += (sm.spart[F] + sm.spart[kD + F]) + (sm.spart[2 * kD + F] + sm.spart[3 * kD + F]);
    rebuild_HT();
    __syncthreads();
  }

  // ---- final state
  float* Ho = a.H + (size_t)u * kD * HD;
#pragma unroll
  for (int i = 0; i < NPW; ++i) {
    const int p = wave + kWaves * i, cs = p >> 2, mt = p & 3;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int F = 32 * mt + 8 * (q >> 2) + 4 * h + (q & 3);
      Ho[(size_t)F * HD + 32 * cs + r] = Hreg[i][q];
    }
  }
  for (int F = tid; F < kD; F += kThreads) a.s[(size_t)u * kD + F] = sm.s32[F];
  for (int i = tid; i < gs; i += kThreads) a.finalG[(size_t)u * lam + i] = sm.G[i];
}

template <class DT, int HD>
static hipError_t launch_chain_t(const ChainArgs& a, int U, hipStream_t st) {
  const size_t lds = chain_lds_bytes(a.vr.lam, a.C, HD, DT::kSplit);
  (void)hipFuncSetAttribute((const void*)chain_kernel<DT, HD>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  hipLaunchKernelGGL((chain_kernel<DT, HD>), dim3(U), dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

hipError_t launch_chain(const ChainArgs& a, int U, bool f32, hipStream_t st) {
  if (U <= 0) return hipSuccess;
  if (a.vr.d == 64)
    return f32 ? launch_chain_t<F32, 64>(a, U, st) : launch_chain_t<BF16, 64>(a, U, st);
  return f32 ? launch_chain_t<F32, 128>(a, U, st) : launch_chain_t<BF16, 128>(a, U, st);
}

}  // namespace lola
