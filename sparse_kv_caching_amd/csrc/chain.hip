// K2: LoLA's serial memory-allocation chain, one step per chunk, one
// workgroup per unit (b, KV head).
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
// error ~1e-8 on these data, far inside the 1e-5 ranking band.  z = phi^T s
// uses the same split on MFMA (s replicated over the 32 rows of a tile).  The
// fold multiplies phi (hi + lo) by V (exact in one bf16 operand, or split for
// fp32 inputs) and accumulates into fp32 H.
//
// Layout.  Wave w keeps columns [32w, 32w + 32) of H in registers in MFMA
// result layout for the whole call (folds accumulate into them in place).
// After each fold H^T is rebuilt in LDS as hi/lo bf16 planes, the A operand
// of the next step's SRE GEMM, whose row tiles (32 candidates) are spread
// over all four waves.
#include "internal.h"

namespace lola {

namespace {

constexpr int kThreads = 256;
constexpr int HTP = kD + 8;   // padded LDS row of H^T (bf16 elements)
constexpr int STP = 32 + 8;   // padded LDS row of fold staging tiles

struct ChainSmem {
  uint16_t* HT_hi;   // [d][HTP]
  uint16_t* HT_lo;
  float* s32;        // [kD]
  uint16_t* s_hi;    // [kD]
  uint16_t* s_lo;
  float* spart;      // [2][kD]
  int32_t* G;        // [lam]
  int32_t* E;        // [lam + C]
  int32_t* S;        // [C + lam]   folded list
  uint64_t* keys;    // [lam + C]
  int32_t* hist;     // [256]
  int32_t* misc;     // [16]
  uint16_t* phT_hi;  // [kD][STP]
  uint16_t* phT_lo;
  uint16_t* VT_hi;   // [d][STP]
  uint16_t* VT_lo;
};

__host__ __device__ inline size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }

__host__ __device__ inline size_t carve(int lam, int C, int d, bool f32, unsigned char* base,
                                        ChainSmem* sm) {
  size_t off = 0;
  auto take = [&](size_t bytes) -> unsigned char* {
    unsigned char* p = base ? base + off : nullptr;
    off = align16(off + bytes);
    return p;
  };
  ChainSmem t;
  t.HT_hi = (uint16_t*)take((size_t)d * HTP * 2);
  t.HT_lo = (uint16_t*)take((size_t)d * HTP * 2);
  t.s32 = (float*)take(kD * 4);
  t.s_hi = (uint16_t*)take(kD * 2);
  t.s_lo = (uint16_t*)take(kD * 2);
  t.spart = (float*)take(2 * kD * 4);
  t.G = (int32_t*)take((size_t)(lam > 0 ? lam : 1) * 4);
  t.E = (int32_t*)take((size_t)(lam + C) * 4);
  t.S = (int32_t*)take((size_t)(lam + C) * 4);
  t.keys = (uint64_t*)take((size_t)(lam + C) * 8);
  t.hist = (int32_t*)take(256 * 4);
  t.misc = (int32_t*)take(16 * 4);
  t.phT_hi = (uint16_t*)take((size_t)kD * STP * 2);
  t.phT_lo = (uint16_t*)take((size_t)kD * STP * 2);
  t.VT_hi = (uint16_t*)take((size_t)d * STP * 2);
  t.VT_lo = (uint16_t*)take(f32 ? (size_t)d * STP * 2 : 16);
  if (sm) *sm = t;
  return off;
}


// exclusive scan of one int per thread over the block
__device__ __forceinline__ int block_excl_scan(int x, int32_t* wsum, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = wave_incl_scan(x);
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int off = 0, tot = 0;
  for (int w = 0; w < kThreads / 64; ++w) {
    int v = wsum[w];
    if (w < wave) off += v;
    tot += v;
  }
  total = tot;
  __syncthreads();
  return off + incl - x;
}

}  // namespace

size_t chain_lds_bytes(int lam, int C, int d, bool f32) {
  return carve(lam, C, d, f32, nullptr, nullptr);
}

template <class DT>
__global__ __launch_bounds__(kThreads) void chain_kernel(ChainArgs a) {
  using T = typename DT::T;
  const VirtRows& vr = a.vr;
  const int d = vr.d, lam = vr.lam, eta = vr.eta;
  const int u = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, r = lane & 31;
  const int nslab = d / 32;
  const bool has_slab = wave < nslab;

  extern __shared__ __align__(16) unsigned char smem[];
  ChainSmem sm;
  carve(lam, a.C, d, DT::kSplit, smem, &sm);

  // ---- load state: H columns [32w, 32w+32) into registers (result layout)
  f32x16 Hreg[4];
  const float* Hg = a.H + (size_t)u * kD * d;
  for (int mt = 0; mt < 4; ++mt)
    for (int i = 0; i < 16; ++i) {
      const int F = 32 * mt + 8 * (i >> 2) + 4 * h + (i & 3);
      Hreg[mt][i] = has_slab ? Hg[(size_t)F * d + 32 * wave + r] : 0.f;
    }
  for (int F = tid; F < kD; F += kThreads) sm.s32[F] = a.s[(size_t)u * kD + F];
  const long long n0 = vr.n0;
  const int gs0 = (int)min((long long)lam, max(0LL, n0 - eta));
  for (int i = tid; i < gs0; i += kThreads) sm.G[i] = i;

  auto rebuild_operands = [&]() {
    if (has_slab) {
      const int c = 32 * wave + r;
      for (int mt = 0; mt < 4; ++mt)
        for (int g4 = 0; g4 < 4; ++g4) {
          const int F = 32 * mt + 8 * g4 + 4 * h;
          uint32_t hi[4], lo[4];
          for (int j = 0; j < 4; ++j) DT::split(Hreg[mt][4 * g4 + j], hi[j], lo[j]);
          u32x2 w;
          w[0] = hi[0] | (hi[1] << 16); w[1] = hi[2] | (hi[3] << 16);
          *reinterpret_cast<u32x2*>(sm.HT_hi + c * HTP + F) = w;
          w[0] = lo[0] | (lo[1] << 16); w[1] = lo[2] | (lo[3] << 16);
          *reinterpret_cast<u32x2*>(sm.HT_lo + c * HTP + F) = w;
        }
    }
    for (int F = tid; F < kD; F += kThreads) {
      uint32_t hi, lo;
      DT::split(sm.s32[F], hi, lo);
      sm.s_hi[F] = (uint16_t)hi;
      sm.s_lo[F] = (uint16_t)lo;
    }
  };
  __syncthreads();
  rebuild_operands();
  __syncthreads();

  int gs = gs0;
  const size_t phi_unit = (size_t)u * a.NV * kD;
  for (int j = 0; j < a.nch; ++j) {
    const long long nj = n0 + (long long)j * a.C;
    const int c = min(a.C, vr.T - j * a.C);

    // ---- 1. snapshot (H_j^T hi/lo, s_j, G_j)
    {
      uint16_t* dst = a.snapHT + ((size_t)u * a.nch + j) * 2 * d * kD;
      const int chunks = d * (kD / 8);  // 16-byte pieces per plane
      for (int i = tid; i < 2 * chunks; i += kThreads) {
        const int pl = i / chunks, rem = i % chunks;
        const int row = rem / (kD / 8), col = (rem % (kD / 8)) * 8;
        const uint16_t* src = (pl ? sm.HT_lo : sm.HT_hi) + row * HTP + col;
        *reinterpret_cast<u32x4*>(dst + (size_t)pl * d * kD + row * kD + col) =
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

    // ---- 4a. SRE of every candidate, 32-row tiles over the four waves
    for (int t = wave; lam > 0 && t * 32 < nE; t += kThreads / 64) {
      const int e = t * 32 + r;
      const bool ev = e < nE;
      const int vi = ev ? sm.E[e] : 0;
      const uint16_t* ph = a.phi_hi + phi_unit + (size_t)vi * kD;
      const uint16_t* pl = a.phi_lo + phi_unit + (size_t)vi * kD;
      f32x16 P[4], Z;
      for (int i = 0; i < 16; ++i) { Z[i] = 0.f; for (int mt = 0; mt < 4; ++mt) P[mt][i] = 0.f; }
      for (int kb = 0; kb < kD / 16; ++kb) {
        const int k0 = kb * 16 + 8 * h;
        u32x4 bh, bl;
        if (ev) { bh = ld16(ph + k0); bl = ld16(pl + k0); }
        else { bh = u32x4{0, 0, 0, 0}; bl = bh; }
        const u32x4 zh = ld16(sm.s_hi + k0), zl = ld16(sm.s_lo + k0);
        Z = DT::mma(zh, bh, Z);
        Z = DT::mma(zh, bl, Z);
        Z = DT::mma(zl, bh, Z);
        for (int mt = 0; mt < nslab; ++mt) {
          const int row = 32 * mt + r;
          const u32x4 ah = ld16(sm.HT_hi + row * HTP + k0);
          const u32x4 al = ld16(sm.HT_lo + row * HTP + k0);
          P[mt] = DT::mma(ah, bh, P[mt]);
          P[mt] = DT::mma(ah, bl, P[mt]);
          P[mt] = DT::mma(al, bh, P[mt]);
        }
      }
      const float z = Z[0];
      const float iz = z > 0.f ? 1.f / z : 0.f;
      float acc = 0.f;
      if (ev) {
        const T* vrow = reinterpret_cast<const T*>(vr.vrow(u, vi, sizeof(T)));
        for (int mt = 0; mt < nslab; ++mt)
          for (int g4 = 0; g4 < 4; ++g4) {
            const int cc = 32 * mt + 8 * g4 + 4 * h;
            float vv[4];
            if constexpr (DT::kSplit) {
              f32x4 x = *reinterpret_cast<const f32x4*>(vrow + cc);
              for (int q = 0; q < 4; ++q) vv[q] = x[q];
            } else {
              u32x2 x = *reinterpret_cast<const u32x2*>(vrow + cc);
              vv[0] = __uint_as_float(x[0] << 16); vv[1] = __uint_as_float(x[0] & 0xFFFF0000u);
              vv[2] = __uint_as_float(x[1] << 16); vv[3] = __uint_as_float(x[1] & 0xFFFF0000u);
            }
            for (int q = 0; q < 4; ++q) {
              const float p = z > 0.f ? P[mt][4 * g4 + q] * iz : 0.f;
              const float df = p - vv[q];
              acc = fmaf(df, df, acc);
            }
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
        for (int b = 0; b < 4; ++b) { cnt[b] = sm.hist[4 * lane + b]; tot += cnt[b]; }
        const int incl = wave_incl_scan(tot);
        const int all = __shfl(incl, 63, 64);
        int above = all - incl;            // elements in bins above this lane's four
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
      int total;
      int kb = block_excl_scan(kept, sm.misc + 4, total);
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
      const int F = tid % kD, tg = tid / kD;   // tg in {0, 1}
      for (int sb = 0; sb < nS; sb += 32) {
        // stage Phi_S^T (hi / lo) and V_S^T for 32 tokens
        {
          uint32_t hb[8], lb[8];
          for (int half = 0; half < 2; ++half) {
            for (int q = 0; q < 8; ++q) {
              const int tok = sb + 16 * tg + 8 * half + q;
              if (tok < nS) {
                const size_t o = phi_unit + (size_t)sm.S[tok] * kD + F;
                hb[q] = a.phi_hi[o];
                lb[q] = a.phi_lo[o];
                sacc += DT::from_bits(hb[q]) + DT::from_bits(lb[q]);
              } else {
                hb[q] = 0; lb[q] = 0;
              }
            }
            const int col = 16 * tg + 8 * half;
            *reinterpret_cast<u32x4*>(sm.phT_hi + F * STP + col) = pack8(hb);
            *reinterpret_cast<u32x4*>(sm.phT_lo + F * STP + col) = pack8(lb);
          }
        }
        {
          // V_S^T: d columns x 32 tokens; 256 threads cover d * 4 groups of 8
          for (int it = tid; it < d * 4; it += kThreads) {
            const int cc = it % d, grp = it / d;
            uint32_t vh[8], vl[8];
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
        }
        __syncthreads();
        if (has_slab) {
          for (int kb = 0; kb < 2; ++kb) {
            const int k0 = 16 * kb + 8 * h;
            const u32x4 bv = ld16(sm.VT_hi + (32 * wave + r) * STP + k0);
            u32x4 bvl;
            if constexpr (DT::kSplit) bvl = ld16(sm.VT_lo + (32 * wave + r) * STP + k0);
            for (int mt = 0; mt < 4; ++mt) {
              const u32x4 ah = ld16(sm.phT_hi + (32 * mt + r) * STP + k0);
              const u32x4 al = ld16(sm.phT_lo + (32 * mt + r) * STP + k0);
              Hreg[mt] = DT::mma(ah, bv, Hreg[mt]);
              Hreg[mt] = DT::mma(al, bv, Hreg[mt]);
              if constexpr (DT::kSplit) Hreg[mt] = DT::mma(ah, bvl, Hreg[mt]);
            }
          }
        }
        __syncthreads();
      }
      sm.spart[tg * kD + F] = sacc;
    }
    __syncthreads();
    for (int F = tid; F < kD; F += kThreads) sm.s32[F] += sm.spart[F] + sm.spart[kD + F];
    __syncthreads();
    rebuild_operands();
    __syncthreads();
  }

  // ---- final state
  if (has_slab) {
    float* Ho = a.H + (size_t)u * kD * d;
    for (int mt = 0; mt < 4; ++mt)
      for (int i = 0; i < 16; ++i) {
        const int F = 32 * mt + 8 * (i >> 2) + 4 * h + (i & 3);
        Ho[(size_t)F * d + 32 * wave + r] = Hreg[mt][i];
      }
  }
  for (int F = tid; F < kD; F += kThreads) a.s[(size_t)u * kD + F] = sm.s32[F];
  for (int i = tid; i < gs; i += kThreads) a.finalG[(size_t)u * lam + i] = sm.G[i];
}

hipError_t launch_chain(const ChainArgs& a, int U, bool f32, hipStream_t st) {
  if (U <= 0) return hipSuccess;
  size_t lds = chain_lds_bytes(a.vr.lam, a.C, a.vr.d, f32);
  if (f32) {
    (void)hipFuncSetAttribute((const void*)chain_kernel<F32>,
                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL(chain_kernel<F32>, dim3(U), dim3(kThreads), lds, st, a);
  } else {
    (void)hipFuncSetAttribute((const void*)chain_kernel<BF16>,
                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL(chain_kernel<BF16>, dim3(U), dim3(kThreads), lds, st, a);
  }
  return hipGetLastError();
}

}  // namespace lola
