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
// error ~1e-8 on these data, far inside the 1e-5 ranking band.  z = phi^T s
// uses the same split on MFMA (s replicated over the 32 rows of a tile).
// The fold multiplies phi (hi + lo) by V (exact in one bf16 operand, or split
// for fp32 inputs) and accumulates into fp32 H.
//
// Layout.  H (D x d, fp32) lives in registers for the whole call in MFMA
// result layout: 32 x 32 tiles (feature block mt, column slab cs), two tiles
// per wave; folds accumulate into them in place.  After each fold H^T is
// rebuilt in LDS as hi/lo planes, the A operand of the next step's SRE GEMM,
// whose (32-candidate tile, column half) work units are spread over the
// eight waves.
#include <type_traits>

#include "internal.h"

namespace lola {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int HTP = kD + 8;   // padded LDS row of H^T (16-bit elements)
constexpr int STP = 64 + 8;   // padded LDS row of fold staging tiles (64 tokens)

// Byte offsets of the LDS arrays (computed by value so that the kernel's
// pointers stay plain LDS pointers).  The candidate list, keys and radix
// histogram of the selection phase share one region with the fold's staging
// tiles, which are live only after the selection.
struct ChainLayout {
  uint32_t HT_hi, HT_lo, s32, s_hi, s_lo, spart, G, Gp, S, misc, kred;
  uint32_t E, keys, hist;                      // selection phase
  uint32_t phT_hi, phT_lo, VT_hi, VT_lo;       // fold phase (same region)
  uint32_t total;
};

__host__ __device__ inline uint32_t align16(uint32_t x) { return (x + 15u) & ~15u; }

__host__ __device__ inline ChainLayout chain_layout(int lam, int C, int d, bool f32) {
  ChainLayout L;
  uint32_t off = 0;
  auto take = [&](uint32_t bytes) { const uint32_t o = off; off = align16(off + bytes); return o; };
  const uint32_t lam1 = lam > 0 ? (uint32_t)lam : 1u;
  L.HT_hi = take((uint32_t)d * HTP * 2);   // [d][HTP]
  L.HT_lo = take((uint32_t)d * HTP * 2);
  L.s32 = take(kD * 4);                    // [kD]
  L.s_hi = take(kD * 2);                   // s split into 16-bit hi / lo
  L.s_lo = take(kD * 2);
  L.spart = take((kThreads / kD) * kD * 4);
  L.G = take(lam1 * 4);                    // cache (virtual indices)
  L.Gp = take(lam1 * 4);                   // cache positions
  L.S = take((uint32_t)C * 4);             // folded list (<= C per step)
  L.misc = take(16 * 4);
  L.kred = take(2 * kWaves * 8);           // per-wave key min / max
  const uint32_t region = off;
  L.E = take((uint32_t)(lam + C) * 4);     // candidates (virtual indices)
  L.keys = take((uint32_t)(lam + C) * 8);  // SRE partials, then keys
  L.hist = take(2048 * 4);                 // radix histogram
  const uint32_t sel_end = off;
  off = region;
  L.phT_hi = take(kD * STP * 2);           // [kD][STP]
  L.phT_lo = take(kD * STP * 2);
  L.VT_hi = take((uint32_t)d * STP * 2);   // [d][STP]
  L.VT_lo = take(f32 ? (uint32_t)d * STP * 2 : 16);
  L.total = off > sel_end ? off : sel_end;
  return L;
}

// Workgroup barrier that orders LDS only.  Inside this kernel no thread reads
// global memory written by another thread, so pending global stores (the
// per-chunk snapshots) need not drain at every barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace

size_t chain_lds_bytes(int lam, int C, int d, bool f32) {
  return chain_layout(lam, C, d, f32).total;
}

template <class DT, int HD>
__global__ __launch_bounds__(kThreads) void chain_kernel(ChainArgs a) {
  using T = typename DT::T;
  constexpr int NSLAB = HD / 32;                  // column slabs of H
  constexpr int NPW = NSLAB * 4 / kWaves;         // H tiles per wave (2 or 4)
  const VirtRows vr = a.vr;
  const int lam = vr.lam, eta = vr.eta;
  const int u = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, r = lane & 31;

  extern __shared__ __align__(16) unsigned char smem[];
  const ChainLayout L = chain_layout(lam, a.C, HD, DT::kSplit);
  struct {
    uint16_t *HT_hi, *HT_lo;
    float* s32;
    uint16_t *s_hi, *s_lo;
    float* spart;
    int32_t *G, *Gp, *S, *misc;
    uint64_t* kred;
    int32_t* E;
    uint64_t* keys;
    int32_t* hist;
    uint16_t *phT_hi, *phT_lo, *VT_hi, *VT_lo;
  } sm = {(uint16_t*)(smem + L.HT_hi), (uint16_t*)(smem + L.HT_lo), (float*)(smem + L.s32),
          (uint16_t*)(smem + L.s_hi), (uint16_t*)(smem + L.s_lo), (float*)(smem + L.spart),
          (int32_t*)(smem + L.G), (int32_t*)(smem + L.Gp), (int32_t*)(smem + L.S),
          (int32_t*)(smem + L.misc), (uint64_t*)(smem + L.kred), (int32_t*)(smem + L.E),
          (uint64_t*)(smem + L.keys), (int32_t*)(smem + L.hist), (uint16_t*)(smem + L.phT_hi),
          (uint16_t*)(smem + L.phT_lo), (uint16_t*)(smem + L.VT_hi), (uint16_t*)(smem + L.VT_lo)};

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
  for (int i = tid; i < gs0; i += kThreads) {
    sm.G[i] = i;
    sm.Gp[i] = vr.cache_pos[(size_t)u * lam + i];
  }

  auto rebuild_HT = [&]() {
    for (int F = tid; F < kD; F += kThreads) {
      uint32_t hi, lo;
      DT::split(sm.s32[F], hi, lo);
      sm.s_hi[F] = (uint16_t)hi;
      sm.s_lo[F] = (uint16_t)lo;
    }
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
  lds_barrier();

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
      for (int i = tid; i < nL; i += kThreads) {
        sm.G[gs + i] = vi_L0 + i;
        sm.Gp[gs + i] = (int32_t)(lo_p + i);
      }
      gs = nE;
      lds_barrier();
      continue;
    }
    for (int i = tid; i < nE; i += kThreads) sm.E[i] = i < gs ? sm.G[i] : vi_L0 + (i - gs);
    for (int i = tid; i < 2048; i += kThreads) sm.hist[i] = 0;
    lds_barrier();

    // ---- 4a. SRE of every candidate, 32-row tiles over the waves.  All of a
    // tile's operand loads are issued first (one memory latency per tile);
    // the output columns are done in two halves to bound registers.
    // Work unit = (32-candidate tile, half of the d columns): partial SRE of
    // the half, z recomputed per unit.  Two waves per SIMD hide each other's
    // load latency.  The two partials meet in the 64-bit key slot of e.
    constexpr int NH = NSLAB / 2;                  // 32-column tiles per half
    const int nunits = lam > 0 ? ((nE + 31) / 32) * 2 : 0;
    for (int wu = wave; wu < nunits; wu += kWaves) {
      const int t = wu >> 1, half = wu & 1;
      const int e = t * 32 + r;
      const bool ev = e < nE;
      const int vi = ev ? sm.E[e] : sm.E[0];
      const T* vrow = reinterpret_cast<const T*>(vr.vrow(u, vi, sizeof(T))) + 4 * h + 32 * NH * half;
      const uint16_t* ph = a.phi_hi + phi_unit + (size_t)vi * kD + 8 * h;
      const uint16_t* pl = a.phi_lo + phi_unit + (size_t)vi * kD + 8 * h;
      u32x4 bh[8], bl[8];
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) { bh[kb] = ld16(ph + 16 * kb); bl[kb] = ld16(pl + 16 * kb); }
      using VRaw = typename std::conditional<DT::kSplit, f32x4, u32x2>::type;
      VRaw vraw[NH][4];
#pragma unroll
      for (int mt = 0; mt < NH; ++mt)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          vraw[mt][g4] = *reinterpret_cast<const VRaw*>(vrow + 32 * mt + 8 * g4);
      // P^T (this half's columns) and z = phi^T s (s replicated over the 32
      // rows of an A operand): NH + 1 independent accumulators, pass-major.
      f32x16 P[NH], Z;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        Z[q] = 0.f;
#pragma unroll
        for (int mt = 0; mt < NH; ++mt) P[mt][q] = 0.f;
      }
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        const int k0 = kb * 16 + 8 * h;
        u32x4 ah[NH], al[NH];
#pragma unroll
        for (int mt = 0; mt < NH; ++mt) {
          const int row = 32 * (NH * half + mt) + r;
          ah[mt] = ld16(sm.HT_hi + row * HTP + k0);
          al[mt] = ld16(sm.HT_lo + row * HTP + k0);
        }
        const u32x4 zh = ld16(sm.s_hi + k0), zl = ld16(sm.s_lo + k0);
#pragma unroll
        for (int mt = 0; mt < NH; ++mt) P[mt] = DT::mma(ah[mt], bh[kb], P[mt]);
        Z = DT::mma(zh, bh[kb], Z);
#pragma unroll
        for (int mt = 0; mt < NH; ++mt) P[mt] = DT::mma(al[mt], bh[kb], P[mt]);
        Z = DT::mma(zl, bh[kb], Z);
#pragma unroll
        for (int mt = 0; mt < NH; ++mt) P[mt] = DT::mma(ah[mt], bl[kb], P[mt]);
        Z = DT::mma(zh, bl[kb], Z);
      }
      const float z = Z[0];
      const float iz = z > 0.f ? 1.f / z : 0.f;   // z == 0: prediction 0
      float acc = 0.f;
#pragma unroll
      for (int mt = 0; mt < NH; ++mt)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          float vv[4];
          if constexpr (DT::kSplit) {
#pragma unroll
            for (int q = 0; q < 4; ++q) vv[q] = vraw[mt][g4][q];
          } else {
            const u32x2 x = vraw[mt][g4];
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
      if (ev && h == 0) reinterpret_cast<float*>(sm.keys)[2 * e + 1 - half] = acc;
    }
    lds_barrier();
    // keys = (SRE bits << 32) | (0xFFFFFFFF - position); SRE = half 0 + half 1
    uint64_t kmin = ~0ull, kmax = 0;
    for (int e = tid; lam > 0 && e < nE; e += kThreads) {
      const float* pp = reinterpret_cast<const float*>(sm.keys) + 2 * e;
      const float sre = pp[1] + pp[0];             // column halves 0 and 1
      const uint32_t pos = e < gs ? (uint32_t)sm.Gp[e] : (uint32_t)(lo_p + (e - gs));
      const uint64_t key = ((uint64_t)__float_as_uint(sre) << 32) | (uint64_t)(0xFFFFFFFFu - pos);
      sm.keys[e] = key;
      kmin = key < kmin ? key : kmin;
      kmax = key > kmax ? key : kmax;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const uint64_t a1 = __shfl_xor(kmin, o, 64), a2 = __shfl_xor(kmax, o, 64);
      kmin = a1 < kmin ? a1 : kmin;
      kmax = a2 > kmax ? a2 : kmax;
    }
    if (lane == 0) { sm.kred[2 * wave] = kmin; sm.kred[2 * wave + 1] = kmax; }
    lds_barrier();
    if (a.dbg_keys) {
      uint64_t* dk = a.dbg_keys + ((size_t)u * a.nch + j) * (lam + a.C);
      for (int e = tid; e < nE; e += kThreads) dk[e] = sm.keys[e];
    }

    // ---- 4b. exact top-lam: radix select of the lam-th largest key with
    // 11-bit digits, starting at the highest bit where the keys differ (one
    // pass separates a few hundred keys in most steps).  lam == 0: nothing
    // is kept.  Thread t owns 2048 / kThreads bins.
    uint64_t prefix = 0, mask = 0;
    if (lam > 0) {
      kmin = sm.kred[0];
      kmax = sm.kred[1];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) {
        kmin = sm.kred[2 * w] < kmin ? sm.kred[2 * w] : kmin;
        kmax = sm.kred[2 * w + 1] > kmax ? sm.kred[2 * w + 1] : kmax;
      }
      // keys are unique, so kmin != kmax; bits above `top` are common
      const int top = 63 - __clzll((long long)(kmin ^ kmax));
      mask = top >= 63 ? 0 : (~0ull << (top + 1));
      prefix = kmin & mask;
      int shift = top - 10 > 0 ? top - 10 : 0;
      int need = lam;
      for (;;) {
        for (int e = tid; e < nE; e += kThreads) {
          const uint64_t k = sm.keys[e];
          if ((k & mask) == prefix) atomicAdd(&sm.hist[(k >> shift) & 2047], 1);
        }
        lds_barrier();
        // thread t owns bins [BPT (T-1-t), BPT (T-1-t) + BPT): scanning the
        // threads in order walks the bins from the top down
        constexpr int BPT = 2048 / kThreads;
        const int b0 = BPT * (kThreads - 1 - tid);
        int cnt[BPT], tot = 0;
#pragma unroll
        for (int q = 0; q < BPT; ++q) { cnt[q] = sm.hist[b0 + q]; tot += cnt[q]; }
        const int incl = wave_incl_scan(tot);
        if (lane == 63) sm.misc[8 + wave] = incl;
        lds_barrier();
        int above = incl - tot;
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
          if (w < wave) above += sm.misc[8 + w];
#pragma unroll
        for (int q = BPT - 1; q >= 0; --q) {
          if (above < need && need <= above + cnt[q]) {
            sm.misc[0] = b0 + q;
            sm.misc[1] = need - above;
            sm.misc[2] = cnt[q];
          }
          above += cnt[q];
        }
        lds_barrier();
        const int bsel = sm.misc[0], cb = sm.misc[2];
        need = sm.misc[1];
        prefix |= (uint64_t)bsel << shift;
        mask |= (uint64_t)2047 << shift;
        if (cb == need || shift == 0) break;
        shift = shift >= 11 ? shift - 11 : 0;
        lds_barrier();   // every thread has read misc before it changes
        for (int i = tid; i < 2048; i += kThreads) sm.hist[i] = 0;
        lds_barrier();
      }
    }

    // ---- 4c. stable compaction: kept -> G (E order), rest -> S.  Wave w
    // takes a contiguous range of E; ballots give the in-wave positions.
    {
      const int seg = ((nE + kWaves - 1) / kWaves + 63) / 64 * 64;
      const int e0 = wave * seg, e1 = min(nE, e0 + seg);
      int kept = 0;
      for (int base = e0; base < e1; base += 64) {
        const int e = base + lane;
        const bool kp = e < e1 && lam > 0 && (sm.keys[e] & mask) >= prefix;
        kept += __popcll(__ballot(kp));
      }
      if (lane == 0) sm.misc[8 + wave] = kept;
      lds_barrier();
      int kb = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w)
        if (w < wave) kb += sm.misc[8 + w];
      for (int base = e0; base < e1; base += 64) {
        const int e = base + lane;
        const bool in = e < e1;
        const bool kp = in && lam > 0 && (sm.keys[e] & mask) >= prefix;
        const unsigned long long bk = __ballot(kp);
        const int before = __popcll(bk & ((1ull << lane) - 1ull));
        if (kp) {
          if (kb + before < lam) {
            sm.G[kb + before] = sm.E[e];
            sm.Gp[kb + before] = (int32_t)(0xFFFFFFFFu - (uint32_t)sm.keys[e]);
          }
        }
        else if (in) {
          const int sidx = e - (kb + before);
          if (sidx < nE - lam) sm.S[sidx] = sm.E[e];
        }
        kb += __popcll(bk);
      }
    }
    gs = lam;
    lds_barrier();

    // ---- 4d. fold the rest into H (MFMA) and s, 64 tokens per block.  The
    // gather is by rows: lane = token, wave = feature / column chunks, with
    // 16-byte loads; the tiles are written transposed (token-contiguous) for
    // the MFMA operands.
    const int nS = nE - lam;
    float sacc = 0.f;
    for (int sb = 0; sb < nS; sb += 64) {
      const int tok = sb + lane;
      const bool tv = tok < nS;
      const int vi = tv ? sm.S[tok] : 0;
      {
        // phi: 16 chunks of 8 features, two per wave
        constexpr int FCW = 16 / kWaves;                 // 8-feature chunks per wave
        u32x4 xh[FCW], xl[FCW];
#pragma unroll
        for (int q = 0; q < FCW; ++q) {
          const int f0 = 8 * (FCW * wave + q);
          xh[q] = tv ? ld16(a.phi_hi + phi_unit + (size_t)vi * kD + f0) : u32x4{0, 0, 0, 0};
          xl[q] = tv ? ld16(a.phi_lo + phi_unit + (size_t)vi * kD + f0) : u32x4{0, 0, 0, 0};
        }
        // V: HD / 8 columns per wave
        constexpr int VC = HD / kWaves;                  // 16 or 8 columns
        float vx[VC];
        {
          const T* vrow = reinterpret_cast<const T*>(vr.vrow(u, vi, sizeof(T))) + VC * wave;
#pragma unroll
          for (int q8 = 0; q8 < VC; q8 += 8) {
            float x[8];
            if (tv) load8_f32(vrow + q8, x);
            else for (int q = 0; q < 8; ++q) x[q] = 0.f;
#pragma unroll
            for (int q = 0; q < 8; ++q) vx[q8 + q] = x[q];
          }
        }
#pragma unroll
        for (int q = 0; q < FCW; ++q) {
          const int f0 = 8 * (FCW * wave + q);
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            sm.phT_hi[(f0 + 2 * w) * STP + lane] = (uint16_t)(xh[q][w] & 0xFFFFu);
            sm.phT_hi[(f0 + 2 * w + 1) * STP + lane] = (uint16_t)(xh[q][w] >> 16);
            sm.phT_lo[(f0 + 2 * w) * STP + lane] = (uint16_t)(xl[q][w] & 0xFFFFu);
            sm.phT_lo[(f0 + 2 * w + 1) * STP + lane] = (uint16_t)(xl[q][w] >> 16);
          }
        }
#pragma unroll
        for (int q = 0; q < VC; ++q) {
          uint32_t hi, lo;
          DT::split(vx[q], hi, lo);
          sm.VT_hi[(VC * wave + q) * STP + lane] = (uint16_t)hi;
          if constexpr (DT::kSplit) sm.VT_lo[(VC * wave + q) * STP + lane] = (uint16_t)lo;
        }
      }
      lds_barrier();
      {
        // s partial sums: feature F, 64 / NPART tokens per part, fixed order
        const int F = tid % kD, qt = tid / kD;
        constexpr int TPP = 64 / (kThreads / kD);
        float part = 0.f;
#pragma unroll
        for (int q = 0; q < TPP; ++q)
          part += DT::from_bits(sm.phT_hi[F * STP + TPP * qt + q]) +
                  DT::from_bits(sm.phT_lo[F * STP + TPP * qt + q]);
        sacc += part;
      }
      const int nkb = min(4, (nS - sb + 15) / 16);
      for (int kb = 0; kb < nkb; ++kb) {
        const int k0 = 16 * kb + 8 * h;
        u32x4 bv[NPW], ah[NPW], al[NPW];
#pragma unroll
        for (int i = 0; i < NPW; ++i) {
          const int p = wave + kWaves * i, cs = p >> 2, mt = p & 3;
          bv[i] = ld16(sm.VT_hi + (32 * cs + r) * STP + k0);
          ah[i] = ld16(sm.phT_hi + (32 * mt + r) * STP + k0);
          al[i] = ld16(sm.phT_lo + (32 * mt + r) * STP + k0);
        }
#pragma unroll
        for (int i = 0; i < NPW; ++i) Hreg[i] = DT::mma(ah[i], bv[i], Hreg[i]);
#pragma unroll
        for (int i = 0; i < NPW; ++i) Hreg[i] = DT::mma(al[i], bv[i], Hreg[i]);
        if constexpr (DT::kSplit) {
#pragma unroll
          for (int i = 0; i < NPW; ++i) {
            const int p = wave + kWaves * i, cs = p >> 2;
            Hreg[i] = DT::mma(ah[i], ld16(sm.VT_lo + (32 * cs + r) * STP + k0), Hreg[i]);
          }
        }
      }
      lds_barrier();
    }
    sm.spart[(tid / kD) * kD + tid % kD] = sacc;
    lds_barrier();
    for (int F = tid; F < kD; F += kThreads) {
      float add = 0.f;
#pragma unroll
      for (int q = 0; q < kThreads / kD; ++q) add += sm.spart[q * kD + F];
      sm.s32[F] += add;
    }
    rebuild_HT();
    lds_barrier();
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
