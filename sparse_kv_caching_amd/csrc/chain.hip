// K2: LoLA's serial memory-allocation chain, one step per chunk.  A unit
// (b, KV head) is processed by k cooperating workgroups (k = 1, 2 or 4, so
// that every workgroup of the grid is resident at once); workgroup r owns
// SPW = (d / 32) / k column slabs of H.
//
// Per chunk j (LoLA notes §2.6, Eq. (15); §2.4, Eqs. (11)-(13)):
//   1. snapshot (H_j, s_j, G_j): the state the chunk's queries read (each
//      workgroup writes its columns of H_j^T);
//   2. candidates E = G_j ++ L_j, L_j = positions leaving the window;
//   3. if |E| <= lam: G_{j+1} = E (keep all);
//   4. else the SRE of every candidate against (H_j, s_j) (notes §2.3,
//      Eq. (10), squared): each workgroup computes the part of the squared
//      error over its own columns, the parts are exchanged through global
//      memory, and every workgroup forms the same keys and runs the same
//      exact top-lam selection (SRE desc, position asc) and stable
//      compaction; each folds the rest into its own columns of H
//      (H += Phi_S^T V_S) and updates s += sum phi (all of s, everywhere).
//
// The SRE of a candidate is the sum of its per-slab parts, always added in
// slab order, so the keys (and the whole chain) are bitwise the same for
// every k.
//
// Precision.  SRE decides an integer (cache membership), so the GEMM
// p = H^T phi runs as a three-pass 16-bit split (hi*hi + hi*lo + lo*hi, fp32
// accumulation; bf16 halves for bf16 inputs, fp16 for fp32 inputs) with
// relative error ~1e-6 or better, inside the 1e-5 ranking band; z = phi^T s
// is an fp32 dot product of the same split phi.  The fold multiplies phi
// (hi + lo) by V (exact in one bf16 operand, or split for fp32 inputs) and
// accumulates into fp32 H.
//
// Layout.  A workgroup's H columns live in registers for the whole call in
// MFMA result layout (32 x 32 tiles (feature block mt, slab)); folds
// accumulate into them in place.  After each fold the columns are written to
// LDS as H^T hi/lo rows, from which every wave loads its slab's A operands of
// the next SRE GEMM once per step.
//
// Work split.  A unit's k workgroups form NG = (d / 32) / SPW slab groups
// times CS candidate groups: workgroup (g, ch) owns the columns of slab group
// g and scores the candidate tiles t with t % CS == ch.  The CS workgroups of
// one slab group hold the same columns and apply the same fold.
//
// Segments.  A launch runs steps j0 .. j1 - 1; the state between segments
// is H and s in global memory and the cache list (virtual rows) in finalG,
// and the exchange tags continue over the call (xstep0), so that the
// attention of finished chunks can run beside the rest of the chain.
//
// Exchange.  Every (slab, candidate) part is written as one 64-bit word
// (value, step tag) with an agent-scope relaxed atomic store (it bypasses the
// non-coherent caches); a reader polls each word with agent-scope atomic
// loads until its tag is the current step's, bounded (a lost partner sets an
// error flag and ends the chain instead of hanging).  Tags are the step
// number + 1 and the buffer is zeroed before every call; parts are
// double-buffered by the parity of the exchange step (a workgroup can only
// write step x + 2 after every partner has published step x + 1, which each
// does after reading step x).
#include <type_traits>

#include "internal.h"

namespace lola {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int HTP = kD + 8;   // padded LDS row of H^T (16-bit elements)
constexpr int STP = 64 + 8;   // padded LDS row of fold staging tiles (64 tokens)
constexpr int kSpinLimit = 1 << 22;   // counter polls before an exchange is declared lost

// Byte offsets of the LDS arrays (computed by value so that the kernel's
// pointers stay plain LDS pointers).  The candidate list, parts, keys and
// radix histogram of the selection phase share one region with the fold's
// staging tiles, which are live only after the selection.
struct ChainLayout {
  uint32_t HT_hi, HT_lo, s32, spart, G, Gp, S, misc, kred;
  uint32_t E, part, keys, hist;                // selection phase
  uint32_t phT_hi, phT_lo, VT_hi, VT_lo;       // fold phase (same region)
  uint32_t total;
};

__host__ __device__ inline uint32_t align16(uint32_t x) { return (x + 15u) & ~15u; }

__host__ __device__ inline ChainLayout chain_layout(int lam, int C, int spw, bool f32) {
  ChainLayout L;
  uint32_t off = 0;
  auto take = [&](uint32_t bytes) { const uint32_t o = off; off = align16(off + bytes); return o; };
  const uint32_t lam1 = lam > 0 ? (uint32_t)lam : 1u;
  const uint32_t ncol = 32u * (uint32_t)spw;   // H columns of the workgroup
  const uint32_t le = (uint32_t)(lam + C);     // candidates per step, at most
  L.HT_hi = take(ncol * HTP * 2);          // [ncol][HTP]
  L.HT_lo = take(ncol * HTP * 2);
  L.s32 = take(kD * 4);                    // [kD]
  L.spart = take((kThreads / kD) * kD * 4);
  L.G = take(lam1 * 4);                    // cache (virtual indices)
  L.Gp = take(lam1 * 4);                   // cache positions
  L.S = take((uint32_t)C * 4);             // folded list (<= C per step)
  L.misc = take(20 * 4);                   // [8..15] per wave, [16] abort
  L.kred = take(2 * kWaves * 8);           // per-wave key min / max
  const uint32_t region = off;
  L.E = take(le * 4);                      // candidates (virtual indices)
  L.part = take((uint32_t)spw * le * 4);   // [slab][candidate] SRE parts
  L.keys = take(le * 8);
  L.hist = take(768 * 4);                  // three radix histograms
  const uint32_t sel_end = off;
  off = region;
  L.phT_hi = take(kD * STP * 2);           // [kD][STP]
  L.phT_lo = take(kD * STP * 2);
  L.VT_hi = take(ncol * STP * 2);          // [ncol][STP]
  L.VT_lo = take(f32 ? ncol * STP * 2 : 16);
  L.total = off > sel_end ? off : sel_end;
  return L;
}

// Workgroup barrier that orders LDS only.  No thread reads global memory
// written by another thread of the workgroup, so pending global stores (the
// per-chunk snapshots) need not drain at every barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}


}  // namespace

size_t chain_lds_bytes(int lam, int C, int d, bool f32) {
  return chain_layout(lam, C, d / 32, f32).total;   // the largest case, k = 1
}

template <class DT, int HD, int SPW>
__global__ __launch_bounds__(kThreads) void chain_kernel(ChainArgs a) {
  using T = typename DT::T;
  constexpr int NSLAB = HD / 32;                  // column slabs of H
  constexpr int NTILE = 4 * SPW;                  // own H tiles (feature block, slab)
  constexpr int NPW = (NTILE + kWaves - 1) / kWaves;   // H tiles per wave (1 or 2)
  constexpr int NG = NSLAB / SPW;                 // slab groups
  const VirtRows vr = a.vr;
  const int lam = vr.lam, eta = vr.eta, k = a.k, CS = a.k / NG;
  const int LE = lam + a.C;                       // candidates per step, at most
  // workgroup -> (unit, rank); with U a multiple of 8 the k workgroups of a
  // unit get blocks of one residue mod 8 (blocks are dealt to the 8 XCDs
  // round-robin, so they share an L2)
  int u, rank;
  if (a.xcd_group) {
    const int b = blockIdx.x, m = b >> 3;
    u = 8 * (m / k) + (b & 7);
    rank = m % k;
  } else {
    u = blockIdx.x / k;
    rank = blockIdx.x % k;
  }
  const int grp = rank % NG, ch = rank / NG;      // slab group, candidate group
  const bool writer = ch == 0;                    // writes this slab group's columns
  const int col0 = 32 * SPW * grp;                // first H column of this workgroup
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, r = lane & 31;

  extern __shared__ __align__(16) unsigned char smem[];
  const ChainLayout L = chain_layout(lam, a.C, SPW, DT::kSplit);
  struct {
    uint16_t *HT_hi, *HT_lo;
    float *s32, *spart;
    int32_t *G, *Gp, *S, *misc;
    uint64_t* kred;
    int32_t* E;
    float* part;
    uint64_t* keys;
    int32_t* hist;
    uint16_t *phT_hi, *phT_lo, *VT_hi, *VT_lo;
  } sm = {(uint16_t*)(smem + L.HT_hi), (uint16_t*)(smem + L.HT_lo), (float*)(smem + L.s32),
          (float*)(smem + L.spart), (int32_t*)(smem + L.G), (int32_t*)(smem + L.Gp),
          (int32_t*)(smem + L.S), (int32_t*)(smem + L.misc), (uint64_t*)(smem + L.kred),
          (int32_t*)(smem + L.E), (float*)(smem + L.part), (uint64_t*)(smem + L.keys),
          (int32_t*)(smem + L.hist), (uint16_t*)(smem + L.phT_hi), (uint16_t*)(smem + L.phT_lo),
          (uint16_t*)(smem + L.VT_hi), (uint16_t*)(smem + L.VT_lo)};

  // ---- own H tiles: tile p = wave + kWaves * i (p < NTILE) -> slab p / 4, mt p % 4
  // (H is stored transposed, H^T [d][kD]: the lane's four consecutive
  // features of a column are one 16-byte load)
  f32x16 Hreg[NPW];
  const float* Hg = a.H + (size_t)u * kD * HD;
#pragma unroll
  for (int i = 0; i < NPW; ++i) {
    const int p = wave + kWaves * i, sw = p >> 2, mt = p & 3;
#pragma unroll
    for (int q = 0; q < 16; ++q) Hreg[i][q] = 0.f;
    if (p < NTILE) {
      const float* hc = Hg + (size_t)(col0 + 32 * sw + r) * kD + 32 * mt + 4 * h;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(hc + 8 * g4);
#pragma unroll
        for (int q = 0; q < 4; ++q) Hreg[i][4 * g4 + q] = x[q];
      }
    }
  }
  for (int F = tid; F < kD; F += kThreads) sm.s32[F] = a.s[(size_t)u * kD + F];
  const long long n0 = vr.n0;
  // the cache at the first step j0: at the call start, cache slots 0..gs0-1;
  // a later segment resumes from the list the previous one wrote to finalG
  // (gs entries: every position that left the window is cached or folded)
  const int gs0 = (int)min((long long)lam, max(0LL, n0 + (long long)a.j0 * a.C - eta));
  for (int i = tid; i < gs0; i += kThreads) {
    const int vi = a.j0 == 0 ? i : a.finalG[(size_t)u * lam + i];
    sm.G[i] = vi;
    sm.Gp[i] = (int32_t)vr.pos_of(u, vi);
  }
  if (tid == 0) sm.misc[16] = 0;

  // own columns of H^T as hi / lo rows (row = column - col0)
  auto rebuild_HT = [&]() {
#pragma unroll
    for (int i = 0; i < NPW; ++i) {
      const int p = wave + kWaves * i, sw = p >> 2, mt = p & 3;
      if (p < NTILE) {
        const int cl = 32 * sw + r;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int F = 32 * mt + 8 * g4 + 4 * h;
          float x[4] = {Hreg[i][4 * g4], Hreg[i][4 * g4 + 1], Hreg[i][4 * g4 + 2], Hreg[i][4 * g4 + 3]};
          uint32_t hi[4], lo[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) DT::split(x[q], hi[q], lo[q]);
          *reinterpret_cast<u32x2*>(sm.HT_hi + cl * HTP + F) = u32x2{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16)};
          *reinterpret_cast<u32x2*>(sm.HT_lo + cl * HTP + F) = u32x2{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)};
        }
      }
    }
  };
  rebuild_HT();
  lds_barrier();

  int gs = gs0;
  int xstep = a.xstep0;                           // exchange steps so far (over the call)
  const size_t phi_unit = (size_t)u * a.NV * kD;
  for (int j = a.j0; j < a.j1; ++j) {
    const long long nj = n0 + (long long)j * a.C;
    const int c = min(a.C, vr.T - j * a.C);

    // ---- 1. snapshot (own rows of H_j^T hi/lo; rank 0: s_j, G_j)
    if (writer) {
      uint16_t* dst = a.snapHT + ((size_t)u * a.nch + j) * 2 * HD * kD;
      constexpr int chunks = 32 * SPW * (kD / 8);   // 16-byte pieces per plane
      for (int i = tid; i < 2 * chunks; i += kThreads) {
        const int pl = i / chunks, rem = i % chunks;
        const int row = rem / (kD / 8), col = (rem % (kD / 8)) * 8;
        const uint16_t* src = (pl ? sm.HT_lo : sm.HT_hi) + row * HTP + col;
        *reinterpret_cast<u32x4*>(dst + (size_t)pl * HD * kD + (size_t)(col0 + row) * kD + col) =
            *reinterpret_cast<const u32x4*>(src);
      }
      if (rank == 0) {
        float* sdst = a.snaps + ((size_t)u * a.nch + j) * kD;
        for (int F = tid; F < kD; F += kThreads) sdst[F] = sm.s32[F];
        int32_t* gdst = a.snapG + ((size_t)u * a.nch + j) * lam;
        for (int i = tid; i < gs; i += kThreads) gdst[i] = sm.G[i];
      }
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
    for (int i = tid; i < 256; i += kThreads) sm.hist[i] = 0;
    lds_barrier();

    // ---- 4a. SRE parts over this workgroup's columns.  Wave w takes slab
    // w % SPW (A operands from its H^T rows in LDS) and the
    // candidate tiles t = w / SPW, w / SPW + kWaves / SPW, ...; per tile the
    // phi rows (B operands) and V columns come from global memory.
    const int ntile = lam > 0 ? (nE + 31) / 32 : 0;
    const int ntile_own = ntile > ch ? (ntile - ch + CS - 1) / CS : 0;
    const uint32_t tag = (uint32_t)(xstep + 1);
    uint64_t* xb = a.xbuf + ((size_t)u * 2 + (xstep & 1)) * NSLAB * LE;
    {
      const int sw = wave % SPW;
      const int t_first = wave / SPW;
      constexpr int TSTEP = kWaves / SPW;
      if (t_first < ntile_own) {
        const uint16_t* Ahi = sm.HT_hi + (32 * sw + r) * HTP + 8 * h;
        const uint16_t* Alo = sm.HT_lo + (32 * sw + r) * HTP + 8 * h;
        for (int lt = t_first; lt < ntile_own; lt += TSTEP) {
          const int e = 32 * (ch + CS * lt) + r;
          const bool ev = e < nE;
          const int vi = ev ? sm.E[e] : sm.E[0];
          const uint16_t* ph = a.phi_hi + phi_unit + (size_t)vi * kD + 8 * h;
          const uint16_t* pl = a.phi_lo + phi_unit + (size_t)vi * kD + 8 * h;
          u32x4 bh[8], bl[8];
#pragma unroll
          for (int kb = 0; kb < 8; ++kb) { bh[kb] = ld16(ph + 16 * kb); bl[kb] = ld16(pl + 16 * kb); }
          const T* vrow = reinterpret_cast<const T*>(vr.vrow(u, vi, sizeof(T))) + col0 + 32 * sw + 4 * h;
          float vv[4][4];
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) load4_f32(vrow + 8 * g4, vv[g4]);
          // z = phi^T s with phi = hi + lo, as the GEMM sees it
          float z = 0.f;
#pragma unroll
          for (int kb = 0; kb < 8; ++kb) {
            const f32x4 s0 = *reinterpret_cast<const f32x4*>(sm.s32 + 16 * kb + 8 * h);
            const f32x4 s1 = *reinterpret_cast<const f32x4*>(sm.s32 + 16 * kb + 8 * h + 4);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const uint32_t wh = bh[kb][q], wl = bl[kb][q];
              const float f0 = DT::from_bits(wh & 0xFFFFu) + DT::from_bits(wl & 0xFFFFu);
              const float f1 = DT::from_bits(wh >> 16) + DT::from_bits(wl >> 16);
              z = fmaf(f0, q < 2 ? s0[2 * q] : s1[2 * q - 4], z);
              z = fmaf(f1, q < 2 ? s0[2 * q + 1] : s1[2 * q - 3], z);
            }
          }
          z += xor32(z);
          // P^T (this slab's 32 columns x 32 candidates), two accumulators
          f32x16 P0, P1;
#pragma unroll
          for (int q = 0; q < 16; ++q) { P0[q] = 0.f; P1[q] = 0.f; }
#pragma unroll
          for (int kb = 0; kb < 8; ++kb) {
            const u32x4 ah = ld16(Ahi + 16 * kb), al = ld16(Alo + 16 * kb);
            f32x16& P = (kb & 1) ? P1 : P0;
            P = DT::mma(ah, bh[kb], P);
            P = DT::mma(al, bh[kb], P);
            P = DT::mma(ah, bl[kb], P);
          }
          const float iz = z > 0.f ? 1.f / z : 0.f;   // z == 0: prediction 0
          float acc = 0.f;
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float df = (P0[4 * g4 + q] + P1[4 * g4 + q]) * iz - vv[g4][q];
              acc = fmaf(df, df, acc);
            }
          acc += xor32(acc);
          if (ev && h == 0) {
            if (k == 1) sm.part[sw * LE + e] = acc;
            else __hip_atomic_store(xb + (size_t)(grp * SPW + sw) * LE + e,
                                    ((uint64_t)tag << 32) | __float_as_uint(acc),
                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      }
    }
    lds_barrier();

    ++xstep;

    // keys = (SRE bits << 32) | (0xFFFFFFFF - position); SRE = slab parts in
    // order (k > 1: read back from the exchange, waiting for each tag)
    uint64_t kmin = ~0ull, kmax = 0;
    bool lost = false;
    for (int e = tid; lam > 0 && e < nE; e += kThreads) {
      float sre = 0.f;
      if (k > 1) {
        uint64_t w[NSLAB];
#pragma unroll
        for (int q = 0; q < NSLAB; ++q)
          w[q] = __hip_atomic_load(xb + (size_t)q * LE + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int q = 0; q < NSLAB; ++q) {
          int spins = 0;
          while ((uint32_t)(w[q] >> 32) != tag && !lost) {
            if (++spins > kSpinLimit) lost = true;
            w[q] = __hip_atomic_load(xb + (size_t)q * LE + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
          sre += __uint_as_float((uint32_t)w[q]);
        }
      } else {
#pragma unroll
        for (int q = 0; q < NSLAB; ++q) sre += sm.part[q * LE + e];
      }
      const uint32_t pos = e < gs ? (uint32_t)sm.Gp[e] : (uint32_t)(lo_p + (e - gs));
      const uint64_t key = ((uint64_t)__float_as_uint(sre) << 32) | (uint64_t)(0xFFFFFFFFu - pos);
      sm.keys[e] = key;
      kmin = key < kmin ? key : kmin;
      kmax = key > kmax ? key : kmax;
    }
    wave_minmax_u64(kmin, kmax);
    if (lane == 63) { sm.kred[2 * wave] = kmin; sm.kred[2 * wave + 1] = kmax; }
    if (lost) sm.misc[16] = 1;
    lds_barrier();
    if (sm.misc[16]) {           // a partner is lost: stop (the error flag is set)
      if (tid == 0) atomicOr(a.err, 1);
      return;
    }
    if (a.dbg_keys && rank == 0) {
      uint64_t* dk = a.dbg_keys + ((size_t)u * a.nch + j) * (lam + a.C);
      for (int e = tid; e < nE; e += kThreads) dk[e] = sm.keys[e];
    }

    // ---- 4b. exact top-lam: radix select of the lam-th largest key with
    // 8-bit digits, from the highest bit where the keys differ down.  Pass p
    // counts into histogram p % 3 and clears histogram (p + 1) % 3 for the
    // next pass; after one barrier every wave scans the 256 bins itself (the
    // same result in every wave), so a pass needs one barrier: a histogram is
    // cleared two passes after it was scanned, behind the barrier of the pass
    // between.  lam == 0: nothing is kept.
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
      int hi_bit = top + 1;          // the digit covers bits [lo, hi_bit)
      int need = lam;
      int buf = 0;
      for (;;) {
        const int lo = hi_bit > 8 ? hi_bit - 8 : 0;
        const uint32_t dmask = (1u << (hi_bit - lo)) - 1u;
        const int nbuf = buf == 2 ? 0 : buf + 1;
        int32_t* H = sm.hist + 256 * buf;
        for (int e = tid; e < nE; e += kThreads) {
          const uint64_t k = sm.keys[e];
          if ((k & mask) == prefix) atomicAdd(&H[(uint32_t)(k >> lo) & dmask], 1);
        }
        for (int i = tid; i < 256; i += kThreads) sm.hist[256 * nbuf + i] = 0;
        lds_barrier();
        // lane l owns bins 255 - 4 l - q: the lanes in order walk the bins
        // from the top down; the one lane whose bin holds the need-th key
        // hands the bin, the rank left in it and its count to the wave
        int cnt[4], tot = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) { cnt[q] = H[255 - 4 * lane - q]; tot += cnt[q]; }
        int above = wave_incl_scan(tot) - tot;
        int fb = 0, fneed = 0, fcnt = 0;
        bool found = false;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (above < need && need <= above + cnt[q]) {
            found = true;
            fb = 255 - 4 * lane - q;
            fneed = need - above;
            fcnt = cnt[q];
          }
          above += cnt[q];
        }
        const int src = (int)__builtin_ctzll(__ballot(found));
        const int bsel = __builtin_amdgcn_readlane(fb, src), cb = __builtin_amdgcn_readlane(fcnt, src);
        need = __builtin_amdgcn_readlane(fneed, src);
        prefix |= (uint64_t)bsel << lo;
        mask |= (uint64_t)dmask << lo;
        if (cb == need || lo == 0) break;
        hi_bit = lo;
        buf = nbuf;
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
          // (diagnostics) the step that folds each of the call's tokens
          if (a.dbg_fold && rank == 0 && sm.E[e] >= lam + eta)
            a.dbg_fold[(size_t)u * vr.T + (sm.E[e] - lam - eta)] = j;
        }
        kb += __popcll(bk);
      }
    }
    gs = lam;
    lds_barrier();

    // ---- 4d. fold the rest into own columns of H (MFMA) and into s, 64
    // tokens per block.  The gather is by rows: lane = token, wave = feature
    // / column chunks, with 16-byte loads where possible; the tiles are
    // written transposed (token-contiguous) for the MFMA operands.
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
        // V: own columns, VC per wave
        constexpr int VC = 32 * SPW / kWaves;            // 4, 8 or 16 columns
        float vx[VC];
        {
          const T* vrow = reinterpret_cast<const T*>(vr.vrow(u, vi, sizeof(T))) + col0 + VC * wave;
#pragma unroll
          for (int q4 = 0; q4 < VC; q4 += 4) {
            float x[4];
            if (tv) load4_f32(vrow + q4, x);
            else for (int q = 0; q < 4; ++q) x[q] = 0.f;
#pragma unroll
            for (int q = 0; q < 4; ++q) vx[q4 + q] = x[q];
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
        static_assert(TPP % 8 == 0, "parts are read as 8-token pieces");
        float part = 0.f;
#pragma unroll
        for (int q8 = 0; q8 < TPP / 8; ++q8) {
          const u32x4 wh = ld16(sm.phT_hi + F * STP + TPP * qt + 8 * q8);
          const u32x4 wl = ld16(sm.phT_lo + F * STP + TPP * qt + 8 * q8);
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const uint32_t bh = (q & 1) ? wh[q >> 1] >> 16 : wh[q >> 1] & 0xFFFFu;
            const uint32_t bl = (q & 1) ? wl[q >> 1] >> 16 : wl[q >> 1] & 0xFFFFu;
            part += DT::from_bits(bh) + DT::from_bits(bl);
          }
        }
        sacc += part;
        // the last block's partial sums go out before its closing barrier
        if (sb + 64 >= nS) sm.spart[(tid / kD) * kD + tid % kD] = sacc;
      }
      const int nkb = min(4, (nS - sb + 15) / 16);
      for (int kb = 0; kb < nkb; ++kb) {
        const int k0 = 16 * kb + 8 * h;
#pragma unroll
        for (int i = 0; i < NPW; ++i) {
          const int p = wave + kWaves * i, sw = p >> 2, mt = p & 3;
          if (p < NTILE) {
            const u32x4 bv = ld16(sm.VT_hi + (32 * sw + r) * STP + k0);
            const u32x4 ah = ld16(sm.phT_hi + (32 * mt + r) * STP + k0);
            const u32x4 al = ld16(sm.phT_lo + (32 * mt + r) * STP + k0);
            Hreg[i] = DT::mma(ah, bv, Hreg[i]);
            Hreg[i] = DT::mma(al, bv, Hreg[i]);
            if constexpr (DT::kSplit)
              Hreg[i] = DT::mma(ah, ld16(sm.VT_lo + (32 * sw + r) * STP + k0), Hreg[i]);
          }
        }
      }
      lds_barrier();
    }
    for (int F = tid; F < kD; F += kThreads) {
      float add = 0.f;
#pragma unroll
      for (int q = 0; q < kThreads / kD; ++q) add += sm.spart[q * kD + F];
      sm.s32[F] += add;
    }
    rebuild_HT();
    lds_barrier();
  }

  // ---- final state: own columns of H (candidate group 0); rank 0: s, the cache list
  float* Ho = a.H + (size_t)u * kD * HD;
#pragma unroll
  for (int i = 0; i < NPW; ++i) {
    const int p = wave + kWaves * i, sw = p >> 2, mt = p & 3;
    if (p < NTILE && writer) {
      float* hc = Ho + (size_t)(col0 + 32 * sw + r) * kD + 32 * mt + 4 * h;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *reinterpret_cast<f32x4*>(hc + 8 * g4) =
            f32x4{Hreg[i][4 * g4], Hreg[i][4 * g4 + 1], Hreg[i][4 * g4 + 2], Hreg[i][4 * g4 + 3]};
    }
  }
  if (rank == 0) {
    for (int F = tid; F < kD; F += kThreads) a.s[(size_t)u * kD + F] = sm.s32[F];
    for (int i = tid; i < gs; i += kThreads) a.finalG[(size_t)u * lam + i] = sm.G[i];
  }
}

template <class DT, int HD, int SPW>
static hipError_t launch_chain_t(const ChainArgs& a, int U, hipStream_t st) {
  const size_t lds = chain_layout(a.vr.lam, a.C, SPW, DT::kSplit).total;
  const void* fn = (const void*)chain_kernel<DT, HD, SPW>;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((chain_kernel<DT, HD, SPW>), dim3(U * a.k), dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

template <class DT, int HD>
static hipError_t launch_chain_k(const ChainArgs& a, int U, hipStream_t st) {
  constexpr int NSLAB = HD / 32;
  if (a.k >= NSLAB) return launch_chain_t<DT, HD, 1>(a, U, st);   // k = NSLAB * CS
  if (a.k == 1) return launch_chain_t<DT, HD, NSLAB>(a, U, st);
  if constexpr (NSLAB == 4) {
    if (a.k == 2) return launch_chain_t<DT, HD, 2>(a, U, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_chain(const ChainArgs& a, int U, bool f32, hipStream_t st) {
  if (U <= 0) return hipSuccess;
  if (a.vr.d == 64)
    return f32 ? launch_chain_k<F32, 64>(a, U, st) : launch_chain_k<BF16, 64>(a, U, st);
  return f32 ? launch_chain_k<F32, 128>(a, U, st) : launch_chain_k<BF16, 128>(a, U, st);
}

}  // namespace lola
