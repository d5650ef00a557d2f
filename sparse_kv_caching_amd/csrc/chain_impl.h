// K2: LoLA's serial memory-allocation chain, one step per chunk.  A unit
// (b, KV head) is processed by k cooperating workgroups, every workgroup of
// the grid resident at once (the work split is below).
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
// LDS as H^T hi/lo rows, from which the waves read their slab's A operands
// of the next SRE GEMM.
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
#pragma once
#include <type_traits>

#include "internal.h"

namespace lola {

namespace chain_ns {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int HTP = kD + 8;   // padded LDS row of H^T (16-bit elements)
// Fold staging: 64 tokens per block, token-major rows of 16-bit elements
// (as gathered, stg_off), read back as MFMA operands with transposing LDS
// reads (ld_tr).
// fold staging buffers: two where the workgroup holds fewer than all slabs
// (the two then fit the LDS of the all-slab layout with one)
template <int HD, int SPW> constexpr int kFoldBufs = SPW < HD / 32 ? 2 : 1;

// Byte offsets of the LDS arrays (computed by value so that the kernel's
// pointers stay plain LDS pointers).  The candidate list, parts, keys and
// radix histogram of the selection phase share one region with the fold's
// staging tiles, which are live only after the selection.
struct ChainLayout {
  uint32_t HT_hi, HT_lo, s32, spart, G, Gp, S, misc, kred;
  uint32_t E, part, keys, hist, stage;         // selection phase
  uint32_t phS_hi, phS_lo, VS_hi, VS_lo;       // fold phase (same region)
  uint32_t total;
};

__host__ __device__ inline uint32_t align16(uint32_t x) { return (x + 15u) & ~15u; }

// nbuf: fold staging buffers (2 lets a block be staged while the previous
// one is multiplied, one barrier per block).  xs: the candidate split (parts
// go through the exchange only; the phi tiles of a round of the SRE are
// staged after the histograms)
__host__ __device__ inline ChainLayout chain_layout(int lam, int C, int spw, bool f32, int nbuf = 1,
                                                   bool xs = false) {
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
  // SRE parts (candidate split: [2][kWaves][32] by round parity, then the
  // z of the round's staged rows [kWaves][32])
  L.part = take(xs ? 3u * kWaves * 32 * 4 : (uint32_t)spw * le * 4);
  L.keys = take(le * 8);
  L.hist = take(768 * 4);                  // three radix histograms
  L.stage = xs ? take((uint32_t)(kWaves / spw) * 2 * 32 * HTP * 2) : 0;   // [tile][plane][32][HTP]
  const uint32_t sel_end = off;
  off = region;
  const uint32_t nb = (uint32_t)nbuf;
  L.phS_hi = take(nb * 64 * kD * 2);       // [nbuf][64][kD]
  L.phS_lo = take(nb * 64 * kD * 2);
  L.VS_hi = take(nb * 64 * ncol * 2);      // [nbuf][64][ncol]
  L.VS_lo = take(f32 ? nb * 64 * ncol * 2 : 16);
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


// The 32 x 32 x 16 MFMA operand of a staged block: lane l gets column
// c0 + l % 32 for rows k0 + 8 (l / 32) .. + 7 (k0: the k-block's first row, a
// multiple of 8), as two transposing reads of 4 rows each.
template <int P>
__device__ __forceinline__ u32x4 ld_op_tr(const uint16_t* buf, int k0, int c0, int lane) {
  const int row = k0 + 8 * (lane >> 5) + ((lane & 15) >> 2);
  const int col = c0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const u32x2 a = ld_tr(buf + stg_off<P>(row, col)), b = ld_tr(buf + stg_off<P>(row + 4, col));
  return u32x4{a[0], a[1], b[0], b[1]};
}

}  // namespace chain_ns

// The chain of one workgroup (block index bid of the chain's grid).  XS: the
// candidate split (the all-slab instance with k > 1), compiled separately so
// that the other instances keep their registers.
template <class DT, int HD, int SPW, bool XS = false>
__device__ __forceinline__ void chain_body(const ChainArgs& a, int bid) {
  using namespace chain_ns;
  using T = typename DT::T;
  constexpr int NSLAB = HD / 32;                  // column slabs of H
  constexpr int NTILE = 4 * SPW;                  // own H tiles (feature block, slab)
  constexpr int NPW = (NTILE + kWaves - 1) / kWaves;   // H tiles per wave (1 or 2)
  constexpr int NG = NSLAB / SPW;                 // slab groups
  // the workgroups of a unit exchange SRE parts when they split the columns
  // (the host launches SPW < NSLAB exactly when k > 1) or the candidates
  // (the candidate split: the all-slab instance with k > 1)
  constexpr bool kExch = SPW < NSLAB;
  static_assert(!XS || SPW == HD / 32, "the candidate split holds all slabs");
  constexpr bool xs = XS;
  const bool xch = kExch || xs;
  const VirtRows vr = a.vr;
  const int lam = vr.lam, eta = vr.eta, k = a.k, CS = a.k / NG;
  const int LE = lam + a.C;                       // candidates per step, at most
  // workgroup -> (unit, rank); with U a multiple of 8 the k workgroups of a
  // unit get blocks of one residue mod 8 (blocks are dealt to the 8 XCDs
  // round-robin, so they share an L2)
  int u, rank;
  if (a.xcd_group) {
    const int b = bid, m = b >> 3;
    u = 8 * (m / k) + (b & 7);
    rank = m % k;
  } else {
    u = bid / k;
    rank = bid % k;
  }
  // a chain that gave up earlier left the state unfinished: nothing to do
  // (every workgroup reads the same word, so the whole grid returns)
  if (__builtin_amdgcn_readfirstlane(*reinterpret_cast<volatile const int*>(a.err)) != 0) return;
  const int grp = rank % NG, ch = rank / NG;      // slab group, candidate group
  const int col0 = 32 * SPW * grp;                // first H column of this workgroup
  // snapshot writers: candidate group 0 of each slab group (its columns), or
  // with the candidate split the first nw workgroups, an equal share of the
  // columns each (nw = NSLAB, or k where k divides NSLAB, else 1)
  const int nw = xs ? (CS >= NSLAB ? NSLAB : (NSLAB % CS == 0 ? CS : 1)) : 1;
  const bool writer = ch < nw;
  const int wr0 = xs ? 32 * (NSLAB / nw) * ch : col0;   // first column written
  const int wrn = xs ? 32 * (NSLAB / nw) : 32 * SPW;    // columns written
  // (the wave index as a uniform value: scalar branches and address math)
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, r = lane & 31;

  extern __shared__ __align__(16) unsigned char smem[];
  const ChainLayout L = chain_layout(lam, a.C, SPW, DT::kSplit, kFoldBufs<HD, SPW>, xs);
  struct {
    uint16_t *HT_hi, *HT_lo;
    float *s32, *spart;
    int32_t *G, *Gp, *S, *misc;
    uint64_t* kred;
    int32_t* E;
    float* part;
    uint64_t* keys;
    int32_t* hist;
    uint16_t *phS_hi, *phS_lo, *VS_hi, *VS_lo;
  } sm = {(uint16_t*)(smem + L.HT_hi), (uint16_t*)(smem + L.HT_lo), (float*)(smem + L.s32),
          (float*)(smem + L.spart), (int32_t*)(smem + L.G), (int32_t*)(smem + L.Gp),
          (int32_t*)(smem + L.S), (int32_t*)(smem + L.misc), (uint64_t*)(smem + L.kred),
          (int32_t*)(smem + L.E), (float*)(smem + L.part), (uint64_t*)(smem + L.keys),
          (int32_t*)(smem + L.hist), (uint16_t*)(smem + L.phS_hi), (uint16_t*)(smem + L.phS_lo),
          (uint16_t*)(smem + L.VS_hi), (uint16_t*)(smem + L.VS_lo)};

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

  // (concurrent read) every store of this workgroup so far has completed at
  // the device's coherence point before one thread counts the snapshot as
  // published
  auto publish = [&]() {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) __hip_atomic_fetch_add(a.ready + u, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };

  int gs = gs0;
  int xstep = a.xstep0;                           // exchange steps so far (over the call)
  const size_t phi_unit = (size_t)u * a.NV * kD;
  for (int j = a.j0; j < a.j1; ++j) {
    const long long nj = n0 + (long long)j * a.C;
    const int c = min(a.C, vr.T - j * a.C);

    // ---- 1. snapshot (own rows of H_j^T hi/lo; rank 0: s_j, G_j).  With a
    // concurrent read the previous chunk's snapshot is published first (its
    // stores were issued a step ago), and the stores are coherent ones.
    if (writer) {
      if (a.ready && j > a.j0) publish();
      uint16_t* dst = a.snapHT + ((size_t)u * a.nch + j) * 2 * HD * kD;
      const int chunks = wrn * (kD / 8);             // 16-byte pieces per plane
      for (int i = tid; i < 2 * chunks; i += kThreads) {
        const int pl = i / chunks, rem = i % chunks;
        const int row = rem / (kD / 8), col = (rem % (kD / 8)) * 8;
        const uint16_t* src = (pl ? sm.HT_lo : sm.HT_hi) + (wr0 - col0 + row) * HTP + col;
        uint16_t* d16 = dst + (size_t)pl * HD * kD + (size_t)(wr0 + row) * kD + col;
        const u32x4 x = *reinterpret_cast<const u32x4*>(src);
        if (a.ready) {
          uint64_t* d64 = reinterpret_cast<uint64_t*>(d16);
          __hip_atomic_store(d64, (uint64_t)x[0] | ((uint64_t)x[1] << 32), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(d64 + 1, (uint64_t)x[2] | ((uint64_t)x[3] << 32), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        } else {
          *reinterpret_cast<u32x4*>(d16) = x;
        }
      }
      if (rank == 0) {
        float* sdst = a.snaps + ((size_t)u * a.nch + j) * kD;
        int32_t* gdst = a.snapG + ((size_t)u * a.nch + j) * lam;
        if (a.ready) {
          for (int F = tid; F < kD; F += kThreads)
            __hip_atomic_store(reinterpret_cast<uint32_t*>(sdst) + F, __float_as_uint(sm.s32[F]),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          for (int i = tid; i < gs; i += kThreads)
            __hip_atomic_store(gdst + i, sm.G[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
          for (int F = tid; F < kD; F += kThreads) sdst[F] = sm.s32[F];
          for (int i = tid; i < gs; i += kThreads) gdst[i] = sm.G[i];
        }
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

    // ---- 4a. SRE parts over this workgroup's columns, by tiles of 32
    // candidates (t with t % CS == ch).  A tile's part over a slab is one
    // wave's work: A operands from the slab's H^T rows in LDS, B operands
    // the candidates' phi rows, then the error over the slab's columns
    // against the candidates' V values (from global memory).
    const int ntile = lam > 0 ? (nE + 31) / 32 : 0;
    const int ntile_own = ntile > ch ? (ntile - ch + CS - 1) / CS : 0;
    const uint32_t tag = (uint32_t)(xstep + 1);
    uint64_t* xb = a.xbuf + ((size_t)u * 2 + (xstep & 1)) * NSLAB * LE;
    // row r of the A operand is slab column 16 ((r >> 2) & 1) + 4 (r >> 3) +
    // (r & 3), so that accumulator row 8 g + 4 h + q (lane half h) is column
    // 16 h + 4 g + q: a lane's 16 columns are contiguous, and its V values
    // whole 16-byte pieces of the row
    const int pr = 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3);
    // the V values of the lane's 16 columns of candidate row vi, slab sw
    auto load_v = [&](u32x4 (&v)[sizeof(T)], int vi, int sw) {
      const T* vrow = reinterpret_cast<const T*>(vr.vrow(u, vi, sizeof(T))) + col0 + 32 * sw + 16 * h;
#pragma unroll
      for (int c = 0; c < (int)sizeof(T); ++c) v[c] = *reinterpret_cast<const u32x4*>(vrow + 16 / sizeof(T) * c);
    };
    // z = phi^T s of a candidate, with phi = hi + lo as the GEMM sees it,
    // in a fixed order that does not depend on which threads hold the
    // features: a partial per 16-byte piece (features 8 p .. 8 p + 7, an fma
    // chain from 0 in feature order), then a pairwise tree over the 16
    // pieces that pairs pieces differing in bit 1 of p, then bit 2, bit 3,
    // and last bit 0 (every addition commutes, so the two holders of a pair
    // form the same value)
    auto zpiece = [&](const u32x4& bh, const u32x4& bl, const float* s8) {
      const f32x4 s0 = *reinterpret_cast<const f32x4*>(s8);
      const f32x4 s1 = *reinterpret_cast<const f32x4*>(s8 + 4);
      float z = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t wh = bh[q], wl = bl[q];
        const float f0 = DT::from_bits(wh & 0xFFFFu) + DT::from_bits(wl & 0xFFFFu);
        const float f1 = DT::from_bits(wh >> 16) + DT::from_bits(wl >> 16);
        z = fmaf(f0, q < 2 ? s0[2 * q] : s1[2 * q - 4], z);
        z = fmaf(f1, q < 2 ? s0[2 * q + 1] : s1[2 * q - 3], z);
      }
      return z;
    };
    // the part over slab sw of the candidate of lane row r (returned in
    // both lane halves), from its phi row's hi / lo pieces (get(kb, hi, lo):
    // lane half h, features 16 kb + 8 h ..: piece 2 kb + h) and V values.
    // merged: z is given (zin) and one pass over kb reads the operands
    // once each; else z first, as the register-held operands allow
    auto sre_tile = [&](auto merged, auto&& get, const u32x4 (&vw)[sizeof(T)], int sw, float zin,
                        auto&& put) {
      const uint16_t* Ahi = sm.HT_hi + (32 * sw + pr) * HTP + 8 * h;
      const uint16_t* Alo = sm.HT_lo + (32 * sw + pr) * HTP + 8 * h;
      float vv[16];
#pragma unroll
      for (int c = 0; c < (int)sizeof(T); ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (sizeof(T) == 2) {
            vv[8 * c + 2 * j] = __uint_as_float(vw[c][j] << 16);
            vv[8 * c + 2 * j + 1] = __uint_as_float(vw[c][j] & 0xFFFF0000u);
          } else {
            vv[4 * c + j] = __uint_as_float(vw[c][j]);
          }
        }
      // z and P^T (this slab's 32 columns x 32 candidates) in two accumulators
      float z = zin;
      f32x16 P0, P1;
#pragma unroll
      for (int q = 0; q < 16; ++q) { P0[q] = 0.f; P1[q] = 0.f; }
      auto prod = [&](int kb, const u32x4& bh, const u32x4& bl) {
        const u32x4 ah = ld16(Ahi + 16 * kb), al = ld16(Alo + 16 * kb);
        f32x16& P = (kb & 1) ? P1 : P0;
        P = DT::mma(ah, bh, P);
        P = DT::mma(al, bh, P);
        P = DT::mma(ah, bl, P);
      };
      if constexpr (decltype(merged)::value) {
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) {
          u32x4 bh, bl;
          get(kb, bh, bl);
          prod(kb, bh, bl);
        }
      } else {
        // pieces 2 kb + h: bits 1..3 of the piece are the bits of kb (in the
        // lane), bit 0 the lane half
        float zq[8];
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) {
          u32x4 bh, bl;
          get(kb, bh, bl);
          zq[kb] = zpiece(bh, bl, sm.s32 + 16 * kb + 8 * h);
        }
        z = ((zq[0] + zq[1]) + (zq[2] + zq[3])) + ((zq[4] + zq[5]) + (zq[6] + zq[7]));
        z += xor32(z);
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) {
          u32x4 bh, bl;
          get(kb, bh, bl);
          prod(kb, bh, bl);
        }
      }
      const float iz = z > 0.f ? 1.f / z : 0.f;   // z == 0: prediction 0
      float acc = 0.f;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float df = (P0[4 * g4 + q] + P1[4 * g4 + q]) * iz - vv[4 * g4 + q];
          acc = fmaf(df, df, acc);
        }
      put(acc + xor32(acc));
    };
    if (!a.vscore && xs) {
      // candidate split: rounds of TPR tiles, each staged in LDS once (rows
      // read 16 lanes to 256 contiguous bytes) and shared by the NSLAB waves
      // of its slabs; the next round's rows and V values are in flight while
      // the current round computes.  The NSLAB parts of a candidate meet in
      // LDS and one word per candidate (their sum in slab order, the same
      // value a reader of per-slab parts forms) goes to the exchange.
      constexpr int TPR = kWaves / NSLAB;            // tiles per round
      static_assert(kThreads == 512, "a thread stages one 16-byte piece of one row per tile and plane");
      uint16_t* stg = reinterpret_cast<uint16_t*>(smem + L.stage);
      const int ts = wave / NSLAB, sw = wave % NSLAB;
      const int nround = (ntile_own + TPR - 1) / TPR;
      // a thread stages piece tid % 16 of row tid / 16 of every tile tt and
      // plane pl (its piece m = 2 tt + pl)
      const int srow = tid >> 4, spc = tid & 15;
      uint16_t* sdst = stg + srow * HTP + 8 * spc;
      u32x4 sg[2 * TPR], vn[sizeof(T)];
      float* rp = sm.part;                           // [2][kWaves][32]: round parity, (tile, slab), row
      auto publish_sums = [&](int ro) {
        if (tid < TPR * 32) {
          const int tt = tid >> 5, row = tid & 31, lt = ro * TPR + tt, e = 32 * (ch + CS * lt) + row;
          if (lt < ntile_own && e < nE) {
            float sre = 0.f;
#pragma unroll
            for (int q = 0; q < NSLAB; ++q) sre += rp[((ro & 1) * kWaves + tt * NSLAB + q) * 32 + row];
            __hip_atomic_store(xb + e, ((uint64_t)tag << 32) | __float_as_uint(sre), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      };
      auto stage_load = [&](int ro) {
#pragma unroll
        for (int tt = 0; tt < TPR; ++tt) {
          const int lt = ro * TPR + tt, e = 32 * (ch + CS * lt) + srow;
          const size_t off = phi_unit + (size_t)(lt < ntile_own && e < nE ? sm.E[e] : sm.E[0]) * kD + 8 * spc;
          sg[2 * tt] = lt < ntile_own ? ld16(a.phi_hi + off) : u32x4{0, 0, 0, 0};
          sg[2 * tt + 1] = lt < ntile_own ? ld16(a.phi_lo + off) : u32x4{0, 0, 0, 0};
        }
        const int lt = ro * TPR + ts, e = 32 * (ch + CS * lt) + r;
        if (lt < ntile_own) load_v(vn, e < nE ? sm.E[e] : sm.E[0], sw);
      };
      if (nround > 0) stage_load(0);
      float* zs = sm.part + 2 * kWaves * 32;         // [TPR][32]: z of the staged rows
      for (int ro = 0; ro < nround; ++ro) {
#pragma unroll
        for (int m = 0; m < 2 * TPR; ++m) *reinterpret_cast<u32x4*>(sdst + m * 32 * HTP) = sg[m];
        // z of the staged rows: this thread's piece, then the tree over the
        // row's 16 pieces (lanes 16 (row % 4) + piece, pairs by lane xor 2,
        // 4, 8, then 1)
#pragma unroll
        for (int tt = 0; tt < TPR; ++tt) {
          float zp = zpiece(sg[2 * tt], sg[2 * tt + 1], sm.s32 + 8 * spc);
          zp += __shfl_xor(zp, 2, 64);
          zp += __shfl_xor(zp, 4, 64);
          zp += __shfl_xor(zp, 8, 64);
          zp += __shfl_xor(zp, 1, 64);
          if (spc == 0) zs[tt * 32 + srow] = zp;
        }
        u32x4 vc[sizeof(T)];
#pragma unroll
        for (int c = 0; c < (int)sizeof(T); ++c) vc[c] = vn[c];
        lds_barrier();
        if (ro > 0) publish_sums(ro - 1);
        if (ro + 1 < nround) stage_load(ro + 1);
        const int lt = ro * TPR + ts;
        if (lt < ntile_own) {
          const uint16_t* sh = stg + ((ts * 2) * 32 + r) * HTP + 8 * h;
          const uint16_t* sl = sh + 32 * HTP;
          sre_tile(std::true_type{}, [&](int kb, u32x4& x, u32x4& y) { x = ld16(sh + 16 * kb); y = ld16(sl + 16 * kb); }, vc, sw,
                   zs[ts * 32 + r], [&](float acc) { if (h == 0) rp[((ro & 1) * kWaves + wave) * 32 + r] = acc; });
        }
        lds_barrier();                               // the round's tiles are read
      }
      if (nround > 0) publish_sums(nround - 1);
    } else if (!a.vscore) {
      // wave w takes slab w % SPW and the tiles t_first = w / SPW,
      // t_first + kWaves / SPW, ...; phi rows and V values from global memory
      const int sw = wave % SPW;
      const int t_first = wave / SPW;
      constexpr int TSTEP = kWaves / SPW;
      for (int lt = t_first; lt < ntile_own; lt += TSTEP) {
        const int e = 32 * (ch + CS * lt) + r;
        const int vi = e < nE ? sm.E[e] : sm.E[0];
        const uint16_t* ph = a.phi_hi + phi_unit + (size_t)vi * kD + 8 * h;
        const uint16_t* pl = a.phi_lo + phi_unit + (size_t)vi * kD + 8 * h;
        u32x4 bh[8], bl[8], vw[sizeof(T)];
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) { bh[kb] = ld16(ph + 16 * kb); bl[kb] = ld16(pl + 16 * kb); }
        load_v(vw, vi, sw);
        sre_tile(std::false_type{}, [&](int kb, u32x4& x, u32x4& y) { x = bh[kb]; y = bl[kb]; }, vw, sw, 0.f,
                 [&](float acc) {
          if (e < nE && h == 0) {
            if (!xch) sm.part[sw * LE + e] = acc;
            else __hip_atomic_store(xb + (size_t)(grp * SPW + sw) * LE + e,
                                    ((uint64_t)tag << 32) | __float_as_uint(acc),
                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        });
      }
    }
    lds_barrier();

    ++xstep;

    // keys = (SRE bits << 32) | (0xFFFFFFFF - position); SRE = slab parts in
    // order (k > 1: read back from the exchange, waiting for each tag)
    uint64_t kmin = ~0ull, kmax = 0;
    // (debug: the host can make every workgroup give up at one exchange step,
    // the same outcome as a lost partner, deterministically)
    bool lost = xstep - 1 == a.fail_at;
    // the candidates of a thread are read back in batches of XB: every word
    // of a batch is requested before any tag is checked, so the batch costs
    // one round trip to L2 rather than one per candidate.  (With an
    // accumulated scoring rule the keys come from the frozen scores: no
    // products, no exchange.)
    if (a.vscore) {
      const int nloc = eta + vr.T;
      for (int e = tid; lam > 0 && e < nE; e += kThreads) {
        const int vi = sm.E[e];
        const float sc = vi < lam ? a.cscore[(size_t)u * lam + vi]
                                  : a.vscore[(size_t)u * nloc + (vi - lam)];
        const uint32_t pos = e < gs ? (uint32_t)sm.Gp[e] : (uint32_t)(lo_p + (e - gs));
        const uint64_t key = ((uint64_t)__float_as_uint(sc) << 32) | (uint64_t)(0xFFFFFFFFu - pos);
        sm.keys[e] = key;
        kmin = key < kmin ? key : kmin;
        kmax = key > kmax ? key : kmax;
      }
    }
    // (per-slab words with the column split; one word, the sum, with the
    // candidate split)
    constexpr int XB = 4;
    constexpr int NQ = kExch ? NSLAB : 1;
    for (int e0 = tid; !a.vscore && lam > 0 && e0 < nE; e0 += XB * kThreads) {
      uint64_t w[XB][NQ];
      if (xch) {
#pragma unroll
        for (int i = 0; i < XB; ++i) {
          const int e = e0 + i * kThreads;
#pragma unroll
          for (int q = 0; q < NQ; ++q)
            w[i][q] = e < nE ? __hip_atomic_load(xb + (size_t)q * LE + e, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT)
                             : ((uint64_t)tag << 32);
        }
      }
#pragma unroll
      for (int i = 0; i < XB; ++i) {
        const int e = e0 + i * kThreads;
        if (e >= nE) break;
        float sre = 0.f;
        if (xch) {
#pragma unroll
          for (int q = 0; q < NQ; ++q) {
            int spins = 0;
            while ((uint32_t)(w[i][q] >> 32) != tag && !lost) {
              if (++spins > a.spin_limit) lost = true;
              w[i][q] = __hip_atomic_load(xb + (size_t)q * LE + e, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
            }
            sre += __uint_as_float((uint32_t)w[i][q]);
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
      const int nit = e1 > e0 ? (e1 - e0 + 63) / 64 : 0;   // 64-candidate rows of the wave
      constexpr int MAXIT = 8;
      if (nit <= MAXIT) {
        // the wave's keys and virtual indices are read once, all at once
        // (rows of the wave only; indices clamped into the candidates: nE
        // >= 1 here), and the first pass's ballots are kept for the second
        uint64_t kk[MAXIT], bks[MAXIT];
        int32_t ev[MAXIT];
#pragma unroll
        for (int it = 0; it < MAXIT; ++it) {
          kk[it] = 0;
          ev[it] = 0;
          if (it < nit) {
            const int ec = min(e0 + 64 * it + lane, nE - 1);
            kk[it] = sm.keys[ec];
            ev[it] = sm.E[ec];
          }
        }
        int kept = 0;
#pragma unroll
        for (int it = 0; it < MAXIT; ++it) {
          const int e = e0 + 64 * it + lane;
          const bool kp = it < nit && e < e1 && lam > 0 && (kk[it] & mask) >= prefix;
          bks[it] = __ballot(kp);
          kept += __popcll(bks[it]);
        }
        if (lane == 0) sm.misc[8 + wave] = kept;
        lds_barrier();
        int kb = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
          if (w < wave) kb += sm.misc[8 + w];
#pragma unroll
        for (int it = 0; it < MAXIT; ++it) {
          if (it >= nit) break;
          const int e = e0 + 64 * it + lane;
          const bool in = e < e1;
          const bool kp = in && lam > 0 && (kk[it] & mask) >= prefix;
          const unsigned long long bk = bks[it];
          const int before = __popcll(bk & ((1ull << lane) - 1ull));
          if (kp) {
            if (kb + before < lam) {
              sm.G[kb + before] = ev[it];
              sm.Gp[kb + before] = (int32_t)(0xFFFFFFFFu - (uint32_t)kk[it]);
            }
          } else if (in) {
            const int sidx = e - (kb + before);
            if (sidx < nE - lam) sm.S[sidx] = ev[it];
            if (a.dbg_fold && rank == 0 && ev[it] >= lam + eta)
              a.dbg_fold[(size_t)u * vr.T + (ev[it] - lam - eta)] = j;
          }
          kb += __popcll(bk);
        }
      } else {
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
    }
    gs = lam;
    lds_barrier();

    // ---- 4d. fold the rest into own columns of H (MFMA) and into s, 64
    // tokens per block.  The gather reads rows four lanes to 64 contiguous
    // bytes (a 16-byte piece each), so that one load instruction touches 16
    // rows rather than 64 (a gather's cost in the vector memory unit grows
    // with the rows one instruction touches): wave w loads plane w / 4 (hi,
    // lo) of feature quarter w % 4 for the block's 64 tokens (tokens
    // 16 i + lane / 4), and the own V columns of tokens 8 w .. 8 w + 7.  The
    // pieces are staged as loaded, token-major (one 16-byte write each), and
    // the MFMA operands (token-contiguous per feature or column) and the s
    // sums are read back with transposing LDS reads.  The gathers of up to
    // GB blocks are issued together (they are latency-bound, and a later
    // block's loads then stay in flight while an earlier block is staged and
    // multiplied); values stay as loaded until they are staged.
    const int nS = nE - lam;
    float sacc = 0.f;
    static_assert(kWaves == 8 && kD == 128, "two planes x four feature quarters, one per wave");
    constexpr int PER = 16 / (int)sizeof(T);             // V elements per 16-byte piece
    constexpr int VPR = 32 * SPW / PER;                  // V pieces of an own row
    constexpr int VL = (8 * VPR + 63) / 64;              // V pieces per lane
    constexpr int GB = SPW == 1 || (XS && !DT::kSplit) ? 4 : 2;   // blocks gathered together
    struct Gather {
      u32x4 x[4];
      u32x4 v[VL];
    };
    const int pq = lane & 3, tq = lane >> 2;             // phi piece, token within 16
    const int fq = 32 * (wave & 3) + 8 * pq;             // the lane's first feature
    const uint16_t* pplane = (wave < 4 ? a.phi_hi : a.phi_lo) + phi_unit + fq;
    constexpr int NBUF = kFoldBufs<HD, SPW>;
    int blk = 0;                                         // blocks staged so far
    for (int sb0 = 0; sb0 < nS; sb0 += 64 * GB) {
      Gather gb[GB];
#pragma unroll
      for (int b = 0; b < GB; ++b) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = sb0 + 64 * b + 16 * i + tq;
          gb[b].x[i] = tok < nS ? ld16(pplane + (size_t)sm.S[tok] * kD) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int m = 0; m < VL; ++m) {
          const int idx = lane + 64 * m, pc = idx % VPR;
          const int tok = sb0 + 64 * b + 8 * wave + idx / VPR;
          gb[b].v[m] = idx < 8 * VPR && tok < nS
                           ? *reinterpret_cast<const u32x4*>(
                                 reinterpret_cast<const T*>(vr.vrow(u, sm.S[tok], sizeof(T))) + col0 + PER * pc)
                           : u32x4{0, 0, 0, 0};
        }
      }
#pragma unroll
      for (int b = 0; b < GB; ++b) {
        const int sb = sb0 + 64 * b;
        if (sb >= nS) break;
        // this block's staging buffer
        const int fb = NBUF == 2 ? (blk & 1) : 0;
        ++blk;
        constexpr int PP = kD / 8, PV = 4 * SPW;           // 16-byte pieces per staged row
        uint16_t* pSh = sm.phS_hi + fb * (64 * kD);
        uint16_t* pSl = sm.phS_lo + fb * (64 * kD);
        uint16_t* vSh = sm.VS_hi + fb * (64 * 32 * SPW);
        uint16_t* vSl = sm.VS_lo + (DT::kSplit ? fb * (64 * 32 * SPW) : 0);
        {
          uint16_t* dst = wave < 4 ? pSh : pSl;
#pragma unroll
          for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(dst + stg_off<PP>(16 * i + tq, fq)) = gb[b].x[i];
        }
#pragma unroll
        for (int m = 0; m < VL; ++m) {
          const int idx = lane + 64 * m, pc = idx % VPR, t = 8 * wave + idx / VPR;
          if (idx < 8 * VPR) {
            if constexpr (DT::kSplit) {
              // four fp32 values: their 16-bit hi and lo parts, two per dword
              uint32_t hi[4], lo[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) DT::split(__uint_as_float(gb[b].v[m][e]), hi[e], lo[e]);
              *reinterpret_cast<u32x2*>(vSh + stg_off<PV>(t, PER * pc)) = u32x2{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16)};
              *reinterpret_cast<u32x2*>(vSl + stg_off<PV>(t, PER * pc)) = u32x2{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)};
            } else {
              *reinterpret_cast<u32x4*>(vSh + stg_off<PV>(t, PER * pc)) = gb[b].v[m];
            }
          }
        }
        // (two buffers: a wave stages block b + 2 into this buffer only
        // after this barrier's successor, which every wave reaches after
        // its products of block b)
        lds_barrier();
        {
          // s partial sums: feature F, 64 / NPART tokens per part, fixed
          // order; a transposing read gives the lane 4 tokens of its feature
          const int F = tid % kD, qt = tid / kD;
          constexpr int TPP = 64 / (kThreads / kD);
          static_assert(TPP % 4 == 0 && kD % 64 == 0, "parts are read as 4-token pieces");
          const int foff = (F & ~15) + 4 * (lane & 3);     // the 16-feature block's column of the lane
          float part = 0.f;
#pragma unroll
          for (int q4 = 0; q4 < TPP / 4; ++q4) {
            const int row = TPP * qt + 4 * q4 + ((lane & 15) >> 2);
            const u32x2 wh = ld_tr(pSh + stg_off<PP>(row, foff));
            const u32x2 wl = ld_tr(pSl + stg_off<PP>(row, foff));
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const uint32_t bh = (q & 1) ? wh[q >> 1] >> 16 : wh[q >> 1] & 0xFFFFu;
              const uint32_t bl = (q & 1) ? wl[q >> 1] >> 16 : wl[q >> 1] & 0xFFFFu;
              part += DT::from_bits(bh) + DT::from_bits(bl);
            }
          }
          sacc += part;
          // the last block's partial sums go out before its closing barrier
          if (sb + 64 >= nS) sm.spart[(tid / kD) * kD + tid % kD] = sacc;
        }
        // The wave's tiles p = wave + kWaves i share the feature block
        // mt = wave % 4, so the phi operands of a k-block are read once for
        // all of them; the wave index is made uniform so that tiles past
        // NTILE are skipped by a scalar branch.
        const int nkb = min(4, (nS - sb + 15) / 16);
        const int wv = __builtin_amdgcn_readfirstlane(wave), mt = wv & 3;
        auto kblock = [&](int kb) {
          const u32x4 ah = ld_op_tr<PP>(pSh, 16 * kb, 32 * mt, lane);
          const u32x4 al = ld_op_tr<PP>(pSl, 16 * kb, 32 * mt, lane);
          // (every wave holds NPW tiles unless there are fewer tiles than waves)
          constexpr bool kAll = NTILE == NPW * kWaves;
          u32x4 bv[NPW];
#pragma unroll
          for (int i = 0; i < NPW; ++i)
            if (kAll || wv + kWaves * i < NTILE)
              bv[i] = ld_op_tr<PV>(vSh, 16 * kb, 32 * ((wv + kWaves * i) >> 2), lane);
#pragma unroll
          for (int i = 0; i < NPW; ++i) {
            const int p = wv + kWaves * i, sw = p >> 2;
            if (kAll || p < NTILE) {
              Hreg[i] = DT::mma(ah, bv[i], Hreg[i]);
              Hreg[i] = DT::mma(al, bv[i], Hreg[i]);
              if constexpr (DT::kSplit)
                Hreg[i] = DT::mma(ah, ld_op_tr<PV>(vSl, 16 * kb, 32 * sw, lane), Hreg[i]);
            }
          }
        };
        for (int kb = 0; kb < nkb; ++kb) kblock(kb);
        if constexpr (NBUF == 1) lds_barrier();
      }
    }
    if constexpr (NBUF == 2) lds_barrier();   // the last block's s partial sums
    for (int F = tid; F < kD; F += kThreads) {
      float add = 0.f;
#pragma unroll
      for (int q = 0; q < kThreads / kD; ++q) add += sm.spart[q * kD + F];
      sm.s32[F] += add;
    }
    rebuild_HT();
    lds_barrier();
  }

  if (a.ready && writer && a.j1 > a.j0) publish();

  // ---- final state: own columns of H (candidate group 0); rank 0: s, the cache list
  float* Ho = a.H + (size_t)u * kD * HD;
#pragma unroll
  for (int i = 0; i < NPW; ++i) {
    const int p = wave + kWaves * i, sw = p >> 2, mt = p & 3;
    if (p < NTILE && ch == 0) {
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

}  // namespace lola
