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
// permuted to match the result layout, see common.h), with V staged as
// key-major fp16 rows and its operand read back with transposing LDS reads.
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
#pragma once
#include <type_traits>

#include "internal.h"

namespace lola {

namespace attn_ns {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int KT = 64;        // keys per staged tile
constexpr float kSlack = 8.f; // log2 headroom of the softmax weights over the running maximum
constexpr int HTS = kD + 8;   // LDS row of H^T (16-bit elements): 68 dwords, 16-byte aligned;
                              // the 16 rows of a 16-byte read pass fall on distinct bank groups

// Byte offsets of the LDS arrays; the key phase reuses the region of the
// linear-read phase.
struct AttnLayout {
  uint32_t tab, tabv;                          // both phases: the key table (below)
  bool wide;
  uint32_t WT, HT_hi, HT_lo, s;                // linear-read phase
  uint32_t K[2], KL[2], VT[2], VTL[2];         // key phase, two buffers (V: key-major rows)
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

// LDS a workgroup may take (the device's 160 KB, less a margin)
constexpr uint32_t kLdsCap = 160 * 1024 - 64;

__host__ __device__ inline AttnLayout attn_layout_t(int d, int lam, int eta, int C, bool f32, bool wide) {
  AttnLayout L;
  uint32_t off = 0;
  auto take = [&](uint32_t b) { const uint32_t o = off; off = al16(off + b); return o; };
  const uint32_t esz = f32 ? 4 : 2;
  // the keys a chunk's queries see: the cache at chunk start, the window,
  // the chunk's own positions.  Wide: the byte addresses of every key's K
  // row and V row (64-bit each); else per key its source (cache, ring,
  // input) and row, packed as (source << 30) | row
  const uint32_t nk = (uint32_t)(lam + eta + C);
  L.wide = wide;
  L.tab = take(nk * (wide ? 8u : 4u));
  L.tabv = wide ? take(nk * 8u) : L.tab;
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
    L.VT[b] = take((uint32_t)KT * d * 2);              // [KT][d] fp16, pieces permuted (stg_off)
    L.VTL[b] = take(f32 ? (uint32_t)KT * d * 2 : 16);  // (fp32 inputs: hi, lo)
  }
  L.total = phaseA > off ? phaseA : off;
  return L;
}

// The wide key table where it fits (a row address is then one LDS read),
// else the packed one
__host__ __device__ inline AttnLayout attn_layout(int d, int lam, int eta, int C, bool f32) {
  const AttnLayout W = attn_layout_t(d, lam, eta, C, f32, true);
  return W.total <= kLdsCap ? W : attn_layout_t(d, lam, eta, C, f32, false);
}

__device__ __forceinline__ u32x2 ld8(const uint16_t* p) { return *reinterpret_cast<const u32x2*>(p); }

// 16 bytes written during this launch by another workgroup: two coherent
// (device-scope atomic) 8-byte loads
__device__ __forceinline__ u32x4 ld16_coherent(const uint16_t* p) {
  uint64_t* q = reinterpret_cast<uint64_t*>(const_cast<uint16_t*>(p));
  const uint64_t x = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t y = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return u32x4{(uint32_t)x, (uint32_t)(x >> 32), (uint32_t)y, (uint32_t)(y >> 32)};
}

// 16 bytes at a global-memory byte address (a global load, not a flat one)
__device__ __forceinline__ u32x4 ldg16(uint64_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(1))) u32x4*>(addr);
}


// The A operand of O^T += V^T P^T (32 V columns x 16 keys of k-block kb,
// columns 32 mo ..) from a V tile staged as key-major rows of P pieces
// (stg_off<P>): lane l gets column 32 mo + l % 32 for the keys sigma_h of the
// block (16 kb + 4 h .. + 3, then 16 kb + 8 + 4 h .. + 3; h = l / 32), as
// two transposing reads of four rows each.  vt_off: the lane's element offset
// for k-block 0 (rows 16 kb and 8 further keep the piece permutation, which
// depends on the row mod 4, so they are plain offsets).
template <int P>
__device__ __forceinline__ int vt_off(int mo, int lane) {
  return stg_off<P>(4 * (lane >> 5) + ((lane & 15) >> 2), 32 * mo + 16 * ((lane >> 4) & 1) + 4 * (lane & 3));
}
template <int P>
__device__ __forceinline__ u32x4 ld_vt(const uint16_t* buf, int kb, int off) {
  const u32x2 a = ld_tr(buf + off + 16 * kb * 8 * P), b = ld_tr(buf + off + (16 * kb + 8) * 8 * P);
  return u32x4{a[0], a[1], b[0], b[1]};
}

typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;

// two floats as a pair of fp16 (round to nearest even), the first in the low half
__device__ __forceinline__ uint32_t f16_pair(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
}

}  // namespace attn_ns

// One workgroup of the read: unit u, chunk ch0 + jrel, position tile pt.
// WIDE: the key table holds row addresses (the layout attn_layout picks
// where it fits), else packed (source, row) words.
template <class DT, int HD, bool WIDE>
__device__ __forceinline__ void attn_body(const AttnArgs& a, int u_, int jrel, int pt_) {
  using namespace attn_ns;
  using T = typename DT::T;
  constexpr int KB = HD / 16;     // 16-wide K blocks over the head dim
  constexpr int NMT = HD / 32;    // 32-row tiles of the output
  constexpr int KRS = HD + 8;     // LDS row of a staged key (elements)
  constexpr int PER = 16 / (int)sizeof(T);       // input elements per 16-byte piece
  constexpr int KPT = KT * HD / PER / kThreads;  // key pieces per thread and tile
  constexpr int VPT = KT * HD / PER / kThreads;  // V pieces per thread and tile (as K)
  constexpr int VP = HD / 8;                     // 16-byte fp16 pieces of a staged V row
  const VirtRows vr = a.vr;
  const int lam = vr.lam, eta = vr.eta;
  // unit fastest: with the unit count a multiple of 8, a unit's chunks share
  // an XCD (blocks are dealt to the 8 XCDs round-robin) and its K/V rows,
  // re-read by every chunk, stay in that XCD's L2
  const int u = u_, j = a.ch0 + jrel, pt = pt_;
  // (the wave index as a uniform value: scalar branches and address math)
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, r = lane & 31;
  const int kvh = u % a.Hkv;
  const long long n0 = vr.n0;
  const long long nj = n0 + (long long)j * a.C;
  const int cj = min(a.C, vr.T - j * a.C);
  const long long pbase = nj + (long long)pt * a.ptile;
  const long long pend = min(pbase + a.ptile, nj + cj);     // exclusive
  if (pbase >= pend) return;                                // whole block idle (uniform)
  // the chain gave up: the snapshots were not written (uniform)
  if (__builtin_amdgcn_readfirstlane(*reinterpret_cast<volatile const int*>(a.err)) != 0) return;
  // (concurrent read) wait until the chain has published this chunk's
  // snapshot: one thread polls, bounded; a chain that gave up, or a poll that
  // runs out, ends the workgroup (the latter sets the error flag)
  if (a.ready) {
    __shared__ int go;
    if (threadIdx.x == 0) {
      const int need = a.ready_need * (j + 1);
      int ok = 1, spins = 0;
      while (__hip_atomic_load(a.ready + u_, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < need) {
        if (*reinterpret_cast<volatile const int*>(a.err) != 0) { ok = 0; break; }
        if (++spins > a.spin_limit) {
          atomicOr(a.err, 2);
          ok = 0;
          break;
        }
        __builtin_amdgcn_s_sleep(4);
      }
      go = ok;
    }
    __syncthreads();
    if (!go) return;
  }
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
  const AttnLayout L = attn_layout_t(HD, lam, eta, a.C, DT::kSplit, WIDE);
  uint32_t* sm_tab = (uint32_t*)(smem + L.tab);
  uint64_t* sm_tabk = (uint64_t*)(smem + L.tab);
  uint64_t* sm_tabv = (uint64_t*)(smem + L.tabv);
  T* sm_WT = (T*)(smem + L.WT);
  uint16_t* sm_HT_hi = (uint16_t*)(smem + L.HT_hi);
  uint16_t* sm_HT_lo = (uint16_t*)(smem + L.HT_lo);
  float* sm_s = (float*)(smem + L.s);

  // the three sources of key rows, this unit's part
  const T* ck = reinterpret_cast<const T*>(vr.cache_k) + (size_t)u * lam * HD;
  const T* cv = reinterpret_cast<const T*>(vr.cache_v) + (size_t)u * lam * HD;
  const T* rk = reinterpret_cast<const T*>(vr.ring_k) + (size_t)u * eta * HD;
  const T* rv = reinterpret_cast<const T*>(vr.ring_v) + (size_t)u * eta * HD;
  const T* ik = reinterpret_cast<const T*>(vr.in_k) + (size_t)u * vr.T * HD;
  const T* iv = reinterpret_cast<const T*>(vr.in_v) + (size_t)u * vr.T * HD;
  // (source, row) of virtual index vi: cache slot, ring slot or input row
  auto vsrc = [&](int vi) -> uint32_t {
    if (vi < lam) return (uint32_t)vi;
    const int off = vi - lam;                       // position n0 - eta + off
    if (off < eta) {
      int slot = n0e + off;
      if (slot >= eta) slot -= eta;
      return (1u << 30) | (uint32_t)slot;
    }
    return (2u << 30) | (uint32_t)(off - eta);
  };
  // the byte address of key kk's row from the table entry e (built once per
  // workgroup below): the cache base plus the distance to the ring (source
  // bit 0) or to the input (source bit 1), plus the row -- adds and masks,
  // no selection among pointers
  const uint64_t bk = (uint64_t)(uintptr_t)ck, bv = (uint64_t)(uintptr_t)cv;
  const uint64_t dk1 = (uint64_t)(uintptr_t)rk - bk, dk2 = (uint64_t)(uintptr_t)ik - bk;
  const uint64_t dv1 = (uint64_t)(uintptr_t)rv - bv, dv2 = (uint64_t)(uintptr_t)iv - bv;
  auto row_addr = [](uint32_t e, uint64_t b, uint64_t d1, uint64_t d2) -> uint64_t {
    const uint64_t m1 = 0ull - (uint64_t)((e >> 30) & 1u), m2 = 0ull - (uint64_t)(e >> 31);
    return b + (d1 & m1) + (d2 & m2) + (uint64_t)(e & 0x3FFFFFFFu) * (HD * sizeof(T));
  };
  // virtual index of key kk: cache G_j, then local positions lo_j ..
  const int vi_loc0 = lam + eta + (int)(lo_j - n0);

  // ---- Q operands (B of S^T = K Q^T): lane = query r, K-slots 8h .. 8h+7.
  // 16-bit inputs: loaded here, in flight with the staging loads below
  u32x4 qh[KB], ql[KB];
  const T* qrow = reinterpret_cast<const T*>(a.q) +
                  (((size_t)u * a.g + (wactive ? hd : 0)) * vr.T + (size_t)(qvalid ? qpos - n0 : 0)) * HD;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const int k0 = 16 * kb + 8 * h;
    if constexpr (!DT::kSplit) {
      qh[kb] = qvalid ? ld16(reinterpret_cast<const uint16_t*>(qrow) + k0) : u32x4{0, 0, 0, 0};
      ql[kb] = u32x4{0, 0, 0, 0};
    }
  }

  // ---- stage W^T (this KV head), H_j^T hi / lo, s_j and the key table.
  // Every global load of this phase is issued before any of them is
  // stored (fixed trip counts, so the loads stay in flight together): the
  // phase then costs one round trip to memory, not one per loop iteration.
  {
    const T* WT = reinterpret_cast<const T*>(a.WT) + (size_t)kvh * kM * HD;
    const bool coh = a.ready != nullptr;   // snapshots written during this launch
    // the key table: cache keys from the snapshot's virtual indices (kept
    // inside the call's rows whatever the snapshot holds), then the local
    // positions.  The snapshot's entries of the first GT * kThreads keys are
    // loaded first: the table, and with it the first key tile's loads, need
    // only them
    const int32_t* Gj = a.snapG + ((size_t)u * a.nch + j) * lam;
    const uint32_t nv = (uint32_t)(lam + eta + vr.T);
    constexpr int GT = 4;
    auto load_g = [&](int i0, uint32_t (&gv)[GT]) {
#pragma unroll
      for (int k = 0; k < GT; ++k) {
        const int i = i0 + k * kThreads + tid;
        gv[k] = i >= gsj ? 0u
                : coh ? (uint32_t)__hip_atomic_load(const_cast<int32_t*>(Gj) + i, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT)
                      : (uint32_t)Gj[i];
      }
    };
    auto store_g = [&](int i0, const uint32_t (&gv)[GT]) {
#pragma unroll
      for (int k = 0; k < GT; ++k) {
        const int i = i0 + k * kThreads + tid;
        if (i < nkeys) {
          const uint32_t e = vsrc(i < gsj ? (int)(gv[k] < nv ? gv[k] : 0u) : vi_loc0 + (i - gsj));
          if constexpr (WIDE) {
            sm_tabk[i] = row_addr(e, bk, dk1, dk2);
            sm_tabv[i] = row_addr(e, bv, dv1, dv2);
          } else {
            sm_tab[i] = e;
          }
        }
      }
    };
    uint32_t gv0[GT];
    load_g(0, gv0);
    constexpr int WPIECES = kM * HD / PER;
    constexpr int HPIECES = HD * (kD / 8);
    static_assert(WPIECES % kThreads == 0 && (2 * HPIECES) % kThreads == 0, "fixed trip counts");
    constexpr int WPT = WPIECES / kThreads, HPT = 2 * HPIECES / kThreads;
    const uint16_t* snap = a.snapHT + ((size_t)u * a.nch + j) * 2 * HD * kD;
    u32x4 wv[WPT], hv[HPT];
#pragma unroll
    for (int k = 0; k < WPT; ++k) {
      const int i = tid + k * kThreads, f = i / (HD / PER), c = (i % (HD / PER)) * PER;
      wv[k] = *reinterpret_cast<const u32x4*>(WT + (size_t)f * HD + c);
    }
#pragma unroll
    for (int k = 0; k < HPT; ++k) {
      const int i = tid + k * kThreads, pl = i / HPIECES, rem = i % HPIECES;
      const int row = rem / (kD / 8), col = (rem % (kD / 8)) * 8;
      const uint16_t* src = snap + (size_t)pl * HD * kD + (size_t)row * kD + col;
      hv[k] = coh ? ld16_coherent(src) : *reinterpret_cast<const u32x4*>(src);
    }
    const float* sj = a.snaps + ((size_t)u * a.nch + j) * kD;
    float sv = 0.f;
    if (tid < kD)
      sv = coh ? __uint_as_float(__hip_atomic_load(const_cast<uint32_t*>(
                                                       reinterpret_cast<const uint32_t*>(sj) + tid),
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
               : sj[tid];
    // the key table (the rest of it, past GT * kThreads keys, read GT per
    // thread at a time)
    store_g(0, gv0);
    for (int i0 = GT * kThreads; i0 < nkeys; i0 += GT * kThreads) {
      uint32_t gv[GT];
      load_g(i0, gv);
      store_g(i0, gv);
    }
#pragma unroll
    for (int k = 0; k < WPT; ++k) {
      const int i = tid + k * kThreads, f = i / (HD / PER), c = (i % (HD / PER)) * PER;
      *reinterpret_cast<u32x4*>(sm_WT + f * KRS + c) = wv[k];
    }
#pragma unroll
    for (int k = 0; k < HPT; ++k) {
      const int i = tid + k * kThreads, pl = i / HPIECES, rem = i % HPIECES;
      const int row = rem / (kD / 8), col = (rem % (kD / 8)) * 8;
      // Each 16-element block of a row is stored with its middle quarters
      // swapped (elements 0-3, 8-11, 4-7, 12-15), so that the K-slots sigma_h
      // of an operand (elements 4h .. 4h + 3 and 8 + 4h .. 8 + 4h + 3) are 8
      // contiguous elements at 8h: one 16-byte read.  A piece is half a
      // block: its two 8-byte halves go to their places.
      uint16_t* dst = (pl ? sm_HT_lo : sm_HT_hi) + row * HTS + (col & ~15) + ((col >> 3) & 1) * 4;
      *reinterpret_cast<u32x2*>(dst) = u32x2{hv[k][0], hv[k][1]};
      *reinterpret_cast<u32x2*>(dst + 8) = u32x2{hv[k][2], hv[k][3]};
    }
    if (tid < kD) sm_s[tid] = sv;
  }

  // (fp32 inputs: split into fp16 hi / lo here.)  The operands are used
  // here on every path: otherwise their loads would count as pending in the
  // key loop, which would then wait for all of its own prefetches before the
  // first product of every tile
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    if constexpr (DT::kSplit) {
      const int k0 = 16 * kb + 8 * h;
      float x[8];
      if (qvalid) load8_f32(qrow + k0, x);
      else for (int q = 0; q < 8; ++q) x[q] = 0.f;
      splitop<DT>(x, qh[kb], ql[kb]);
    }
    __asm__ volatile("" :: "v"(qh[kb]), "v"(ql[kb]));
  }
  __syncthreads();

  // ---- the key tiles' loads, staging and buffers (the loop below).  Rows
  // past the last key are loaded from the last key's row (finite values
  // whose weights are exactly 0 after the mask), so the loads need no
  // branch.
  u32x4 kreg[KPT];
  u32x4 vreg[VPT];
  int vto[NMT];                                   // the lane's V operand offsets (ld_vt)
#pragma unroll
  for (int mo = 0; mo < NMT; ++mo) vto[mo] = vt_off<VP>(mo, lane);
  auto load_k = [&](int t0) {
#pragma unroll
    for (int q = 0; q < KPT; ++q) {
      const int pc = q * kThreads + tid, kl = pc / (HD / PER), c = (pc % (HD / PER)) * PER;
      const int kk = min(t0 + kl, nkeys - 1);
      kreg[q] = ldg16((WIDE ? sm_tabk[kk] : row_addr(sm_tab[kk], bk, dk1, dk2)) + c * sizeof(T));
    }
  };
  auto load_v = [&](int t0) {
#pragma unroll
    for (int q = 0; q < VPT; ++q) {
      const int pc = q * kThreads + tid, kl = pc / (HD / PER), c = (pc % (HD / PER)) * PER;
      const int kk = min(t0 + kl, nkeys - 1);
      vreg[q] = ldg16((WIDE ? sm_tabv[kk] : row_addr(sm_tab[kk], bv, dv1, dv2)) + c * sizeof(T));
    }
  };
  // buffer b's arrays (selects, so that the offsets stay in registers)
  auto buf_off = [&](const uint32_t (&o)[2], int b) -> uint32_t { return b ? o[1] : o[0]; };
  auto store_k = [&](int b) {
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
  };
  // V piece q of the thread into buffer b: key-major fp16 row pieces (bf16
  // inputs: 8 values to fp16, one 16-byte store; fp32 inputs: 4 values
  // split into fp16 hi and lo, 8 bytes to each plane)
  auto store_v_piece = [&](int b, int q) {
    uint16_t* VTb = (uint16_t*)(smem + buf_off(L.VT, b));
    uint16_t* VTLb = (uint16_t*)(smem + buf_off(L.VTL, b));
    const int pc = q * kThreads + tid, kl = pc / (HD / PER), c = (pc % (HD / PER)) * PER;
    const int off = stg_off<VP>(kl, c);
    if constexpr (DT::kSplit) {
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) DT::split(__uint_as_float(vreg[q][e]), hi[e], lo[e]);
      *reinterpret_cast<u32x2*>(VTb + off) = u32x2{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16)};
      *reinterpret_cast<u32x2*>(VTLb + off) = u32x2{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)};
    } else {
      u32x4 w;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        w[j] = f16_pair(__uint_as_float(vreg[q][j] << 16), __uint_as_float(vreg[q][j] & 0xFFFF0000u));
      *reinterpret_cast<u32x4*>(VTb + off) = w;
    }
  };
  auto store_v = [&](int b) {
#pragma unroll
    for (int q = 0; q < VPT; ++q) store_v_piece(b, q);
  };
  // cache keys hidden from the read: the key loop starts past them
  const int kbase = (a.branches & LOLA_READ_CACHE) ? 0 : gsj;
  const int ntiles = (nkeys - kbase + KT - 1) / KT;
  // the first tile's rows load while phi(q) and the linear read run
  // (16-bit inputs; fp32 inputs hold too many registers there)
  if (!DT::kSplit && ntiles > 0) {
    load_k(kbase);
    load_v(kbase);
  }

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
        const u32x4 ah = ld16(sm_HT_hi + row * HTS + 16 * kb + 8 * h);
        const u32x4 al = ld16(sm_HT_lo + row * HTS + 16 * kb + 8 * h);
        O[mo] = DT::mma(ah, bh, O[mo]);
        O[mo] = DT::mma(ah, bl, O[mo]);
        O[mo] = DT::mma(al, bh, O[mo]);
      }
    }
  }
  __syncthreads();   // the key tiles reuse the linear-read region

  // ---- explicit branch: key tiles of KT, double-buffered.  The linear
  // terms enter with logit 0 (weight 2^-m2); without them (state hidden, or
  // z_lin = 0: an empty state) the running maximum starts at -inf, so that
  // the weights of very negative logits do not all underflow
  float m2 = zlin > 0.f ? 0.f : -INFINITY, l = zlin;
  const float scale2 = 1.4426950408889634f / sqrtf((float)HD);
  // The key loop is a three-stage pipeline over tiles of KT keys.  At the
  // top of iteration t the LDS holds K of tile t + 1 and V of tile t, the
  // registers hold the scores of tile t (computed in iteration t - 1) and
  // the raw global loads of K of tile t + 2 and V of tile t + 1 (issued in
  // iteration t - 1).  Iteration t stages those loads into the buffers
  // nobody reads in this iteration, issues the loads of K of tile t + 3
  // and V of tile t + 2, and multiplies: S_{t+1} = K Q^T next to tile t's
  // exponentials, then O += V_t P_t.  For 16-bit inputs the staging goes
  // between the score products and the loads between the value products
  // (scheduling fences fix the order), so the matrix cores are fed while
  // the vector, LDS and memory work of the pipeline is done; one barrier
  // per tile publishes the staged buffers.  The first tile's rows were
  // loaded before phi(q) (16-bit inputs).
  // S^T = K Q^T of the tile in K buffer b (32 keys x 32 queries per half kh)
  auto scores = [&](int b, f32x16 (&Sx)[2]) {
    const uint16_t* Kb = (const uint16_t*)(smem + buf_off(L.K, b));
    const uint16_t* KLb = (const uint16_t*)(smem + buf_off(L.KL, b));
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
      for (int i = 0; i < 16; ++i) Sx[kh][i] = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int k0 = 16 * kb + 8 * h;
        const u32x4 ah = ld16(Kb + (32 * kh + r) * KRS + k0);
        Sx[kh] = DT::mma(ah, qh[kb], Sx[kh]);
        if constexpr (DT::kSplit) {
          const u32x4 al = ld16(KLb + (32 * kh + r) * KRS + k0);
          Sx[kh] = DT::mma(ah, ql[kb], Sx[kh]);
          Sx[kh] = DT::mma(al, qh[kb], Sx[kh]);
        }
      }
    }
  };
  // the scores of a tile and of the next one: two register sets whose roles
  // alternate from tile to tile (16-bit inputs: the loop runs two tiles per
  // iteration, so that the sets stay in fixed registers and are never copied)
  f32x16 Sb[DT::kSplit ? 1 : 2][2];
  if (ntiles > 0) {
    if constexpr (DT::kSplit) {
      load_k(kbase);
      load_v(kbase);
    }
    store_k(0);
    store_v(0);
  }
  if (ntiles > 1) {
    load_k(kbase + KT);
    store_k(1);
    load_v(kbase + KT);               // staged in iteration 0
  }
  if (ntiles > 2) load_k(kbase + 2 * KT);   // staged in iteration 0
  __syncthreads();
  if (ntiles > 0 && wactive && kbase <= wlast) scores(0, Sb[0]);
  // (iteration 0 overwrites K buffer 0 with tile 2: every wave has read it)
  __syncthreads();
  // tile t, its scores in Sb[P], the next tile's into Sb[P ^ 1]
  auto tile_step = [&](int t, auto parity) {
    // (fp32 inputs: the next tile's scores are taken after this tile's
    // products, into the same registers; two sets would not fit)
    constexpr int P = DT::kSplit ? 0 : decltype(parity)::value;
    f32x16 (&S)[2] = Sb[P];
    f32x16 (&Sn)[2] = Sb[DT::kSplit ? 0 : P ^ 1];
    const int t0 = kbase + t * KT, b = t & 1;
    // staged here: K of tile t + 2 into K buffer b, V of tile t + 1 into V
    // buffer b ^ 1; loaded here: K of tile t + 3, V of tile t + 2
    // (16-bit inputs: always, past the last tile too: the rows are clamped to
    // the last key, and a buffer staged past the end is one nobody reads in
    // this iteration and whose products are never used; loads without a
    // condition keep the staging registers free of copies)
    const bool stk = !DT::kSplit || t + 2 < ntiles, stv = !DT::kSplit || t + 1 < ntiles;
    const bool ldk = !DT::kSplit || t + 3 < ntiles, ldv = !DT::kSplit || t + 2 < ntiles;
    if (wactive && t0 <= wlast) {
      const uint16_t* VTb = (const uint16_t*)(smem + buf_off(L.VT, b));
      const uint16_t* VTLb = (const uint16_t*)(smem + buf_off(L.VTL, b));
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
        const float alpha = __builtin_amdgcn_exp2f(m2 - mnew);   // 0 from m2 = -inf
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
          for (int i = 0; i < 16; ++i) O[mt][i] *= alpha;
        l *= alpha;
        m2 = mnew;
      }
      // (m2 is still -inf only while every key so far is masked for this
      // query: its weights are then 0, exp2(-inf))
      const float msub = m2 == -INFINITY ? 0.f : m2;
      float rs = 0.f;
      if constexpr (DT::kSplit) {
        if (stk) store_k(b);
        if (stv) store_v(b ^ 1);
        if (ldk) load_k(t0 + 3 * KT);
        if (ldv) load_v(t0 + 2 * KT);
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            S[kh][i] = __builtin_amdgcn_exp2f(fmaf(S[kh][i], scale2, -msub));
            rs += S[kh][i];
          }
#pragma unroll
        for (int kb = 0; kb < KT / 16; ++kb) {
          const int kh = kb >> 1, i0 = 8 * (kb & 1);
          u32x4 ph8, pl8;
          float pv[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) pv[q] = S[kh][i0 + q];
          splitop<DT>(pv, ph8, pl8);
#pragma unroll
          for (int mo = 0; mo < NMT; ++mo) {
            const u32x4 vh = ld_vt<VP>(VTb, kb, vto[mo]);
            const u32x4 vl = ld_vt<VP>(VTLb, kb, vto[mo]);
            O[mo] = DT::mma(vh, ph8, O[mo]);
            O[mo] = DT::mma(vh, pl8, O[mo]);
            O[mo] = DT::mma(vl, ph8, O[mo]);
          }
        }
        // (fp32 inputs take three products per operand pair: the next
        // tile's scores come after this tile's products, in the same
        // registers, as two sets of them would not fit)
        scores(b ^ 1, Sn);
      } else {
        // The next tile's score products, one at a time, each followed by
        // EPC of this tile's weights (the exponentials, rounded to fp16 as
        // the value products take them) and, early on, the staging of the
        // loaded rows; a scheduling fence after each step keeps that order.
        // Operands are read from LDS LA products ahead.  (After a wave's
        // last tile the products are taken of whatever the buffer holds and
        // never used.)
        constexpr int LA = 3;
        constexpr int NS = 2 * KB;                 // score products
        constexpr int EPC = 32 / NS;               // weights per product
        constexpr int NP = (KT / 16) * NMT;        // value products
        static_assert(NS >= 8 && NP >= 4, "staging and loads are spread over these steps");
        const uint16_t* Kn = (const uint16_t*)(smem + buf_off(L.K, b ^ 1));
        auto kaddr = [&](int c) { return Kn + (32 * (c & 1) + r) * KRS + 16 * (c >> 1) + 8 * h; };
        auto vop = [&](int c) { return ld_vt<VP>(VTb, c / NMT, vto[c % NMT]); };
        u32x4 ka[LA], va[LA];
#pragma unroll
        for (int i = 0; i < LA; ++i) ka[i] = ld16(kaddr(i));
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int i = 0; i < 16; ++i) Sn[kh][i] = 0.f;
        f16x8 p8[KT / 16];
#pragma unroll
        for (int c = 0; c < NS; ++c) {
          const int kh = c & 1, kb = c >> 1;
          const u32x4 ac = ka[c % LA];
          if (c + LA < NS) ka[c % LA] = ld16(kaddr(c + LA));
          else va[(c + LA - NS) % LA] = vop(c + LA - NS);
          Sn[kh] = DT::mma(ac, qh[kb], Sn[kh]);
#pragma unroll
          for (int x = 0; x < EPC; ++x) {
            const int e = EPC * c + x, kp = e >> 3, q = e & 7;   // weight e: block kp, slot q
            p8[kp][q] = (_Float16)__builtin_amdgcn_exp2f(
                fmaf(S[kp >> 1][8 * (kp & 1) + q], scale2, -msub));
          }
          if (c == 0 && stk) store_k(b);
          if (c < VPT && stv) store_v_piece(b ^ 1, c);
          __builtin_amdgcn_sched_barrier(0);
        }
        // the value products, each with one step of the row sum (pairwise
        // dot products of the same rounded weights with 1), and the next
        // loads
        constexpr int DPC = 16 / NP;               // row-sum steps per product
        constexpr f16x2 one2 = {(_Float16)1.f, (_Float16)1.f};
#pragma unroll
        for (int c = 0; c < NP; ++c) {
          const int kb = c / NMT, mo = c % NMT;
          const u32x4 vc = va[c % LA];
          if (c + LA < NP) va[c % LA] = vop(c + LA);
          O[mo] = mfma_f16(__builtin_bit_cast(f16x8, vc), p8[kb], O[mo]);
#pragma unroll
          for (int x = 0; x < DPC; ++x) {
            const int pq = DPC * c + x, kp = pq >> 2, w = pq & 3;   // pair w of block kp
            rs = __builtin_amdgcn_fdot2(f16x2{p8[kp][2 * w], p8[kp][2 * w + 1]}, one2, rs, false);
          }
          if (c == 1 && ldk) load_k(t0 + 3 * KT);
          if (c == 3 && ldv) load_v(t0 + 2 * KT);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      rs = half_sum(rs);
      l += rs;
    } else {
      if (stk) store_k(b);
      if (stv) store_v(b ^ 1);
      if (ldk) load_k(t0 + 3 * KT);
      if (ldv) load_v(t0 + 2 * KT);
    }
    __syncthreads();
  };
  if constexpr (DT::kSplit) {
    for (int t = 0; t < ntiles; ++t) tile_step(t, std::integral_constant<int, 0>{});
  } else {
    int t = 0;
    for (; t + 1 < ntiles; t += 2) {
      tile_step(t, std::integral_constant<int, 0>{});
      tile_step(t + 1, std::integral_constant<int, 1>{});
    }
    if (t < ntiles) tile_step(t, std::integral_constant<int, 0>{});
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

}  // namespace lola
