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
// The step is bound by HBM traffic: H and s are read and written once, the
// window and cache K/V read once.  One workgroup (4 waves) per unit.
//
//   * Every wave owns a 32-column slab of H, loaded at the start (buffer
//     loads, all in flight together) and held in registers in MFMA operand
//     layout: lane (c, h) holds H[16 kb + sigma_h(j)][c].
//   * The keys a query sees, in the order cache 0..gs-1, window (oldest
//     first), new pair, are streamed through LDS in chunks of kc rows (one
//     chunk for the decode shapes here), every load of a chunk issued before
//     the first is waited for.  The leaving pair is key gs, so the candidate
//     rows of the SRE are exactly keys 0..gs.
//   * Per chunk: logits S^T = K Q^T on MFMA; phi of the chunk's candidate rows
//     (x W^T on MFMA, W transposed once at state creation) computed by every
//     wave for itself, so that the phi registers feed P^T = H_slab^T phi (hi/lo
//     16-bit split, three passes) directly, giving the wave's columns of the
//     SRE predictions; online softmax (running max starting at 0); P V on the
//     VALU with every V row read once per workgroup.
//   * The query rows get phi(q) and the linear read H^T phi(q), phi(q)^T s the
//     same way.  Then the argmin key, the output, and the rank-1 fold of the
//     evicted pair into the register-resident H, written back once.
#include "internal.h"

namespace lola {

namespace {
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

// Byte offsets of the LDS arrays.
struct DecLayout {
  uint32_t wt, kst, vst, q, lk, lv, slot, slotz, logit, spart, phe, nlin, zq, ml, pv, red, total;
};
constexpr int WP = 8;   // row padding (elements) of W^T, K, V and q in LDS (bank spread)
constexpr uint32_t kSlotBytes = 8 * 2 * 64 * 16;   // B operands of one 32-row phi tile

inline __host__ __device__ uint32_t al16(uint32_t x) { return (x + 15u) & ~15u; }

__host__ __device__ inline DecLayout dec_layout(int lam, int d, int g, int esz, int kc, int nslot) {
  DecLayout L;
  uint32_t off = 0;
  auto take = [&](uint32_t b) { const uint32_t o = off; off = al16(off + b); return o; };
  const uint32_t row = (uint32_t)(d + WP) * esz;
  L.wt = take(kM * row);                               // [kM][d + WP] W^T of this KV head
  L.kst = take((uint32_t)kc * row);                    // [kc][d + WP] key chunk
  L.vst = take((uint32_t)kc * row);                    // [kc][d + WP] value chunk
  L.q = take(4 * row);                                 // [g][d + WP] queries
  L.lk = take((uint32_t)d * esz);                      // leaving key
  L.lv = take((uint32_t)d * esz);                      // leaving value
  L.slot = take((uint32_t)nslot * kSlotBytes);         // [slot][kb][hi, lo][lane] phi operands
  L.slotz = take((uint32_t)nslot * 32 * 4);            // [slot][row] phi^T s
  L.logit = take((uint32_t)4 * kc * 4);                // [kc][4] logits, then weights
  L.spart = take((uint32_t)(d / 32) * (lam + 1) * 4);  // [slab][candidate] partial SRE
  L.phe = take(kD * 4);                                // phi of the folded row
  L.nlin = take((uint32_t)g * d * 4);                  // [g][d] H^T phi(q)
  L.zq = take(4 * 4);                                  // [g] phi(q)^T s
  L.ml = take(3 * 4 * 4);                              // [4] running max, sum, rescale
  L.pv = take((uint32_t)kWaves * 4 * d * 4);           // [wave][4][d] P V partials
  L.red = take(kWaves * 16);                           // the folded row
  L.total = off;
  return L;
}
constexpr size_t kDecLdsBudget = 160 * 1024;

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
template <class DT>
__device__ __forceinline__ f32x16 mma_x(u32x4 ah, u32x4 al, u32x4 bh, u32x4 bl, f32x16 c) {
  c = DT::mma(ah, bh, c);
  if constexpr (DT::kSplit) {
    c = DT::mma(ah, bl, c);
    c = DT::mma(al, bh, c);
  }
  return c;
}

__device__ __forceinline__ float ldf(const uint16_t* p) { return bf16_bits_to_f32(*p); }
__device__ __forceinline__ float ldf(const float* p) { return *p; }

// phi of 32 rows (lane (r, h) supplies row r); W^T rows f = 32 mt + r, row
// stride HD + WP elements (LDS).
// Result: ph[half][mt][i] = phi[64 half + 32 mt + 8 (i/4) + 4 h + (i%4)] of row r.
template <class DT, int HD>
__device__ __forceinline__ void phi_tile(const DT& dt, const typename DT::T* xrow,
                                         const typename DT::T* WT, int h, int r,
                                         float (&ph)[2][2][16]) {
  constexpr int KB = HD / 16;
  f32x16 U2[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) U2[mt][i] = 0.f;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const int k0 = 16 * kb + 8 * h;
    u32x4 bh, bl;
    if (xrow) xop(dt, xrow + k0, bh, bl);
    else bh = bl = u32x4{0, 0, 0, 0};
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      u32x4 ah, al;
      xop(dt, WT + (32 * mt + r) * (HD + WP) + k0, ah, al);
      U2[mt] = mma_x<DT>(ah, al, bh, bl, U2[mt]);
    }
  }
  float mx = -INFINITY, mn = INFINITY;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) { mx = fmaxf(mx, U2[mt][i]); mn = fminf(mn, U2[mt][i]); }
  mx = fmaxf(mx, xor32(mx));
  mn = fminf(mn, xor32(mn));
  // e^(u - max) = 2^(u log2 e - max log2 e)
  constexpr float kL2E = 1.4426950408889634f;
  const float mxl = mx * kL2E, mnl = mn * kL2E;
  float sp = 0.f, sn = 0.f;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      ph[0][mt][i] = __builtin_amdgcn_exp2f(fmaf(U2[mt][i], kL2E, -mxl));
      ph[1][mt][i] = __builtin_amdgcn_exp2f(fmaf(-U2[mt][i], kL2E, mnl));
      sp += ph[0][mt][i];
      sn += ph[1][mt][i];
    }
  sp += xor32(sp);
  sn += xor32(sn);
  const float ip = 1.f / sp, in_ = 1.f / sn;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) { ph[0][mt][i] *= ip; ph[1][mt][i] *= in_; }
}

// feature of K-slot j of k-block kb for lane half h (the sigma_h permutation)
__device__ __forceinline__ int sigma_feat(int kb, int h, int j) {
  return 16 * kb + (j < 4 ? 4 * h + j : 8 + 4 * h + (j - 4));
}
// byte offset of H row sigma_feat(kb, 0, j) (the lane part 4 h rows is separate)
__device__ __forceinline__ int h_soff(int kb, int j, int hd) {
  return (16 * kb + (j < 4 ? j : 8 + (j - 4))) * hd * 4;
}
// buffer resource word 3 for gfx9-class raw (untyped) dword access
constexpr int kBufWord3 = 0x00020000;

// phi of a 32-row tile into an LDS slot: B operands of the H product in
// sigma order ([kb][hi, lo][lane] 16-byte pieces, the lane's own layout) and
// z = phi^T s per row (fp32 phi; the split operands differ from it by less
// than 2^-17 relative).
template <class DT, int HD>
__device__ __forceinline__ void phi_to_slot(const DT& dt, const typename DT::T* xrow,
                                            const typename DT::T* WT, const float (&sv)[8][8],
                                            int lane, int h, int r, u32x4* slot, float* slotz) {
  float ph[2][2][16];
  phi_tile<DT, HD>(dt, xrow, WT, h, r, ph);
  float zz = 0.f;
#pragma unroll
  for (int kb = 0; kb < 8; ++kb) {
    const int half = kb >> 2, mt = (kb & 3) >> 1, i0 = 8 * (kb & 1);
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      x[j] = ph[half][mt][i0 + j];
      zz = fmaf(x[j], sv[kb][j], zz);
    }
    u32x4 Bh, Bl;
    splitop<DT>(x, Bh, Bl);
    slot[(2 * kb) * 64 + lane] = Bh;
    slot[(2 * kb + 1) * 64 + lane] = Bl;
  }
  zz += xor32(zz);
  if (h == 0) slotz[r] = zz;
}

// P^T = H_slab^T phi for the 32 rows of a slot, three split passes with the
// slab's pre-split operands.  Lane (r, h) gets P^T[32 slab + 8 (i/4) + 4 h + (i%4)][r].
template <class DT>
__device__ __forceinline__ f32x16 slab_product(const u32x4* slot, const u32x4 (&Ah)[8],
                                              const u32x4 (&Al)[8], int lane) {
  f32x16 P0, P1;
#pragma unroll
  for (int i = 0; i < 16; ++i) { P0[i] = 0.f; P1[i] = 0.f; }
#pragma unroll
  for (int kb = 0; kb < 8; ++kb) {
    const u32x4 Bh = slot[(2 * kb) * 64 + lane], Bl = slot[(2 * kb + 1) * 64 + lane];
    f32x16& P = (kb & 1) ? P1 : P0;
    P = DT::mma(Ah[kb], Bh, P);
    P = DT::mma(Ah[kb], Bl, P);
    P = DT::mma(Al[kb], Bh, P);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) P0[i] += P1[i];
  return P0;
}

// N consecutive elements (N = 1 or 2) as float
template <int N>
__device__ __forceinline__ void load_cols(const uint16_t* p, float* o) {
  if constexpr (N == 2) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
    o[0] = __uint_as_float(w << 16);
    o[1] = __uint_as_float(w & 0xFFFF0000u);
  } else {
    o[0] = bf16_bits_to_f32(*p);
  }
}
template <int N>
__device__ __forceinline__ void load_cols(const float* p, float* o) {
#pragma unroll
  for (int j = 0; j < N; ++j) o[j] = p[j];
}

}  // namespace

// Rows per staged key chunk and phi slots: all lam + eta + 1 keys if they fit
// (rows rounded up to 8), with as many slots (<= 4) as the phi rows need and
// the LDS holds; else fewer rows.  kc = 0: nothing fits.
void decode_plan(int lam, int eta, int d, int g, bool f32, int* kc_out, int* nslot_out) {
  const int esz = f32 ? 4 : 2;
  const int nk = lam + eta + 1;
  const int tiles = (lam + 1 + g + 31) / 32;
  const int want_slots = tiles < 4 ? tiles : 4;
  for (int kc = (nk + 7) / 8 * 8; kc >= 32; kc -= 8) {
    for (int ns = want_slots; ns >= 1; --ns)
      if (dec_layout(lam, d, g, esz, kc, ns).total <= kDecLdsBudget) {
        *kc_out = kc;
        *nslot_out = ns;
        return;
      }
  }
  *kc_out = 0;
  *nslot_out = 0;
}

size_t decode_lds_bytes(int lam, int eta, int d, int g, bool f32) {
  int kc, ns;
  decode_plan(lam, eta, d, g, f32, &kc, &ns);
  if (kc == 0) return kDecLdsBudget + 1;
  return dec_layout(lam, d, g, f32 ? 4 : 2, kc, ns).total;
}

template <class DT, int HD>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
  using T = typename DT::T;
  constexpr int NS = HD / 32;        // column slabs of H (one per wave)
  constexpr int KB = HD / 16;        // k-blocks of a d-long contraction
  constexpr int PER = 16 / (int)sizeof(T);   // elements per 16-byte piece
  constexpr int PPR = HD / PER;              // pieces per row
  constexpr int RS = HD + WP;                // LDS row stride (elements)
  constexpr int NB = 24;                     // staged pieces in flight per thread
  const DT dt{};
  const int u = blockIdx.x, lam = a.lam, eta = a.eta, g = a.g, KC = a.kc, NSLOT = a.nslot;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, r = lane & 31;
  const int kvh = u % a.Hkv;
  const long long n = a.n;
  const int gs = (int)min((long long)lam, max(0LL, n - eta));
  const bool has_leave = n >= eta;                 // eta == 0: the new pair leaves at once
  const bool full = has_leave && gs + 1 > lam;     // score and fold
  const int ncand = full ? gs + 1 : 0;             // candidate rows = keys 0..gs
  const int w_len = (int)min((long long)eta, n);   // window positions n - w_len .. n - 1
  const int nk = gs + w_len + 1;                   // keys a query sees (cache, window, itself)
  const int ring0 = eta > 0 ? (int)((n - w_len) % eta) : 0;   // ring slot of the oldest window row
  const int ringn = eta > 0 ? (int)(n % eta) : 0;             // ring slot of position n (and n - eta)

  extern __shared__ __align__(16) unsigned char smem[];
  const DecLayout L = dec_layout(lam, HD, g, (int)sizeof(T), KC, NSLOT);
  T* sm_wt = (T*)(smem + L.wt);
  T* sm_k = (T*)(smem + L.kst);
  T* sm_v = (T*)(smem + L.vst);
  T* sm_q = (T*)(smem + L.q);
  T* sm_lk = (T*)(smem + L.lk);
  T* sm_lv = (T*)(smem + L.lv);
  u32x4* sm_slot = (u32x4*)(smem + L.slot);
  float* sm_slotz = (float*)(smem + L.slotz);
  float* sm_logit = (float*)(smem + L.logit);
  float* sm_spart = (float*)(smem + L.spart);
  float* sm_phe = (float*)(smem + L.phe);
  float* sm_nlin = (float*)(smem + L.nlin);
  float* sm_zq = (float*)(smem + L.zq);
  float* sm_ml = (float*)(smem + L.ml);            // [0..3] max, [4..7] sum, [8..11] rescale
  float* sm_pv = (float*)(smem + L.pv);
  int32_t* sm_redi = (int32_t*)(smem + L.red);

  const T* qg = reinterpret_cast<const T*>(a.q) + (size_t)u * a.q_su;
  const T* kin = reinterpret_cast<const T*>(a.k) + (size_t)u * a.kv_su;
  const T* vin = reinterpret_cast<const T*>(a.v) + (size_t)u * a.kv_su;
  T* ringk = reinterpret_cast<T*>(a.ring_k) + (size_t)u * eta * HD;
  T* ringv = reinterpret_cast<T*>(a.ring_v) + (size_t)u * eta * HD;
  T* ck = reinterpret_cast<T*>(a.cache_k) + (size_t)u * lam * HD;
  T* cv = reinterpret_cast<T*>(a.cache_v) + (size_t)u * lam * HD;
  const T* WT = reinterpret_cast<const T*>(a.WT) + (size_t)kvh * kM * HD;
  const float* sg = a.s + (size_t)u * kD;
  // the leaving pair (position n - eta): ring slot n % eta, or the new pair
  const T* leave_k = eta > 0 ? ringk + (size_t)ringn * HD : kin;
  const T* leave_v = eta > 0 ? ringv + (size_t)ringn * HD : vin;
  // global rows of key kk
  auto key_row = [&](int kk, bool val) -> const T* {
    if (kk < gs) return (val ? cv : ck) + (size_t)kk * HD;
    if (kk < gs + w_len) {
      int slot = ring0 + (kk - gs);
      if (slot >= eta) slot -= eta;
      return (val ? ringv : ringk) + (size_t)slot * HD;
    }
    return val ? vin : kin;
  };
  // Stage K and V rows k0 .. k0 + kn into LDS, NB 16-byte loads in flight
  // per thread before the first is written.
  auto stage_chunk = [&](int k0, int kn) {
    const int total = 2 * kn * PPR;
    for (int b0 = 0; b0 < total; b0 += NB * kThreads) {
      u32x4 buf[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int i = b0 + j * kThreads + tid;
        if (i < total) {
          const bool isv = i >= kn * PPR;
          const int ii = isv ? i - kn * PPR : i;
          buf[j] = *reinterpret_cast<const u32x4*>(key_row(k0 + ii / PPR, isv) + (ii % PPR) * PER);
        }
      }
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int i = b0 + j * kThreads + tid;
        if (i < total) {
          const bool isv = i >= kn * PPR;
          const int ii = isv ? i - kn * PPR : i;
          *reinterpret_cast<u32x4*>((isv ? sm_v : sm_k) + (ii / PPR) * RS + (ii % PPR) * PER) = buf[j];
        }
      }
    }
  };

  // ---- every read of the step that does not depend on the argmin, in flight together
  // H slab through a buffer resource: one lane offset plus a uniform offset per
  // element (waves without a slab, d = 64, read a valid column they never use)
  const bool has_slab = NS >= kWaves || wave < NS;
  const int cc = 32 * wave + r;                    // this lane's H column
  const __amdgpu_buffer_rsrc_t Hrs =
      __builtin_amdgcn_make_buffer_rsrc(a.H + (size_t)u * kD * HD, 0, kD * HD * 4, kBufWord3);
  const int hoff = (4 * h * HD + (cc & (HD - 1))) * 4;
  float Hs[8][8];
#pragma unroll
  for (int kb = 0; kb < 8; ++kb)
#pragma unroll
    for (int j = 0; j < 8; ++j)
      Hs[kb][j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(Hrs, hoff, h_soff(kb, j, HD), 0));
  // s at this lane's features (the same sigma pattern as its H rows)
  float sv[8][8];
#pragma unroll
  for (int kb = 0; kb < 8; ++kb) {
    const f32x4 s0 = *reinterpret_cast<const f32x4*>(sg + 16 * kb + 4 * h);
    const f32x4 s1 = *reinterpret_cast<const f32x4*>(sg + 16 * kb + 8 + 4 * h);
#pragma unroll
    for (int j = 0; j < 4; ++j) { sv[kb][j] = s0[j]; sv[kb][4 + j] = s1[j]; }
  }
  {
    constexpr int WPT = kM * PPR / kThreads;       // W^T pieces per thread
    u32x4 wb[WPT], qb, lb;
#pragma unroll
    for (int j = 0; j < WPT; ++j) {
      const int i = j * kThreads + tid;
      wb[j] = *reinterpret_cast<const u32x4*>(WT + (size_t)(i / PPR) * HD + (i % PPR) * PER);
    }
    const bool hq = tid < g * PPR, hl = has_leave && tid < 2 * PPR;
    if (hq) qb = *reinterpret_cast<const u32x4*>(qg + (size_t)(tid / PPR) * a.q_sh + (tid % PPR) * PER);
    if (hl) lb = *reinterpret_cast<const u32x4*>((tid < PPR ? leave_k : leave_v) + (tid % PPR) * PER);
    stage_chunk(0, min(KC, nk));
#pragma unroll
    for (int j = 0; j < WPT; ++j) {
      const int i = j * kThreads + tid;
      *reinterpret_cast<u32x4*>(sm_wt + (i / PPR) * RS + (i % PPR) * PER) = wb[j];
    }
    if (hq) *reinterpret_cast<u32x4*>(sm_q + (tid / PPR) * RS + (tid % PPR) * PER) = qb;
    if (hl) *reinterpret_cast<u32x4*>((tid < PPR ? sm_lk : sm_lv) + (tid % PPR) * PER) = lb;
  }
  if (tid < 4) { sm_ml[tid] = 0.f; sm_ml[4 + tid] = 0.f; sm_ml[8 + tid] = 1.f; }
  __syncthreads();

  constexpr float kL2E = 1.4426950408889634f;
  const float scale2 = kL2E / sqrtf((float)HD);   // logits in the log2 domain
  constexpr int CPL = HD / 64;                     // P V columns per lane
  float acc[4][CPL];
#pragma unroll
  for (int hd = 0; hd < 4; ++hd)
#pragma unroll
    for (int j = 0; j < CPL; ++j) acc[hd][j] = 0.f;
  bool phe_in_slot = false;                        // the folded row's phi is still in a slot

  // ---- key chunks (one for the decode shapes here)
  for (int k0 = 0; k0 < nk; k0 += KC) {
    const int kn = min(KC, nk - k0);
    const bool last = k0 + KC >= nk;
    if (k0 > 0) {
      __syncthreads();                             // the previous chunk's readers are done
      stage_chunk(k0, kn);
      __syncthreads();
    }
    // phi rows of the chunk: its candidate rows, then (last chunk) the queries
    const int cn = max(0, min(kn, ncand - k0));
    const int nr = cn + (last ? g : 0);
    const int nt = (nr + 31) / 32;
    const int nrounds = max(1, (nt + NSLOT - 1) / NSLOT);
    phe_in_slot = k0 == 0 && last && nt <= NSLOT;
    for (int R = 0; R < nrounds; ++R) {
      const int t_lo = R * NSLOT, t_n = max(0, min(NSLOT, nt - t_lo));
      if (R > 0) __syncthreads();                  // the previous round's slots are consumed
      // phase A: wave w < t_n computes phi of tile t_lo + w into slot w; the
      // other waves (then all) compute the chunk's logits S^T = K Q^T
      if (wave < t_n) {
        const int row = 32 * (t_lo + wave) + r;
        const T* xrow = row < cn ? sm_k + row * RS : (row < nr ? sm_q + (row - cn) * RS : nullptr);
        phi_to_slot<DT, HD>(dt, xrow, sm_wt, sv, lane, h, r, sm_slot + wave * (kSlotBytes / 16),
                            sm_slotz + wave * 32);
      }
      if (R == 0) {
        for (int kt = (wave - t_n + kWaves) % kWaves; 32 * kt < kn; kt += kWaves) {
          const int row = 32 * kt + r;
          f32x16 S;
#pragma unroll
          for (int i = 0; i < 16; ++i) S[i] = 0.f;
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            u32x4 kh, kl, qh, ql;
            if (row < kn) xop(dt, sm_k + row * RS + 16 * kb + 8 * h, kh, kl);
            else kh = kl = u32x4{0, 0, 0, 0};
            if (r < g) xop(dt, sm_q + r * RS + 16 * kb + 8 * h, qh, ql);
            else qh = ql = u32x4{0, 0, 0, 0};
            S = mma_x<DT>(kh, kl, qh, ql, S);
          }
          if (r < g) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int j = 32 * kt + 8 * (i / 4) + 4 * h + (i % 4);
              if (j < kn) sm_logit[4 * j + r] = S[i] * scale2;
            }
          }
        }
      }
      __syncthreads();                             // slots (and logits)
      // phase B: every slab wave, its columns of the SRE parts / linear read,
      // with the slab's split operands
      if (has_slab) {
        u32x4 Ah[8], Al[8];
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) splitop<DT>(Hs[kb], Ah[kb], Al[kb]);
        for (int t = 0; t < t_n; ++t) {
          const f32x16 P = slab_product<DT>(sm_slot + t * (kSlotBytes / 16), Ah, Al, lane);
          const int row = 32 * (t_lo + t) + r;
          const float z = sm_slotz[t * 32 + r];
          if (row < cn) {
            const float iz = z > 0.f ? 1.f / z : 0.f;
            float part = 0.f;
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              float vv[4];
              load4_f32(sm_v + row * RS + 32 * wave + 8 * g4 + 4 * h, vv);
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const float p = P[4 * g4 + q] * iz;
                part = fmaf(p - vv[q], p - vv[q], part);
              }
            }
            part += xor32(part);
            if (h == 0) sm_spart[wave * (lam + 1) + k0 + row] = part;
          } else if (row < nr) {
            const int hd = row - cn;
#pragma unroll
            for (int i = 0; i < 16; ++i) sm_nlin[hd * HD + 32 * wave + 8 * (i / 4) + 4 * h + (i % 4)] = P[i];
            if (wave == 0 && h == 0) sm_zq[hd] = z;
          }
        }
      }
    }

    // online softmax per head (wave = head), log2 domain; running max starts at 0
    if (wave < g) {
      float* lg = sm_logit + wave;
      const float m_old = sm_ml[wave];
      float m = m_old;
      for (int j = lane; j < kn; j += 64) m = fmaxf(m, lg[4 * j]);
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
      float l = 0.f;
      for (int j = lane; j < kn; j += 64) {
        const float p = __builtin_amdgcn_exp2f(lg[4 * j] - m);
        lg[4 * j] = p;
        l += p;
      }
      l = wave_sum(l);
      if (lane == 0) {
        const float alpha = __builtin_amdgcn_exp2f(m_old - m);
        sm_ml[wave] = m;
        sm_ml[4 + wave] = sm_ml[4 + wave] * alpha + l;
        sm_ml[8 + wave] = alpha;
      }
    }
    __syncthreads();                               // weights, rescale factors

    // P V: wave w takes rows w, w + 4, ... of the chunk; four heads always
    // (rows of absent heads are never read back)
#pragma unroll
    for (int hd = 0; hd < 4; ++hd) {
      const float alpha = sm_ml[8 + hd];
#pragma unroll
      for (int j = 0; j < CPL; ++j) acc[hd][j] *= alpha;
    }
    int j0 = wave;
    for (; j0 + 3 * kWaves < kn; j0 += 4 * kWaves) {
      float vv[4][CPL];
      f32x4 pp[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        load_cols<CPL>(sm_v + (j0 + e * kWaves) * RS + CPL * lane, vv[e]);
        pp[e] = *reinterpret_cast<const f32x4*>(sm_logit + 4 * (j0 + e * kWaves));
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int hd = 0; hd < 4; ++hd)
#pragma unroll
          for (int c = 0; c < CPL; ++c) acc[hd][c] = fmaf(pp[e][hd], vv[e][c], acc[hd][c]);
    }
    for (; j0 < kn; j0 += kWaves) {
      float vv[CPL];
      load_cols<CPL>(sm_v + j0 * RS + CPL * lane, vv);
      const f32x4 pp = *reinterpret_cast<const f32x4*>(sm_logit + 4 * j0);
#pragma unroll
      for (int hd = 0; hd < 4; ++hd)
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[hd][c] = fmaf(pp[hd], vv[c], acc[hd][c]);
    }
  }
#pragma unroll
  for (int hd = 0; hd < 4; ++hd)
#pragma unroll
    for (int j = 0; j < CPL; ++j) sm_pv[(wave * 4 + hd) * HD + CPL * lane + j] = acc[hd][j];

  // ---- the candidate to fold: lowest SRE, ties to the newer position
  // (the lowest key (SRE, 0xFFFFFFFF - pos)); candidates are few, one wave
  int fold_row = -1;   // < gs: cache slot; == gs: the leaving pair
  if (full && wave == 0) {
    float best = INFINITY;
    int bpos = -1, bi = 0;
    for (int e = lane; e < ncand; e += 64) {
      float sre = 0.f;
#pragma unroll
      for (int w = 0; w < NS; ++w) sre += sm_spart[w * (lam + 1) + e];
      const int pos = e < gs ? a.cache_pos[(size_t)u * lam + e] : (int)(n - eta);
      if (sre < best || (sre == best && pos > bpos)) { best = sre; bpos = pos; bi = e; }
    }
    float m = best;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fminf(m, __shfl_xor(m, o, 64));
    int p = best == m ? bpos : -1;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) p = max(p, __shfl_xor(p, o, 64));
    const uint64_t win = __ballot(best == m && bpos == p);
    const int wl = (int)__builtin_ctzll(win);
    bi = __shfl(bi, wl, 64);
    if (lane == 0) sm_redi[0] = bi;
  }
  __syncthreads();                                 // pv partials, the folded row
  if (full) fold_row = sm_redi[0];

  // ---- phi of the folded row (last wave): hi + lo from its slot as the
  // products above saw it, else recomputed (MFMA); the others write y
  if (fold_row >= 0 && wave == kWaves - 1) {
    if (phe_in_slot) {
      if (r == (fold_row & 31)) {
        const u32x4* sl = sm_slot + (fold_row >> 5) * (kSlotBytes / 16);
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) {
          const u32x4 bh = sl[(2 * kb) * 64 + lane], bl = sl[(2 * kb + 1) * 64 + lane];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const uint32_t hw = bh[j >> 1] >> (16 * (j & 1)), lw = bl[j >> 1] >> (16 * (j & 1));
            sm_phe[sigma_feat(kb, h, j)] = DT::from_bits(hw & 0xFFFFu) + DT::from_bits(lw & 0xFFFFu);
          }
        }
      }
    } else {
      const T* xrow = r == 0 ? (fold_row < gs ? ck + (size_t)fold_row * HD : sm_lk) : nullptr;
      float ph[2][2][16];
      phi_tile<DT, HD>(dt, xrow, sm_wt, h, r, ph);
      if (r == 0) {
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i)
              sm_phe[64 * half + 32 * mt + 8 * (i / 4) + 4 * h + (i % 4)] = ph[half][mt][i];
      }
    }
  }
  for (int i = tid; i < g * HD; i += kThreads) {
    const int hd = i / HD, c = i % HD;
    const float em = __builtin_amdgcn_exp2f(-sm_ml[hd]);
    float num = em * sm_nlin[i];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) num += sm_pv[(w * 4 + hd) * HD + c];
    const float den = sm_ml[4 + hd] + em * sm_zq[hd];
    a.out[(size_t)u * a.o_su + (size_t)hd * a.o_sh + c] = num / den;
  }
  __syncthreads();   // phe; every read of the cache and ring is done

  // ---- update: fold, cache slot, ring slot
  if (fold_row >= 0) {
    if (has_slab) {
      // v of the folded row: staged V row (single chunk), else the cache
      const float ve = ldf(fold_row == gs ? sm_lv + cc
                                          : (nk <= KC ? sm_v + fold_row * RS + cc
                                                      : cv + (size_t)fold_row * HD + cc));
#pragma unroll
      for (int kb = 0; kb < 8; ++kb)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float hv = fmaf(sm_phe[sigma_feat(kb, h, j)], ve, Hs[kb][j]);
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(hv), Hrs, hoff, h_soff(kb, j, HD), 0);
        }
    }
    for (int F = tid; F < kD; F += kThreads) a.s[(size_t)u * kD + F] = sg[F] + sm_phe[F];
  }
  __syncthreads();   // the folded cache row has been read
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
  if (eta > 0) {
    T* dk = ringk + (size_t)ringn * HD;
    T* dv = ringv + (size_t)ringn * HD;
    for (int i = tid; i < 2 * PPR; i += kThreads) {
      const int k = (i % PPR) * PER;
      if (i < PPR) *reinterpret_cast<u32x4*>(dk + k) = *reinterpret_cast<const u32x4*>(kin + k);
      else *reinterpret_cast<u32x4*>(dv + k) = *reinterpret_cast<const u32x4*>(vin + k);
    }
  }
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
  if (a.kc < 32 || a.nslot < 1) return hipErrorInvalidValue;
  const size_t lds = dec_layout(a.lam, HD, a.g, (int)sizeof(typename DT::T), a.kc, a.nslot).total;
  const void* fn = (const void*)decode_kernel<DT, HD>;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_kernel<DT, HD>), dim3(U), dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int U, bool f32, hipStream_t st) {
  if (U <= 0) return hipSuccess;
  if (a.d == 128) return f32 ? launch_decode_t<F32, 128>(a, U, st) : launch_decode_t<BF16, 128>(a, U, st);
  return f32 ? launch_decode_t<F32, 64>(a, U, st) : launch_decode_t<BF16, 64>(a, U, st);
}

}  // namespace lola
