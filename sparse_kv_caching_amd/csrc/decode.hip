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
// The step is bound by HBM traffic (H, s, window and cache K/V are read once,
// H and s written once), so the dense products are kept on MFMA: phi of the
// lam + 1 candidates and g queries (x W), and one GEMM H^T [phi_E | phi_q]
// (hi/lo 16-bit split, as in the chain kernel) that gives both the SRE
// predictions and the linear read.  Attention over <= lam + eta + 1 keys for g
// heads is small and runs on the VALU.
#include "internal.h"

namespace lola {

namespace {
constexpr int kThreads = 256;
constexpr int WP = 8;                // W^T row padding (bf16)

// Byte offsets of the LDS arrays.
struct DecLayout {
  uint32_t WT_hi, WT_lo, s, q, lk, lv, nlin, zq, spart, keys, phe, logit, misc, total;
};

inline __host__ __device__ uint32_t al16(uint32_t x) { return (x + 15u) & ~15u; }

__host__ __device__ inline DecLayout dec_layout(int lam, int eta, int d, int g, bool f32) {
  DecLayout L;
  uint32_t off = 0;
  auto take = [&](uint32_t b) { const uint32_t o = off; off = al16(off + b); return o; };
  L.WT_hi = take((uint32_t)kM * (d + WP) * 2);         // [kM][d + WP]
  L.WT_lo = take(f32 ? (uint32_t)kM * (d + WP) * 2 : 16);
  L.s = take(kD * 4);                                  // [kD]
  L.q = take((uint32_t)g * d * 4);                     // [g][d]
  L.lk = take((uint32_t)d * 4);                        // leaving key [d]
  L.lv = take((uint32_t)d * 4);                        // leaving value [d]
  L.nlin = take((uint32_t)g * d * 4);                  // [g][d] H^T phi(q)
  L.zq = take(16 * 4);                                 // [g]
  L.spart = take(4 * 32 * 4);                          // [4][32]
  L.keys = take((uint32_t)(lam + 1) * 8);              // [lam + 1]
  L.phe = take(kD * 4);                                // phi of the folded row
  L.logit = take((uint32_t)g * (lam + eta + 1) * 4);   // [g][lam + eta + 1]
  L.misc = take(8 * 4);
  L.total = off;
  return L;
}

__device__ __forceinline__ float ldx(const uint16_t* p) { return bf16_bits_to_f32(*p); }
__device__ __forceinline__ float ldx(const float* p) { return *p; }
__device__ __forceinline__ void stx(uint16_t* p, float x) { *p = (uint16_t)f32_to_bf16_bits(x); }
__device__ __forceinline__ void stx(float* p, float x) { *p = x; }

}  // namespace

size_t decode_lds_bytes(int lam, int eta, int d, int g, bool f32) {
  return dec_layout(lam, eta, d, g, f32).total;
}

template <class DT>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
  using T = typename DT::T;
  const int u = blockIdx.x, d = a.d, lam = a.lam, eta = a.eta, g = a.g;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, r = lane & 31;
  const int kvh = u % a.Hkv;
  const long long n = a.n;
  const int gs = (int)min((long long)lam, max(0LL, n - eta));
  const bool has_leave = n >= eta;                 // eta == 0: the new pair leaves at once
  const bool full = has_leave && gs + 1 > lam;     // score and fold
  const int nslab = d / 32;

  extern __shared__ __align__(16) unsigned char smem[];
  const DecLayout L = dec_layout(lam, eta, d, g, DT::kSplit);
  struct {
    uint16_t *WT_hi, *WT_lo;
    float *s, *q, *lk, *lv, *nlin, *zq, *spart;
    uint64_t* keys;
    float *phe, *logit;
    int32_t* misc;
  } sm = {(uint16_t*)(smem + L.WT_hi), (uint16_t*)(smem + L.WT_lo), (float*)(smem + L.s),
          (float*)(smem + L.q), (float*)(smem + L.lk), (float*)(smem + L.lv),
          (float*)(smem + L.nlin), (float*)(smem + L.zq), (float*)(smem + L.spart),
          (uint64_t*)(smem + L.keys), (float*)(smem + L.phe), (float*)(smem + L.logit),
          (int32_t*)(smem + L.misc)};

  const T* Wg = reinterpret_cast<const T*>(a.W) + (size_t)kvh * d * kM;
  for (int i = tid; i < d * kM; i += kThreads) {
    const int k = i / kM, f = i % kM;
    uint32_t hi, lo;
    DT::split(DT::to_f32(Wg[i]), hi, lo);
    sm.WT_hi[f * (d + WP) + k] = (uint16_t)hi;
    if (DT::kSplit) sm.WT_lo[f * (d + WP) + k] = (uint16_t)lo;
  }
  for (int F = tid; F < kD; F += kThreads) sm.s[F] = a.s[(size_t)u * kD + F];
  const T* qg = reinterpret_cast<const T*>(a.q) + (size_t)u * a.q_su;
  for (int i = tid; i < g * d; i += kThreads) sm.q[i] = DT::to_f32(qg[(size_t)(i / d) * a.q_sh + i % d]);
  const T* kin = reinterpret_cast<const T*>(a.k) + (size_t)u * a.kv_su;
  const T* vin = reinterpret_cast<const T*>(a.v) + (size_t)u * a.kv_su;
  T* ringk = reinterpret_cast<T*>(a.ring_k);
  T* ringv = reinterpret_cast<T*>(a.ring_v);
  T* ck = reinterpret_cast<T*>(a.cache_k);
  T* cv = reinterpret_cast<T*>(a.cache_v);
  if (has_leave) {
    const T* srck = eta > 0 ? ringk + ((size_t)u * eta + (size_t)((n - eta) % eta)) * d : kin;
    const T* srcv = eta > 0 ? ringv + ((size_t)u * eta + (size_t)((n - eta) % eta)) * d : vin;
    for (int c = tid; c < d; c += kThreads) { sm.lk[c] = DT::to_f32(srck[c]); sm.lv[c] = DT::to_f32(srcv[c]); }
  }
  __syncthreads();

  // H columns [32w, 32w+32): lane (c, h) holds H[16kb + sigma_h(jj)][c]
  const bool has_slab = wave < nslab;
  const int cc = 32 * wave + r;
  float Hs[8][8];
  u32x4 Ahi[8], Alo[8];
  const float* Hg = a.H + (size_t)u * kD * d;
  for (int kb = 0; kb < 8; ++kb) {
    for (int jj = 0; jj < 8; ++jj) {
      const int F = 16 * kb + (jj < 4 ? 4 * h + jj : 8 + 4 * h + jj - 4);
      Hs[kb][jj] = has_slab ? Hg[(size_t)F * d + cc] : 0.f;
    }
    splitop<DT>(Hs[kb], Ahi[kb], Alo[kb]);
  }

  // ---- rows: [0, lam) cache slots, lam = leaving pair, lam + 1 + hd = query hd
  const int nrows = lam + 1 + g;
  for (int t0 = 0; t0 < nrows; t0 += 32) {
    // rows needed in this tile?
    const int row = t0 + r;
    bool need;
    if (row < lam) need = full && row < gs;
    else if (row == lam) need = full;
    else need = row < nrows;
    const bool any = __syncthreads_or(need) != 0;
    if (!any) continue;
    // x row as MFMA B operand (K = d, natural slots)
    const T* xrow = nullptr;
    const float* xl = nullptr;
    if (need) {
      if (row < lam) xrow = ck + ((size_t)u * lam + row) * d;
      else if (row == lam) xl = sm.lk;
      else xl = sm.q + (size_t)(row - lam - 1) * d;
    }
    f32x16 U2[2];
    for (int mt = 0; mt < 2; ++mt) for (int i = 0; i < 16; ++i) U2[mt][i] = 0.f;
    for (int kb = 0; kb < d / 16; ++kb) {
      const int k0 = 16 * kb + 8 * h;
      float x[8];
      if (xrow) load8_f32(xrow + k0, x);
      else if (xl) for (int q = 0; q < 8; ++q) x[q] = xl[k0 + q];
      else for (int q = 0; q < 8; ++q) x[q] = 0.f;
      u32x4 bh, bl;
      splitop<DT>(x, bh, bl);
      for (int mt = 0; mt < 2; ++mt) {
        const int f = 32 * mt + r;
        const u32x4 ah = ld16(sm.WT_hi + f * (d + WP) + k0);
        U2[mt] = DT::mma(ah, bh, U2[mt]);
        if constexpr (DT::kSplit) {
          const u32x4 al = ld16(sm.WT_lo + f * (d + WP) + k0);
          U2[mt] = DT::mma(ah, bl, U2[mt]);
          U2[mt] = DT::mma(al, bh, U2[mt]);
        }
      }
    }
    // softmax halves -> phi (lane: row r, features 64*half + 32mt + 8(i/4) + 4h + (i%4))
    float ph[2][2][16];
    {
      float mx = -INFINITY, mn = INFINITY;
      for (int mt = 0; mt < 2; ++mt)
        for (int i = 0; i < 16; ++i) { mx = fmaxf(mx, U2[mt][i]); mn = fminf(mn, U2[mt][i]); }
      mx = fmaxf(mx, xor32(mx));
      mn = fminf(mn, xor32(mn));
      float sp = 0.f, sn = 0.f;
      for (int mt = 0; mt < 2; ++mt)
        for (int i = 0; i < 16; ++i) {
          ph[0][mt][i] = expf(U2[mt][i] - mx);
          ph[1][mt][i] = expf(mn - U2[mt][i]);
          sp += ph[0][mt][i];
          sn += ph[1][mt][i];
        }
      sp += xor32(sp);
      sn += xor32(sn);
      const float ip = 1.f / sp, in_ = 1.f / sn;
      for (int mt = 0; mt < 2; ++mt)
        for (int i = 0; i < 16; ++i) { ph[0][mt][i] *= ip; ph[1][mt][i] *= in_; }
    }
    // z = phi^T s  (the hi + lo value the GEMM sees)
    float z = 0.f;
    u32x4 Bh[8], Bl[8];
    for (int kb = 0; kb < 8; ++kb) {
      const int half = kb >> 2, mt = (kb & 3) >> 1, i0 = 8 * (kb & 1);
      uint32_t hb[8], lb[8];
      for (int jj = 0; jj < 8; ++jj) {
        DT::split(ph[half][mt][i0 + jj], hb[jj], lb[jj]);
        const int F = 16 * kb + (jj < 4 ? 4 * h + jj : 8 + 4 * h + jj - 4);
        z = fmaf(DT::from_bits(hb[jj]) + DT::from_bits(lb[jj]), sm.s[F], z);
      }
      Bh[kb] = pack8(hb);
      Bl[kb] = pack8(lb);
    }
    z += xor32(z);
    // P^T[c][row] = (H^T phi)[c] for this wave's 32 columns
    f32x16 P;
    for (int i = 0; i < 16; ++i) P[i] = 0.f;
    if (has_slab) {
      for (int kb = 0; kb < 8; ++kb) {
        P = DT::mma(Ahi[kb], Bh[kb], P);
        P = DT::mma(Ahi[kb], Bl[kb], P);
        P = DT::mma(Alo[kb], Bh[kb], P);
      }
    }
    // candidate rows: partial SRE over this wave's columns; query rows: keep N_lin
    float part = 0.f;
    if (has_slab && need) {
      if (row <= lam) {
        const float iz = z > 0.f ? 1.f / z : 0.f;
        for (int g4 = 0; g4 < 4; ++g4)
          for (int q = 0; q < 4; ++q) {
            const int c = 32 * wave + 8 * g4 + 4 * h + q;
            const float vv = row < lam ? DT::to_f32(cv[((size_t)u * lam + row) * d + c]) : sm.lv[c];
            const float p = z > 0.f ? P[4 * g4 + q] * iz : 0.f;
            part = fmaf(p - vv, p - vv, part);
          }
      } else {
        const int hd = row - lam - 1;
        for (int g4 = 0; g4 < 4; ++g4)
          for (int q = 0; q < 4; ++q) {
            const int c = 32 * wave + 8 * g4 + 4 * h + q;
            sm.nlin[hd * d + c] = P[4 * g4 + q];
          }
        if (wave == 0 && h == 0) sm.zq[hd] = z;
      }
    }
    part += xor32(part);
    if (h == 0) sm.spart[wave * 32 + r] = part;
    __syncthreads();
    if (tid < 32) {
      const int rw = t0 + tid;
      if (rw <= lam && rw < nrows) {
        bool nd = rw < lam ? (full && rw < gs) : full;
        if (nd) {
          float sre = 0.f;
          for (int w = 0; w < nslab; ++w) sre += sm.spart[w * 32 + tid];
          const long long pos = rw < lam ? (long long)a.cache_pos[(size_t)u * lam + rw] : n - eta;
          sm.keys[rw] = ((uint64_t)__float_as_uint(sre) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)pos);
        }
      }
    }
    __syncthreads();
  }

  // ---- argmin: the candidate to fold (lowest SRE; equal SRE -> newer position)
  if (full && wave == 0) {
    uint64_t best = ~0ull;
    int bi = lam;
    for (int e = lane; e <= lam; e += 64) {
      const uint64_t k = sm.keys[e];
      if (k < best) { best = k; bi = e; }
    }
    for (int o = 32; o > 0; o >>= 1) {
      const uint64_t ob = __shfl_xor(best, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (ob < best) { best = ob; bi = oi; }
    }
    if (lane == 0) sm.misc[0] = bi;
  }

  // ---- attention for the g heads (VALU), merged with the linear read
  const int w_len = (int)min((long long)eta, n);    // window positions n - w_len .. n - 1
  const int nk = gs + w_len + 1;
  const float scale = 1.f / sqrtf((float)d);
  for (int hd = wave; hd < g; hd += kThreads / 64) {
    const float* qv = sm.q + (size_t)hd * d;
    float* lg = sm.logit + (size_t)hd * (lam + eta + 1);
    float mloc = 0.f;   // running max starts at 0 (linear terms unscaled when no logit is > 0)
    for (int kk = lane; kk < nk; kk += 64) {
      const T* krow;
      if (kk < gs) krow = ck + ((size_t)u * lam + kk) * d;
      else if (kk < gs + w_len) krow = ringk + ((size_t)u * eta + (size_t)((n - w_len + (kk - gs)) % eta)) * d;
      else krow = kin;
      float dot = 0.f;
      for (int c = 0; c < d; c += 8) {
        float x[8];
        load8_f32(krow + c, x);
        for (int q = 0; q < 8; ++q) dot = fmaf(qv[c + q], x[q], dot);
      }
      lg[kk] = dot * scale;
      mloc = fmaxf(mloc, dot * scale);
    }
    __threadfence_block();
    for (int o = 32; o > 0; o >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, o, 64));
    float lsum = 0.f;
    for (int kk = lane; kk < nk; kk += 64) {
      const float p = expf(lg[kk] - mloc);
      lg[kk] = p;
      lsum += p;
    }
    lsum = wave_sum(lsum);
    __threadfence_block();   // other lanes' p values are read below
    const float em = expf(-mloc);
    const float l = lsum + em * sm.zq[hd];
    float* orow = a.out + (size_t)u * a.o_su + (size_t)hd * a.o_sh;
    for (int c = lane; c < d; c += 64) {
      float acc = em * sm.nlin[hd * d + c];
      for (int kk = 0; kk < nk; ++kk) {
        const T* vrow;
        if (kk < gs) vrow = cv + ((size_t)u * lam + kk) * d;
        else if (kk < gs + w_len) vrow = ringv + ((size_t)u * eta + (size_t)((n - w_len + (kk - gs)) % eta)) * d;
        else vrow = vin;
        acc = fmaf(lg[kk], ldx(vrow + c), acc);
      }
      orow[c] = acc / l;
    }
  }
  __syncthreads();   // every read of H, cache and ring is done

  // ---- update: cache / fold, then the ring
  if (has_leave) {
    int fold_row = -1;        // row index: < lam cache slot, == lam the leaving pair
    int slot_in = -1;         // cache slot receiving the leaving pair
    if (!full) slot_in = gs;
    else {
      fold_row = sm.misc[0];
      if (fold_row < lam) slot_in = fold_row;
    }
    if (slot_in >= 0) {
      // the folded cache row must be read (below) before it is overwritten
    }
    if (fold_row >= 0) {
      // phi of the folded row on the VALU, wave 0: lane = feature f of a half
      if (wave == 0) {
        const T* krow = fold_row < lam ? ck + ((size_t)u * lam + fold_row) * d : nullptr;
        float uacc = 0.f;
        for (int k = 0; k < d; ++k) {
          const float x = krow ? DT::to_f32(krow[k]) : sm.lk[k];
          float w = DT::from_bits(sm.WT_hi[lane * (d + WP) + k]);
          if (DT::kSplit) w += DT::from_bits(sm.WT_lo[lane * (d + WP) + k]);
          uacc = fmaf(x, w, uacc);
        }
        float mx = uacc, mn = uacc;
        for (int o = 32; o > 0; o >>= 1) {
          mx = fmaxf(mx, __shfl_xor(mx, o, 64));
          mn = fminf(mn, __shfl_xor(mn, o, 64));
        }
        const float ep = expf(uacc - mx), en = expf(mn - uacc);
        const float sp = wave_sum(ep), sn = wave_sum(en);
        sm.phe[lane] = ep / sp;
        sm.phe[kM + lane] = en / sn;
      }
      __syncthreads();
      // H[F][c] += phi_e[F] v_e[c]   (this wave's slab), written back
      if (has_slab) {
        const float ve = fold_row < lam ? DT::to_f32(cv[((size_t)u * lam + fold_row) * d + cc]) : sm.lv[cc];
        float* Ho = a.H + (size_t)u * kD * d;
        for (int kb = 0; kb < 8; ++kb)
          for (int jj = 0; jj < 8; ++jj) {
            const int F = 16 * kb + (jj < 4 ? 4 * h + jj : 8 + 4 * h + jj - 4);
            Ho[(size_t)F * d + cc] = fmaf(sm.phe[F], ve, Hs[kb][jj]);
          }
      }
      for (int F = tid; F < kD; F += kThreads) a.s[(size_t)u * kD + F] = sm.s[F] + sm.phe[F];
      __syncthreads();
    }
    if (slot_in >= 0) {
      T* dk = ck + ((size_t)u * lam + slot_in) * d;
      T* dv = cv + ((size_t)u * lam + slot_in) * d;
      for (int c = tid; c < d; c += kThreads) { stx(dk + c, sm.lk[c]); stx(dv + c, sm.lv[c]); }
      if (tid == 0) a.cache_pos[(size_t)u * lam + slot_in] = (int32_t)(n - eta);
    }
  }
  if (eta > 0) {
    T* dk = ringk + ((size_t)u * eta + (size_t)(n % eta)) * d;
    T* dv = ringv + ((size_t)u * eta + (size_t)(n % eta)) * d;
    for (int c = tid; c < d; c += kThreads) { dk[c] = kin[c]; dv[c] = vin[c]; }
  }
}

hipError_t launch_decode(const DecodeArgs& a, int U, bool f32, hipStream_t st) {
  if (U <= 0) return hipSuccess;
  size_t lds = decode_lds_bytes(a.lam, a.eta, a.d, a.g, f32);
  if (f32) {
    (void)hipFuncSetAttribute((const void*)decode_kernel<F32>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL(decode_kernel<F32>, dim3(U), dim3(kThreads), lds, st, a);
  } else {
    (void)hipFuncSetAttribute((const void*)decode_kernel<BF16>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL(decode_kernel<BF16>, dim3(U), dim3(kThreads), lds, st, a);
  }
  return hipGetLastError();
}

}  // namespace lola
