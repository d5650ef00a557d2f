// The accumulated cache scoring rules (LoLA notes §4.5, Table 4, an ablation
// of the rule that decides which pairs stay cached): a key's score sums a
// term over the local queries that see it through the sliding window,
// e = exp(q.k / sqrt(d)) the exponential kernel and c = phi(q)^T phi(k) the
// feature kernel of one (query, key) pair:
//   LOLA_SCORE_KERNEL_SQ    (e - c)^2
//   LOLA_SCORE_KERNEL_ABS   |e - c|
//   LOLA_SCORE_KERNEL_RATIO c / e
//   LOLA_SCORE_LOCAL_ATTN   e
// summed over every query head of the key's KV head, and frozen when the key
// leaves the window.  Query t (chunk start n_t) sees the local key at
// position i iff max(0, n_t - eta) <= i <= t.
//
// One workgroup per (unit, block of 32 local keys: the window at the call's
// start, then the call's own keys).  The call's queries that can see any key
// of the block are taken 8 positions at a time, with phi(q) for them and
// all query heads formed in LDS; eight lanes per key split the dot products
// and sum them in a fixed order, and every key adds its terms query by
// query, head by head, so the sums are the same on every run.  fp32 on the
// vector units: this is an ablation path, not one of the tuned kernels.
#include "internal.h"

namespace lola {

namespace {
constexpr int kThreads = 256;
constexpr int KBLK = 32;     // keys per workgroup
constexpr int LPK = kThreads / KBLK;   // lanes per key
constexpr int QT = 8;        // query positions per staged tile
constexpr int QR = QT * 4;   // staged query rows (positions x at most 4 heads)

// LDS layout (floats), rows padded by one
template <int HD> struct ScoreLds {
  static constexpr int k = 0;                             // [KBLK][HD + 1] keys
  static constexpr int fk = k + KBLK * (HD + 1);          // [KBLK][kD + 1] phi of the keys
  static constexpr int q = fk + KBLK * (kD + 1);          // [QR][HD + 1] queries
  static constexpr int uq = q + QR * (HD + 1);            // [QR][kM + 1] q W
  static constexpr int fq = uq + QR * (kM + 1);           // [QR][kD + 1] phi(q)
  static constexpr int w = fq + QR * (kD + 1);            // [HD][kM + 1] W of the KV head
  static constexpr int total = w + HD * (kM + 1);
};
}  // namespace

size_t score_lds_bytes(int d) {
  return (d == 128 ? ScoreLds<128>::total : ScoreLds<64>::total) * sizeof(float);
}

template <class DT, int HD>
__global__ __launch_bounds__(kThreads) void score_kernel(ScoreArgs a) {
  using T = typename DT::T;
  const VirtRows vr = a.vr;
  const int u = blockIdx.y, tid = threadIdx.x;
  const int g = a.g, eta = vr.eta, C = a.C;
  const int kvh = u % a.Hkv;
  const long long n0 = vr.n0, nend = n0 + vr.T;
  const int nloc = eta + vr.T;                       // local rows: window, then the call
  const int kv0 = blockIdx.x * KBLK;
  const long long pos0 = n0 - eta + kv0;             // position of local row kv0

  extern __shared__ __align__(16) float lds[];
  using Ly = ScoreLds<HD>;
  auto sk = reinterpret_cast<float(*)[HD + 1]>(lds + Ly::k);
  auto sfk = reinterpret_cast<float(*)[kD + 1]>(lds + Ly::fk);
  auto sq = reinterpret_cast<float(*)[HD + 1]>(lds + Ly::q);   // row = position x g + head
  auto su = reinterpret_cast<float(*)[kM + 1]>(lds + Ly::uq);
  auto sfq = reinterpret_cast<float(*)[kD + 1]>(lds + Ly::fq);
  auto sw = reinterpret_cast<float(*)[kM + 1]>(lds + Ly::w);

  // stage the block's keys and their phi (rows of negative positions or past
  // the call stay zero and are never scored)
  for (int i = tid; i < KBLK * HD; i += kThreads) {
    const int kk = i / HD, c = i % HD, kv = kv0 + kk;
    const long long p = pos0 + kk;
    float x = 0.f;
    if (kv < nloc && p >= 0)
      x = DT::to_f32(reinterpret_cast<const T*>(vr.krow(u, vr.lam + kv, sizeof(T)))[c]);
    sk[kk][c] = x;
  }
  for (int i = tid; i < KBLK * kD; i += kThreads) {
    const int kk = i / kD, f = i % kD, kv = kv0 + kk;
    const long long p = pos0 + kk;
    float x = 0.f;
    if (kv < nloc && p >= 0) {
      const size_t o = ((size_t)u * a.NV + vr.lam + kv) * kD + f;
      x = DT::from_bits(a.phi_hi[o]) + DT::from_bits(a.phi_lo[o]);
    }
    sfk[kk][f] = x;
  }
  const T* W = reinterpret_cast<const T*>(a.W) + (size_t)kvh * HD * kM;
  for (int i = tid; i < HD * kM; i += kThreads) sw[i / kM][i % kM] = DT::to_f32(W[i]);

  // the call's queries that can see a key of the block: from the block's
  // first position (or n0) to the end of the chunk holding its last position
  // + eta (or the call's end)
  const long long plast = min(pos0 + KBLK - 1, nend - 1);
  long long q_lo = max(n0, pos0), q_hi;
  {
    const long long x = plast + eta;
    q_hi = x >= nend ? nend : min(nend, n0 + (long long)C * ((x - n0) / C + 1));
  }
  const int kk = tid / LPK, part = tid % LPK;         // LPK lanes per key
  const long long pk = pos0 + kk;
  const bool kvalid = kv0 + kk < nloc && pk >= 0;
  const float rs = 1.f / sqrtf((float)HD);
  float acc = 0.f;
  __syncthreads();

  for (long long qp0 = q_lo; qp0 < q_hi; qp0 += QT) {
    const int nq = (int)min((long long)QT, q_hi - qp0);
    const int rows = nq * g;                         // row r = (position r / g, head r % g)
    __syncthreads();                                 // the previous tile is consumed
    for (int i = tid; i < rows * HD; i += kThreads) {
      const int r = i / HD, c = i % HD;
      const long long p = qp0 + r / g;
      const int hd = r % g;
      sq[r][c] = DT::to_f32(reinterpret_cast<const T*>(a.q)[(((size_t)u * g + hd) * vr.T +
                                                             (size_t)(p - n0)) * HD + c]);
    }
    __syncthreads();
    for (int i = tid; i < rows * kM; i += kThreads) {
      const int r = i / kM, f = i % kM;
      float x = 0.f;
      for (int c = 0; c < HD; ++c) x = fmaf(sq[r][c], sw[c][f], x);
      su[r][f] = x;
    }
    __syncthreads();
    // phi(q) = [softmax(u), softmax(-u)]: one thread per (row, half)
    for (int i = tid; i < rows * 2; i += kThreads) {
      const int r = i >> 1, half = i & 1;
      float mx = -INFINITY;
      for (int f = 0; f < kM; ++f) mx = fmaxf(mx, half ? -su[r][f] : su[r][f]);
      float sum = 0.f;
      for (int f = 0; f < kM; ++f) {
        const float e = expf((half ? -su[r][f] : su[r][f]) - mx);
        sfq[r][kM * half + f] = e;
        sum += e;
      }
      const float inv = 1.f / sum;
      for (int f = 0; f < kM; ++f) sfq[r][kM * half + f] *= inv;
    }
    __syncthreads();
    for (int r = 0; r < rows; ++r) {
      const long long p = qp0 + r / g;
      // dot products over this lane's quarter of the dimensions and features
      float qk = 0.f, ff = 0.f;
      for (int c = part; c < HD; c += LPK) qk = fmaf(sq[r][c], sk[kk][c], qk);
      for (int f = part; f < kD; f += LPK) ff = fmaf(sfq[r][f], sfk[kk][f], ff);
#pragma unroll
      for (int o = 1; o < LPK; o <<= 1) {
        qk += __shfl_xor(qk, o, 64);
        ff += __shfl_xor(ff, o, 64);
      }
      const long long nt = n0 + (long long)C * ((p - n0) / C);   // chunk start of p
      const bool vis = kvalid && pk <= p && pk >= nt - eta;
      if (vis) {
        const float e = expf(qk * rs);
        float t;
        switch (a.rule) {
          case LOLA_SCORE_KERNEL_SQ: t = (e - ff) * (e - ff); break;
          case LOLA_SCORE_KERNEL_ABS: t = fabsf(e - ff); break;
          case LOLA_SCORE_KERNEL_RATIO: t = ff / e; break;
          default: t = e; break;
        }
        acc += t;
      }
    }
  }
  if (part == 0 && kv0 + kk < nloc) {
    float total = acc;
    if (kvalid && pk < n0) total += a.ring_score[(size_t)u * eta + (size_t)(pk % eta)];
    a.vscore[(size_t)u * nloc + kv0 + kk] = kvalid ? total : 0.f;
  }
}

// After the chain: the new cache's frozen scores (in the new cache's slot
// order) and the running scores of the window.
__global__ __launch_bounds__(kThreads) void score_writeback_kernel(ScoreWriteArgs a) {
  if (__builtin_amdgcn_readfirstlane(*reinterpret_cast<volatile const int*>(a.err)) != 0) return;
  const VirtRows vr = a.vr;
  const int u = blockIdx.x, lam = vr.lam, eta = vr.eta;
  const int nloc = eta + vr.T;
  const long long nend = vr.n0 + vr.T;
  for (int i = threadIdx.x; i < lam; i += kThreads) {
    float x = 0.f;
    if (i < a.gs_final) {
      const int vi = a.finalG[(size_t)u * lam + i];
      x = vi < lam ? a.cscore_in[(size_t)u * lam + vi] : a.vscore[(size_t)u * nloc + (vi - lam)];
    }
    a.cscore_out[(size_t)u * lam + i] = x;
  }
  const long long p_lo = max(0LL, nend - eta);
  for (long long p = p_lo + threadIdx.x; p < nend; p += kThreads)
    a.ring_score[(size_t)u * eta + (size_t)(p % eta)] =
        a.vscore[(size_t)u * nloc + (size_t)(p - (vr.n0 - eta))];
}

hipError_t launch_score(const ScoreArgs& a, int U, bool f32, hipStream_t st) {
  const int nloc = a.vr.eta + a.vr.T;
  if (U <= 0 || nloc <= 0) return hipSuccess;
  if (a.g < 1 || a.g > 4) return hipErrorInvalidValue;
  const dim3 grid((nloc + KBLK - 1) / KBLK, U);
  const size_t lds = score_lds_bytes(a.vr.d);
  const void* fn = a.vr.d == 128
      ? (f32 ? (const void*)score_kernel<F32, 128> : (const void*)score_kernel<BF16, 128>)
      : (f32 ? (const void*)score_kernel<F32, 64> : (const void*)score_kernel<BF16, 64>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  if (a.vr.d == 128) {
    if (f32) hipLaunchKernelGGL((score_kernel<F32, 128>), grid, dim3(kThreads), lds, st, a);
    else hipLaunchKernelGGL((score_kernel<BF16, 128>), grid, dim3(kThreads), lds, st, a);
  } else {
    if (f32) hipLaunchKernelGGL((score_kernel<F32, 64>), grid, dim3(kThreads), lds, st, a);
    else hipLaunchKernelGGL((score_kernel<BF16, 64>), grid, dim3(kThreads), lds, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_score_writeback(const ScoreWriteArgs& a, int U, hipStream_t st) {
  if (U <= 0) return hipSuccess;
  hipLaunchKernelGGL(score_writeback_kernel, dim3(U), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace lola
