// Diagnostics of a prefill call: the Self-Recall Error of every memory inside
// the linear state at the start of every chunk (LoLA notes §4.4, Fig. 3: the
// SRE of Eq. (10) of the pairs already written to H, s, chunk by chunk; the
// relative SRE of Eq. (26) is this minus its value at the first chunk whose
// state holds the pair).
//
// One workgroup per (unit, chunk j): H_j^T is rebuilt in fp32 from the
// chunk's hi/lo snapshot planes into LDS, then every thread takes call
// tokens p and, for those the chain folded before chunk j, evaluates
//   z = phi(k_p)^T s_j,  P = H_j^T phi(k_p) / z  (0 when z = 0),
//   SRE = sum_c (P_c - v_pc)^2
// with phi(k_p) = hi + lo from the phi planes; fp32 throughout.  Tokens not
// in the state (window, cache, or folded later) get 0.
#include "internal.h"

namespace lola {

namespace {

constexpr int kThreads = 256;

template <class DT, int HD>
__global__ __launch_bounds__(kThreads) void sre_map_kernel(SreMapArgs a) {
  using T = typename DT::T;
  const VirtRows vr = a.vr;
  // the chain gave up: the snapshots and fold chunks were not written
  if (__builtin_amdgcn_readfirstlane(*reinterpret_cast<volatile const int*>(a.err)) != 0) return;
  const int u = blockIdx.x, j = blockIdx.y, tid = threadIdx.x;
  const int lam = vr.lam, eta = vr.eta, Tn = vr.T;
  extern __shared__ __align__(16) unsigned char smem[];
  float* Ht = reinterpret_cast<float*>(smem);     // [HD][kD]
  float* sj = Ht + HD * kD;                        // [kD]
  const uint16_t* snap = a.snapHT + ((size_t)u * a.nch + j) * 2 * HD * kD;
  for (int i = tid; i < HD * kD; i += kThreads)
    Ht[i] = DT::from_bits(snap[i]) + DT::from_bits(snap[HD * kD + i]);
  for (int F = tid; F < kD; F += kThreads) sj[F] = a.snaps[((size_t)u * a.nch + j) * kD + F];
  __syncthreads();
  const int32_t* fold = a.fold + (size_t)u * Tn;
  float* out = a.out + ((size_t)u * a.nch + j) * Tn;
  for (int p = tid; p < Tn; p += kThreads) {
    const int fc = fold[p];
    float sre = 0.f;
    if (fc >= 0 && fc < j) {
      const int vi = lam + eta + p;                // the call's token p
      const size_t prow = ((size_t)u * a.NV + vi) * kD;
      float ph[kD];
      float z = 0.f;
#pragma unroll
      for (int f = 0; f < kD; ++f) {
        ph[f] = DT::from_bits(a.phi_hi[prow + f]) + DT::from_bits(a.phi_lo[prow + f]);
        z = fmaf(ph[f], sj[f], z);
      }
      const float iz = z > 0.f ? 1.f / z : 0.f;
      const T* vrow = reinterpret_cast<const T*>(vr.vrow(u, vi, sizeof(T)));
      for (int c = 0; c < HD; ++c) {
        float pc = 0.f;
#pragma unroll
        for (int f = 0; f < kD; ++f) pc = fmaf(ph[f], Ht[c * kD + f], pc);
        const float e = pc * iz - DT::to_f32(vrow[c]);
        sre = fmaf(e, e, sre);
      }
    }
    out[p] = sre;
  }
}

template <class DT, int HD>
hipError_t launch_sre_map_t(const SreMapArgs& a, int U, hipStream_t st) {
  const size_t lds = ((size_t)HD * kD + kD) * sizeof(float);
  const void* fn = (const void*)sre_map_kernel<DT, HD>;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((sre_map_kernel<DT, HD>), dim3(U, a.nch), dim3(kThreads), lds, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sre_map(const SreMapArgs& a, int U, bool f32, hipStream_t st) {
  if (U <= 0 || a.nch <= 0 || a.vr.T <= 0) return hipSuccess;
  if (a.vr.d == 64)
    return f32 ? launch_sre_map_t<F32, 64>(a, U, st) : launch_sre_map_t<BF16, 64>(a, U, st);
  return f32 ? launch_sre_map_t<F32, 128>(a, U, st) : launch_sre_map_t<BF16, 128>(a, U, st);
}

}  // namespace lola
