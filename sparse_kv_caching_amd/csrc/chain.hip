// K2: the chain kernel (its body, and the notes on what it computes, are
// in chain_impl.h) and its launchers.
#include "chain_impl.h"

namespace lola {

size_t chain_lds_bytes(int lam, int C, int d, bool f32) {
  // the largest of the instances the library can launch: one slab per
  // workgroup and two slabs (two fold buffers), all slabs (one)
  const int nslab = d / 32;
  size_t m = chain_ns::chain_layout(lam, C, nslab, f32, 1).total;
  for (int spw = 1; spw < nslab; spw *= 2) {
    const size_t x = chain_ns::chain_layout(lam, C, spw, f32, 2).total;
    if (x > m) m = x;
  }
  return m;
}

template <class DT, int HD, int SPW, bool XS>
__global__ __launch_bounds__(chain_ns::kThreads) void chain_kernel(ChainArgs a) {
  chain_body<DT, HD, SPW, XS>(a, blockIdx.x);
}

// LDS layout of the candidate split (every workgroup holding all slabs)
size_t chain_split_lds_bytes(int lam, int C, int d, bool f32) {
  return chain_ns::chain_layout(lam, C, d / 32, f32, 1, true).total;
}

template <class DT, int HD, int SPW, bool XS = false>
static hipError_t launch_chain_t(const ChainArgs& a, int U, hipStream_t st) {
  const size_t lds =
      chain_ns::chain_layout(a.vr.lam, a.C, SPW, DT::kSplit, chain_ns::kFoldBufs<HD, SPW>, XS).total;
  const void* fn = (const void*)chain_kernel<DT, HD, SPW, XS>;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((chain_kernel<DT, HD, SPW, XS>), dim3(U * a.k), dim3(chain_ns::kThreads), lds, st, a);
  return hipGetLastError();
}

// k >= NSLAB: one column slab per workgroup; k == 2 (NSLAB = 4): two; k == 1:
// all of them (the only instance that exchanges nothing); the candidate split:
// all of them, k candidate groups
template <class DT, int HD>
static hipError_t launch_chain_k(const ChainArgs& a, int U, hipStream_t st) {
  constexpr int NSLAB = HD / 32;
  if (a.xs && a.k > 1) return launch_chain_t<DT, HD, NSLAB, true>(a, U, st);
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
