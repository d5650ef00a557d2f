// The chain (K2) and the read of finished chunks (K3) in one launch.
//
// The read of chunk j only needs the snapshot the chain writes at step j
// (LoLA notes §2.6: every chunk reads the state at its start), so it can run
// while the chain is still on later chunks.  The chain is a serial
// recurrence that keeps a fixed set of workgroups busy; with half of the
// compute units given to it, the other half reads the chunks it has
// finished.  One grid holds both: blocks 0 .. nchain - 1 are the chain's
// workgroups (each takes a compute unit, and they are dispatched before any
// block of the read, so all of them are resident as the chain's exchange
// requires), the rest are the read's workgroups in the order unit, position
// tile, chunk, so that the read advances chunk by chunk behind the chain.
// A read workgroup polls its unit's counter of published snapshots
// (bounded) and reads the snapshot with coherent loads; the chain writes it
// with coherent stores and publishes it after all of them have completed.
#include "attn_impl.h"
#include "chain_impl.h"

namespace lola {

namespace {
struct OverlapArgs {
  ChainArgs c;
  AttnArgs a;
  int nchain;      // chain workgroups (U * k), first in the grid
  int U;           // units
  int nptile;      // position tiles per chunk
};
static_assert(chain_ns::kThreads == attn_ns::kThreads, "one block size for both roles");
}  // namespace

template <class DT, int HD, int SPW, bool XS>
__global__ __launch_bounds__(chain_ns::kThreads) void overlap_kernel(OverlapArgs o) {
  const int b = blockIdx.x;
  if (b < o.nchain) {
    chain_body<DT, HD, SPW, XS>(o.c, b);
    return;
  }
  const int w = b - o.nchain;
  const int u = w % o.U, rest = w / o.U;
  attn_body<DT, HD, true>(o.a, u, rest / o.nptile, rest % o.nptile);
}

template <class DT, int HD, int SPW, bool XS = false>
static hipError_t launch_overlap_t(const OverlapArgs& o, hipStream_t st) {
  const size_t lc =
      chain_ns::chain_layout(o.c.vr.lam, o.c.C, SPW, DT::kSplit, chain_ns::kFoldBufs<HD, SPW>, XS).total;
  // (the read's part: the wide key table; the library takes this schedule
  // only where that layout fits)
  const attn_ns::AttnLayout L = attn_ns::attn_layout(HD, o.a.vr.lam, o.a.vr.eta, o.a.C, DT::kSplit);
  if (!L.wide) return hipErrorInvalidValue;
  const size_t la = L.total;
  const size_t lds = lc > la ? lc : la;
  const void* fn = (const void*)overlap_kernel<DT, HD, SPW, XS>;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int nread = o.U * o.nptile * o.a.nch_launch;
  hipLaunchKernelGGL((overlap_kernel<DT, HD, SPW, XS>), dim3(o.nchain + nread), dim3(chain_ns::kThreads),
                     lds, st, o);
  return hipGetLastError();
}

template <class DT, int HD>
static hipError_t launch_overlap_k(const OverlapArgs& o, hipStream_t st) {
  constexpr int NSLAB = HD / 32;
  if (o.c.xs && o.c.k > 1) return launch_overlap_t<DT, HD, NSLAB, true>(o, st);
  if (o.c.k >= NSLAB) return launch_overlap_t<DT, HD, 1>(o, st);
  if (o.c.k == 1) return launch_overlap_t<DT, HD, NSLAB>(o, st);
  if constexpr (NSLAB == 4) {
    if (o.c.k == 2) return launch_overlap_t<DT, HD, 2>(o, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_overlap(const ChainArgs& c, const AttnArgs& a, int U, bool f32, hipStream_t st) {
  if (U <= 0 || a.nch_launch <= 0) return hipSuccess;
  if (a.ch0 != 0 || a.nch_launch != a.nch || c.j0 != 0 || c.j1 != c.nch || !c.ready ||
      c.ready != a.ready)
    return hipErrorInvalidValue;
  OverlapArgs o;
  o.c = c;
  o.a = a;
  o.nchain = U * c.k;
  o.U = U;
  o.nptile = (a.C + a.ptile - 1) / a.ptile;
  if (a.vr.d == 64)
    return f32 ? launch_overlap_k<F32, 64>(o, st) : launch_overlap_k<BF16, 64>(o, st);
  return f32 ? launch_overlap_k<F32, 128>(o, st) : launch_overlap_k<BF16, 128>(o, st);
}

}  // namespace lola
