// K3: the attention kernel (its body, and the notes on what it computes,
// are in attn_impl.h) and its launchers.
#include "attn_impl.h"

namespace lola {

size_t attn_lds_bytes(int d, int lam, int eta, int C, bool f32) {
  return attn_ns::attn_layout(d, lam, eta, C, f32).total;
}

bool attn_wide_table(int d, int lam, int eta, int C, bool f32) {
  return attn_ns::attn_layout(d, lam, eta, C, f32).wide;
}

template <class DT, int HD, bool WIDE>
__global__ __launch_bounds__(attn_ns::kThreads) void attn_kernel(AttnArgs a) {
  attn_body<DT, HD, WIDE>(a, blockIdx.x, blockIdx.y, blockIdx.z);
}

template <class DT, int HD, bool WIDE>
static hipError_t launch_attn_w(const AttnArgs& a, int U, size_t lds, hipStream_t st) {
  const int nptile = (a.C + a.ptile - 1) / a.ptile;
  dim3 grid(U, a.nch_launch, nptile);
  const void* fn = (const void*)attn_kernel<DT, HD, WIDE>;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_kernel<DT, HD, WIDE>), grid, dim3(attn_ns::kThreads), lds, st, a);
  return hipGetLastError();
}

template <class DT, int HD>
static hipError_t launch_attn_t(const AttnArgs& a, int U, hipStream_t st) {
  const attn_ns::AttnLayout L = attn_ns::attn_layout(HD, a.vr.lam, a.vr.eta, a.C, DT::kSplit);
  return L.wide ? launch_attn_w<DT, HD, true>(a, U, L.total, st)
                : launch_attn_w<DT, HD, false>(a, U, L.total, st);
}

int attn_positions_per_block(int C, int g) {
  const int p = 32 * attn_ns::kWaves / g;
  return C < p ? (C + 31) / 32 * 32 : p;
}

hipError_t launch_attn(const AttnArgs& a, int U, bool f32, hipStream_t st) {
  if (U <= 0 || a.nch_launch <= 0) return hipSuccess;
  if (a.ch0 < 0 || a.ch0 + a.nch_launch > a.nch) return hipErrorInvalidValue;
  if (a.vr.d == 64)
    return f32 ? launch_attn_t<F32, 64>(a, U, st) : launch_attn_t<BF16, 64>(a, U, st);
  return f32 ? launch_attn_t<F32, 128>(a, U, st) : launch_attn_t<BF16, 128>(a, U, st);
}

}  // namespace lola
