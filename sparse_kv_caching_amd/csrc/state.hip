// State maintenance after a prefill call, and the canonical export / import
// layout of the persistent state (window oldest -> newest, cache by position).
//
// The persistent state per unit is the eta-token window, the lam-entry cache,
// H and s: (eta + lam)(d_k + d_v) + D d_v + D elements (LoLA notes §2.7).
#include <algorithm>

#include "internal.h"

namespace lola {

namespace {
constexpr int kThreads = 256;

template <class T>
__device__ void copy_row(T* dst, const T* src, int d) {
  for (int c = threadIdx.x & 63; c < d; c += 64) dst[c] = src[c];
}
}  // namespace

// New cache (compacted into the other buffer), then the window ring, as two
// launches so that every ring row the new cache takes is read before the
// ring is overwritten.  Rows move as 16-byte pieces, many rows per block.
__global__ __launch_bounds__(kThreads) void finalize_cache_kernel(FinalizeArgs a, int esz) {
  // the chain gave up: finalG was not written (the state is poisoned)
  if (__builtin_amdgcn_readfirstlane(*reinterpret_cast<volatile const int*>(a.err)) != 0) return;
  const VirtRows vr = a.vr;
  const int u = blockIdx.y, lam = vr.lam;
  const int pieces = vr.d * esz / 16;                  // 16-byte pieces per row
  const int rows_per_block = kThreads / pieces;
  const int i = blockIdx.x * rows_per_block + threadIdx.x / pieces;
  const int pc = threadIdx.x % pieces;
  if (i >= lam || threadIdx.x >= rows_per_block * pieces) return;
  const size_t dst = ((size_t)u * lam + i) * vr.d * esz + (size_t)pc * 16;
  if (i < a.gs_final) {
    const int vi = a.finalG[(size_t)u * lam + i];
    *reinterpret_cast<u32x4*>((char*)a.new_cache_k + dst) =
        *reinterpret_cast<const u32x4*>(vr.krow(u, vi, esz) + pc * 16);
    *reinterpret_cast<u32x4*>((char*)a.new_cache_v + dst) =
        *reinterpret_cast<const u32x4*>(vr.vrow(u, vi, esz) + pc * 16);
    if (pc == 0) a.new_cache_pos[(size_t)u * lam + i] = (int32_t)vr.pos_of(u, vi);
  } else if (pc == 0) {
    a.new_cache_pos[(size_t)u * lam + i] = -1;
  }
}

__global__ __launch_bounds__(kThreads) void finalize_ring_kernel(FinalizeArgs a, int esz) {
  if (__builtin_amdgcn_readfirstlane(*reinterpret_cast<volatile const int*>(a.err)) != 0) return;
  const VirtRows vr = a.vr;
  const int u = blockIdx.y, eta = vr.eta;
  const long long nend = vr.n0 + vr.T;
  const long long p_lo = max(vr.n0, nend - eta);
  const int pieces = vr.d * esz / 16;
  const int rows_per_block = kThreads / pieces;
  const long long p = p_lo + (long long)blockIdx.x * rows_per_block + threadIdx.x / pieces;
  const int pc = threadIdx.x % pieces;
  if (p >= nend || threadIdx.x >= rows_per_block * pieces) return;
  const size_t row_b = (size_t)vr.d * esz;
  const size_t slot = ((size_t)u * eta + (size_t)(p % eta)) * row_b + (size_t)pc * 16;
  const size_t src = ((size_t)u * vr.T + (size_t)(p - vr.n0)) * row_b + (size_t)pc * 16;
  *reinterpret_cast<u32x4*>((char*)a.ring_k + slot) =
      *reinterpret_cast<const u32x4*>((const char*)vr.in_k + src);
  *reinterpret_cast<u32x4*>((char*)a.ring_v + slot) =
      *reinterpret_cast<const u32x4*>((const char*)vr.in_v + src);
}

hipError_t launch_finalize(const FinalizeArgs& a, int U, bool f32, hipStream_t st) {
  if (U <= 0) return hipSuccess;
  const int esz = f32 ? 4 : 2;
  const int pieces = a.vr.d * esz / 16;
  const int rpb = kThreads / pieces;
  if (a.vr.lam > 0) {
    dim3 g1((a.vr.lam + rpb - 1) / rpb, U);
    hipLaunchKernelGGL(finalize_cache_kernel, g1, dim3(kThreads), 0, st, a, esz);
  }
  if (a.vr.eta > 0) {
    const long long nend = a.vr.n0 + a.vr.T;
    const long long nrows = nend - std::max<long long>(a.vr.n0, nend - a.vr.eta);
    if (nrows > 0) {
      dim3 g2((unsigned)((nrows + rpb - 1) / rpb), U);
      hipLaunchKernelGGL(finalize_ring_kernel, g2, dim3(kThreads), 0, st, a, esz);
    }
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// export: window ring -> oldest..newest rows; cache slots -> ascending
// positions (rank by counting), -1 padding.
template <class T>
__global__ __launch_bounds__(kThreads) void export_kernel(
    const T* ring_k, const T* ring_v, const T* cache_k, const T* cache_v,
    const int32_t* cache_pos, T* win_k, T* win_v, T* out_ck, T* out_cv,
    int32_t* out_pos, long long n, int eta, int lam, int gs, int d) {
  const int u = blockIdx.x, wave = threadIdx.x >> 6;
  const int w = (int)min((long long)eta, n);
  for (int jj = wave; jj < eta; jj += kThreads / 64) {
    T* dk = win_k + ((size_t)u * eta + jj) * d;
    T* dv = win_v + ((size_t)u * eta + jj) * d;
    if (jj < w) {
      const long long p = n - w + jj;
      const size_t slot = (size_t)u * eta + (size_t)(p % eta);
      copy_row(dk, ring_k + slot * d, d);
      copy_row(dv, ring_v + slot * d, d);
    } else {
      for (int c = threadIdx.x & 63; c < d; c += 64) { dk[c] = T(0); dv[c] = T(0); }
    }
  }
  for (int i = wave; i < lam; i += kThreads / 64) {
    if (i >= gs) {
      if ((threadIdx.x & 63) == 0) out_pos[(size_t)u * lam + i] = -1;
      T* dk = out_ck + ((size_t)u * lam + i) * d;
      T* dv = out_cv + ((size_t)u * lam + i) * d;
      for (int c = threadIdx.x & 63; c < d; c += 64) { dk[c] = T(0); dv[c] = T(0); }
      continue;
    }
    const int32_t p = cache_pos[(size_t)u * lam + i];
    int rank = 0;
    for (int o = threadIdx.x & 63; o < gs; o += 64) rank += cache_pos[(size_t)u * lam + o] < p;
    rank = wave_sum_i(rank);
    copy_row(out_ck + ((size_t)u * lam + rank) * d, cache_k + ((size_t)u * lam + i) * d, d);
    copy_row(out_cv + ((size_t)u * lam + rank) * d, cache_v + ((size_t)u * lam + i) * d, d);
    if ((threadIdx.x & 63) == 0) out_pos[(size_t)u * lam + rank] = p;
  }
}

// import: canonical rows -> ring slots / cache slots (cache kept in order)
template <class T>
__global__ __launch_bounds__(kThreads) void import_kernel(
    T* ring_k, T* ring_v, T* cache_k, T* cache_v, int32_t* cache_pos,
    const T* win_k, const T* win_v, const T* in_ck, const T* in_cv,
    const int32_t* in_pos, long long n, int eta, int lam, int gs, int d) {
  const int u = blockIdx.x, wave = threadIdx.x >> 6;
  const int w = (int)min((long long)eta, n);
  for (int jj = wave; jj < w; jj += kThreads / 64) {
    const long long p = n - w + jj;
    const size_t slot = (size_t)u * eta + (size_t)(p % eta);
    copy_row(ring_k + slot * d, win_k + ((size_t)u * eta + jj) * d, d);
    copy_row(ring_v + slot * d, win_v + ((size_t)u * eta + jj) * d, d);
  }
  for (int i = wave; i < lam; i += kThreads / 64) {
    copy_row(cache_k + ((size_t)u * lam + i) * d, in_ck + ((size_t)u * lam + i) * d, d);
    copy_row(cache_v + ((size_t)u * lam + i) * d, in_cv + ((size_t)u * lam + i) * d, d);
    if ((threadIdx.x & 63) == 0)
      cache_pos[(size_t)u * lam + i] = i < gs ? in_pos[(size_t)u * lam + i] : -1;
  }
}

hipError_t launch_export(bool f32, int U, const void* ring_k, const void* ring_v,
                         const void* cache_k, const void* cache_v, const int32_t* cache_pos,
                         void* win_k, void* win_v, void* out_ck, void* out_cv, int32_t* out_pos,
                         long long n, int eta, int lam, int gs, int d, hipStream_t st) {
  if (U <= 0) return hipSuccess;
  if (f32)
    hipLaunchKernelGGL(export_kernel<float>, dim3(U), dim3(kThreads), 0, st,
                       (const float*)ring_k, (const float*)ring_v, (const float*)cache_k,
                       (const float*)cache_v, cache_pos, (float*)win_k, (float*)win_v,
                       (float*)out_ck, (float*)out_cv, out_pos, n, eta, lam, gs, d);
  else
    hipLaunchKernelGGL(export_kernel<uint16_t>, dim3(U), dim3(kThreads), 0, st,
                       (const uint16_t*)ring_k, (const uint16_t*)ring_v,
                       (const uint16_t*)cache_k, (const uint16_t*)cache_v, cache_pos,
                       (uint16_t*)win_k, (uint16_t*)win_v, (uint16_t*)out_ck,
                       (uint16_t*)out_cv, out_pos, n, eta, lam, gs, d);
  return hipGetLastError();
}

hipError_t launch_import(bool f32, int U, void* ring_k, void* ring_v, void* cache_k,
                         void* cache_v, int32_t* cache_pos, const void* win_k,
                         const void* win_v, const void* in_ck, const void* in_cv,
                         const int32_t* in_pos, long long n, int eta, int lam, int gs, int d,
                         hipStream_t st) {
  if (U <= 0) return hipSuccess;
  if (f32)
    hipLaunchKernelGGL(import_kernel<float>, dim3(U), dim3(kThreads), 0, st, (float*)ring_k,
                       (float*)ring_v, (float*)cache_k, (float*)cache_v, cache_pos,
                       (const float*)win_k, (const float*)win_v, (const float*)in_ck,
                       (const float*)in_cv, in_pos, n, eta, lam, gs, d);
  else
    hipLaunchKernelGGL(import_kernel<uint16_t>, dim3(U), dim3(kThreads), 0, st,
                       (uint16_t*)ring_k, (uint16_t*)ring_v, (uint16_t*)cache_k,
                       (uint16_t*)cache_v, cache_pos, (const uint16_t*)win_k,
                       (const uint16_t*)win_v, (const uint16_t*)in_ck,
                       (const uint16_t*)in_cv, in_pos, n, eta, lam, gs, d);
  return hipGetLastError();
}

// positions of the cache at every chunk start (debug export)
__global__ void snappos_kernel(VirtRows vr, const int32_t* snapG, int32_t* out, int nch, int C,
                               const int* err) {
  if (__builtin_amdgcn_readfirstlane(*reinterpret_cast<volatile const int*>(err)) != 0) return;
  const int u = blockIdx.y, j = blockIdx.x;
  const long long nj = vr.n0 + (long long)j * C;
  const int gs = (int)min((long long)vr.lam, max(0LL, nj - vr.eta));
  for (int i = threadIdx.x; i < vr.lam; i += blockDim.x) {
    const size_t o = ((size_t)u * nch + j) * vr.lam + i;
    out[o] = i < gs ? (int32_t)vr.pos_of(u, snapG[o]) : -1;
  }
}

hipError_t launch_snappos(const VirtRows& vr, const int32_t* snapG, int32_t* out, int nch,
                          int C, int U, const int* err, hipStream_t st) {
  if (U <= 0 || nch <= 0 || vr.lam <= 0) return hipSuccess;
  hipLaunchKernelGGL(snappos_kernel, dim3(nch, U), dim3(256), 0, st, vr, snapG, out, nch, C, err);
  return hipGetLastError();
}

// fill n 32-bit words with 0 (a kernel, so that the call is safe to capture)
__global__ void zero_u32_kernel(unsigned* p, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

hipError_t launch_zero_u32(unsigned* p, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

// Up to kMaxFill spans of 32-bit words, each set to its own value, in one
// launch (row y of the grid: span y; 16-byte stores where the span allows)
struct FillArgs {
  FillSpan s[kMaxFill];
};

__global__ __launch_bounds__(256) void fill_u32_kernel(FillArgs a) {
  const FillSpan sp = a.s[blockIdx.y];
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if ((reinterpret_cast<uintptr_t>(sp.p) & 15) == 0) {
    const size_t n4 = sp.n / 4;
    const u32x4 v = u32x4{sp.v, sp.v, sp.v, sp.v};
    for (size_t j = i; j < n4; j += stride) reinterpret_cast<u32x4*>(sp.p)[j] = v;
    for (size_t j = 4 * n4 + i; j < sp.n; j += stride) sp.p[j] = sp.v;
  } else {
    for (; i < sp.n; i += stride) sp.p[i] = sp.v;
  }
}

hipError_t launch_fill_u32(const FillSpan* spans, int n, hipStream_t st) {
  if (n < 0 || n > kMaxFill) return hipErrorInvalidValue;
  FillArgs a;
  int m = 0;
  size_t most = 0;
  for (int i = 0; i < n; ++i) {
    if (spans[i].n == 0) continue;
    a.s[m++] = spans[i];
    most = std::max(most, spans[i].n);
  }
  if (m == 0) return hipSuccess;
  // 16-byte stores: a quarter of the words per thread pass; at most 1024
  // blocks per span (grid-stride beyond)
  const size_t blocks = std::min<size_t>(1024, (most / 4 + 255) / 256 + 1);
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)blocks, (unsigned)m), dim3(256), 0, st, a);
  return hipGetLastError();
}

// dst[b][c][r] = src[b][r][c]: 32 x 32 tiles through LDS (export / import of
// H, whose device layout is H^T)
__global__ void transpose_f32_kernel(const float* src, float* dst, int rows, int cols) {
  __shared__ float tile[32][33];
  const int b = blockIdx.z;
  const int r0 = blockIdx.y * 32, c0 = blockIdx.x * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;   // 32 x 8 threads
  const float* s = src + (size_t)b * rows * cols;
  float* d = dst + (size_t)b * rows * cols;
  for (int y = ty; y < 32; y += 8)
    if (r0 + y < rows && c0 + tx < cols) tile[y][tx] = s[(size_t)(r0 + y) * cols + c0 + tx];
  __syncthreads();
  for (int y = ty; y < 32; y += 8)
    if (c0 + y < cols && r0 + tx < rows) d[(size_t)(c0 + y) * rows + r0 + tx] = tile[tx][y];
}

hipError_t launch_transpose_f32(const float* src, float* dst, int batch, int rows, int cols,
                                hipStream_t st) {
  if (batch <= 0 || rows <= 0 || cols <= 0) return hipSuccess;
  const dim3 grid((unsigned)((cols + 31) / 32), (unsigned)((rows + 31) / 32), (unsigned)batch);
  hipLaunchKernelGGL(transpose_f32_kernel, grid, dim3(256), 0, st, src, dst, rows, cols);
  return hipGetLastError();
}

}  // namespace lola
