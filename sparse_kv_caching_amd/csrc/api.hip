// Host runtime behind include/lola.h: validation, state and workspace memory,
// and the stream-ordered launch sequence of one prefill call:
//   K1 phi of every candidate row  ->  K2 serial SRE/top-lam/fold chain
//   (writes one snapshot per chunk)  ->  K3 attention of all chunks in
//   parallel  ->  finalize (new cache rows, window ring).
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <string>
#include <vector>

#include "internal.h"
#include "lola.h"

using namespace lola;


struct lola_state {
  lola_config cfg;
  int U, g, d, esz;
  bool f32;
  int64_t n;
  int device;
  hipStream_t last;
  bool poisoned;
  int branches;             // read mask (LOLA_READ_*)
  int order;                // LOLA_READ_BEFORE_UPDATE / LOLA_READ_AFTER_UPDATE
  int64_t* nseq;            // position of every sequence (host, B entries)
  bool ragged;              // some sequences sit at other positions than others
  long long* npos_dev;      // [2][B] sequence positions for ragged decode steps
  int npos_cur;             // the half decode reads next
  float* H;
  float* s;
  float* pend;              // [U][kPend][kD + d] decode folds not yet written to H
  int32_t* npend;           // [U] how many (H proper = H + their terms, in order)
  mutable bool pend_maybe;  // a decode step ran since the last flush (terms may be held)
  void* ring_k;
  void* ring_v;
  void* cache_k[2];
  void* cache_v[2];
  int32_t* cache_pos[2];
  int cur;
  void* W;
  void* WT;                 // W transposed [Hkv, kM, d] (decode operands)
  int* dev_err;             // device error flags (exchange timeouts)
  int rule;                 // cache scoring rule (LOLA_SCORE_*)
  float* ring_score;        // [U, eta] running scores of the window (rule != SRE)
  float* cache_score[2];    // [U, lam] frozen scores of the cache, with its two buffers
  int spin_limit;           // exchange polls before a partner counts as lost (lola_debug_set)
  int fail_at;              // debug: exchange step at which the chain gives up (-1: never)
  int overlap;              // prefill schedule: -1 auto, 0 sequential, 1 concurrent read
  int split;                // chain work split (k > 1): -1 auto, 0 slabs x candidates, 1 candidates
  int force_k;              // chain workgroups per unit (0: automatic)
  int ncu;                  // compute units of the device
  void* own_ws;
  size_t own_ws_bytes;
  // optional per-kernel timing with HIP events on the launch stream
  bool prof_on;
  bool no_alloc_call;       // inside lola_prefill_chunk_noalloc: no timing events
  struct Pending { int kind; hipEvent_t a, b; };
  std::vector<Pending>* prof_pending;
  double prof_ms[LOLA_KERNEL_COUNT];
  long long prof_n[LOLA_KERNEL_COUNT];
};

namespace {

thread_local std::string g_err;
constexpr size_t kMaxLds = 160 * 1024;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(lola_state* st, hipError_t e, const char* what) {
  if (st) st->poisoned = true;
  return fail(LOLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Brackets one kernel launch with events when timing is on.
struct ProfScope {
  lola_state* st;
  int kind;
  hipStream_t s;
  hipEvent_t a = nullptr, b = nullptr;
  ProfScope(lola_state* st_, int kind_, hipStream_t s_) : st(st_), kind(kind_), s(s_) {
    if (!st->prof_on || st->no_alloc_call) return;
    hipEventCreate(&a);
    hipEventCreate(&b);
    hipEventRecord(a, s);
  }
  ~ProfScope() {
    if (!a) return;
    hipEventRecord(b, s);
    st->prof_pending->push_back({kind, a, b});
  }
};

// ---------------------------------------------------------------------------
// Workspace of lola_prefill_chunk_noalloc: a file-scope device array, one copy
// per GPU the library runs on, held until the process ends.  Host code never
// passes `scratch` itself (its name is a host-side stand-in): each device's
// address comes from hipGetSymbolAddress, taken once per device with that
// device current (at lola_state_init) and kept in scratch_ptr_of.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;   // per device, nullptr until looked up
std::vector<int> g_scratch_err;     // per device, the lookup's hipError_t

// Look up (once) the address of `scratch` on the current device, `dev`.
void scratch_setup(int dev) {
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (dev < 0) return;
  if ((size_t)dev >= g_scratch_ptr.size()) {
    g_scratch_ptr.resize(dev + 1, nullptr);
    g_scratch_err.resize(dev + 1, -1);
  }
  if (g_scratch_ptr[dev]) return;
  void* p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  g_scratch_err[dev] = (int)e;
  if (e == hipSuccess) g_scratch_ptr[dev] = p;
}

void* scratch_ptr_of(int dev, int* err) {
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (dev < 0 || (size_t)dev >= g_scratch_ptr.size()) { *err = -1; return nullptr; }
  *err = g_scratch_err[dev];
  return g_scratch_ptr[dev];
}

struct WsLayout {
  size_t phi_hi, phi_lo, snapHT, snaps, snapG, finalG, xbuf, vscore, ready, total;
};

WsLayout ws_layout(const lola_state* st, int T, int C) {
  const size_t U = st->U, lam = st->cfg.cache, eta = st->cfg.window, d = st->d;
  const size_t NV = lam + eta + (size_t)T;
  const size_t nch = ((size_t)T + C - 1) / C;
  const size_t lam1 = lam > 0 ? lam : 1;
  WsLayout w;
  size_t off = 0;
  w.phi_hi = off; off = align256(off + U * NV * kD * 2);
  w.phi_lo = off; off = align256(off + U * NV * kD * 2);
  w.snapHT = off; off = align256(off + U * nch * 2 * d * kD * 2);
  w.snaps = off; off = align256(off + U * nch * kD * 4);
  w.snapG = off; off = align256(off + U * nch * lam1 * 4);
  w.finalG = off; off = align256(off + U * lam1 * 4);
  w.xbuf = off; off = align256(off + U * 2 * (d / 32) * (lam + (size_t)C) * 8);
  w.vscore = off;                 // scores of the local rows (accumulated rules only)
  if (st->rule != LOLA_SCORE_SRE) off = align256(off + U * (eta + (size_t)T) * 4);
  w.ready = off; off = align256(off + U * 4);   // published chunks per unit (concurrent read)
  w.total = off;
  return w;
}

// Workgroups per unit for the chain: the whole grid must be resident (one
// workgroup per compute unit, ncu of them available).  k = (d / 32) x CS:
// the columns' slabs times CS candidate groups, as many groups as fit, up to
// one per tile of 32 candidates.  Measured on the Llama-shaped layer (8
// units, 10 tiles per step), 8 / 16 / 32 workgroups per unit took 633 / 573
// / 552 us per call (chain then read); in the one-launch schedule 16 / 20 /
// 28 took 0.678 / 0.653 / 0.636 ms.
int chain_workgroups(int U, int ncu, int d, int lam, int C) {
  const int nslab = d / 32;
  const long long cap = ncu / std::max(U, 1);
  if (cap < 2) return 1;
  if (cap < nslab) return nslab >= 4 && cap >= 2 ? 2 : 1;
  const int tiles = (lam + C + 31) / 32;
  const int cs = (int)std::min<long long>({cap / nslab, std::max(1, tiles), 32LL});
  return nslab * cs;
}

// Chain workgroups per unit when the read of finished chunks runs beside
// the chain in one launch, or 0 when the call runs the two one after the
// other.  The concurrent schedule hides the read behind a chain that runs on
// fewer workgroups; the read is latency-bound and loses much less than half
// of its speed on half of the device.  Measured on MI355X (prefill call,
// ms, sequential -> concurrent): T = 32768 single sequence 5.11 -> 3.72; 8
// sequences of T = 8192 3.67 -> 3.13; Llama-shaped T = 4096 0.679 -> 0.671.
// The read keeps max(ncu / 8, R / 4) compute units, at most 5/8 of them,
// with R its 64-key tiles per chunk over all units (a compute unit reads about
// four such tiles in the time of a short chain step), but leaves the chain
// two workgroups per unit where half of the device allows (the candidate
// split needs two): the long workload's read takes 160 units (its chain 12
// workgroups per unit, six 32-candidate tiles each: 3.11 -> 2.99 ms per call
// against 128 units and 16 workgroups, 3.19 at 11, 3.11 at 13 and 14), the
// batched one's half of the device (2 per unit; 3.31 ms at 1), the
// Llama-shaped one's 32 units (its chain then runs on 28 workgroups per unit).
// The automatic choice takes the schedule whenever the chain fits and the
// call has >= 4 chunks.
int overlap_workgroups(const lola_state* st, int T, int C, int nch) {
  (void)T;
  if (st->overlap == 0 || nch < 2) return 0;
  const int U = st->U, lam = st->cfg.cache, eta = st->cfg.window;
  if (!attn_wide_table(st->d, lam, eta, C, st->f32)) return 0;
  const int g = st->cfg.q_heads / st->cfg.kv_heads;
  const long long nptile = (C + attn_positions_per_block(C, g) - 1) / attn_positions_per_block(C, g);
  const long long R = (long long)U * nptile * ((lam + eta + C + 63) / 64);
  int keep = (int)std::min<long long>(st->ncu * 5 / 8, std::max<long long>(st->ncu / 8, R / 4));
  if (st->ncu - keep < 2 * U && 2 * U <= st->ncu / 2) keep = st->ncu - 2 * U;
  const int chain_cus = st->ncu - keep;
  const int k = st->force_k > 0 ? st->force_k : chain_workgroups(U, chain_cus, st->d, lam, C);
  if ((long long)U * k > (st->force_k > 0 ? st->ncu - 1 : chain_cus)) return 0;
  if (st->overlap == 1) return k;
  return nch >= 4 ? k : 0;
}

int check_state(const lola_state* st) {
  if (!st) return fail(LOLA_ERR_INVALID_ARG, "state is NULL");
  if (st->poisoned)
    return fail(LOLA_ERR_STATE, "state is poisoned (an earlier HIP failure or a device fault "
                "flag); import a state or reset it");
  return LOLA_OK;
}

int supported_C(const lola_state* st, int C) {
  if (C == 1) return LOLA_OK;
  if (C % 32 != 0 || C > 256)
    return fail(LOLA_ERR_UNSUPPORTED, "chunk length C=%d: need C == 1 or a multiple of 32 <= 256", C);
  if (chain_lds_bytes(st->cfg.cache, C, st->d, st->f32) + 64 > kMaxLds)
    return fail(LOLA_ERR_UNSUPPORTED, "lambda + C too large for the chain kernel's LDS");
  if (attn_lds_bytes(st->d, st->cfg.cache, st->cfg.window, C, st->f32) + 64 > kMaxLds)
    return fail(LOLA_ERR_UNSUPPORTED, "lambda + eta + C too large for the attention kernel's LDS");
  return LOLA_OK;
}

// Every sequence at position n.
void set_uniform(lola_state* st, int64_t n) {
  st->n = n;
  for (int b = 0; b < st->cfg.batch; ++b) st->nseq[b] = n;
  st->ragged = false;
}

// A read after the update with eta = 0 sees no window: it needs a memory
// that is never empty then (the cache if lambda > 0, else the state).
int check_read_config(const lola_state* st) {
  if (st->order != LOLA_READ_AFTER_UPDATE || st->cfg.window > 0) return LOLA_OK;
  const bool ok = st->cfg.cache > 0 ? (st->branches & LOLA_READ_CACHE) != 0
                                    : (st->branches & LOLA_READ_STATE) != 0;
  if (!ok)
    return fail(LOLA_ERR_INVALID_ARG, "read after update with window 0: the read branches "
                "must include the %s", st->cfg.cache > 0 ? "cache" : "state");
  return LOLA_OK;
}

// H proper everywhere: the decode steps' held-back folds written into H
hipError_t flush_pending(const lola_state* st, hipStream_t s) {
  if (!st->pend_maybe) return hipSuccess;   // nothing can be held
  const hipError_t e = launch_flush_pending(st->H, st->pend, st->npend, st->U, st->d, s);
  if (e == hipSuccess) st->pend_maybe = false;
  return e;
}

// One token through the decode kernel at position a.n: read, then update;
// or (read after update) an update launch, then a read launch of the
// updated state at a.n + 1.
hipError_t decode_token(lola_state* st, DecodeArgs a, hipStream_t s) {
  hipError_t e;
  st->pend_maybe = true;
  if (st->ragged) {   // the kernel reads each sequence's position, writes it + 1
    a.npos = st->npos_dev + (size_t)st->npos_cur * st->cfg.batch;
    a.npos_next = st->npos_dev + (size_t)(st->npos_cur ^ 1) * st->cfg.batch;
  } else {
    a.npos = nullptr;
    a.npos_next = nullptr;
  }
  if (st->order != LOLA_READ_AFTER_UPDATE) {
    a.phase = 0;
    ProfScope ps(st, LOLA_KERNEL_DECODE, s);
    return launch_decode(a, st->U, st->f32, s);
  }
  a.phase = 1;
  { ProfScope ps(st, LOLA_KERNEL_DECODE, s); e = launch_decode(a, st->U, st->f32, s); }
  if (e != hipSuccess) return e;
  a.phase = 2;
  a.n += 1;
  if (a.npos) {
    a.npos = a.npos_next;
    a.npos_next = nullptr;
  }
  ProfScope ps(st, LOLA_KERNEL_DECODE, s);
  return launch_decode(a, st->U, st->f32, s);
}

// After a decode step: every sequence one token further.
void advance_positions(lola_state* st) {
  if (!st->ragged) {
    set_uniform(st, st->n + 1);
    return;
  }
  for (int b = 0; b < st->cfg.batch; ++b) st->nseq[b] += 1;
  st->npos_cur ^= 1;
}

// Checks of a state view about to be imported (units of it, position n), on
// the host (LoLA notes §2.7: the state is the window, the cache, H and s):
//  * the cache holds gs = min(lam, max(0, n - eta)) pairs: positions
//    ascending, non-negative and older than the window, then -1 padding;
//  * s >= 0 and 1^T s = 2 N_fold with N_fold = max(0, n - eta) - gs (each
//    half of phi sums to one, so every folded pair adds 2), to 1e-3 relative
//    (fp32 accumulation of the split features);
//  * H is finite.
int check_view(const lola_state* st, const lola_state_view* src, size_t units, hipStream_t s) {
  const size_t d = st->d;
  const int lam = st->cfg.cache, eta = st->cfg.window;
  const int64_t n = src->n;
  const int gs = (int)std::min<int64_t>(lam, std::max<int64_t>(0, n - eta));
  const int64_t w = std::min<int64_t>(eta, n);
  std::vector<int32_t> pos(units * (size_t)lam);
  std::vector<float> sv(units * kD), hv(units * kD * d);
  hipError_t e = hipSuccess;
  if (lam > 0) e = hipMemcpyAsync(pos.data(), src->cache_pos, pos.size() * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipMemcpyAsync(sv.data(), src->s, sv.size() * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipMemcpyAsync(hv.data(), src->H, hv.size() * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(LOLA_ERR_HIP, "import: %s", hipGetErrorString(e));
  const double nfold = (double)(std::max<int64_t>(0, n - eta) - gs);
  for (size_t u = 0; u < units; ++u) {
    for (int i = 0; i < lam; ++i) {
      const int32_t p = pos[u * lam + i];
      if (i < gs ? (p < 0 || p >= n - w || (i > 0 && p <= pos[u * lam + i - 1])) : p != -1)
        return fail(LOLA_ERR_STATE, "import: cache positions of unit %zu must be %d ascending "
                    "positions older than the window, then -1 padding", u, gs);
    }
    double sum = 0.0;
    for (int F = 0; F < kD; ++F) {
      const float x = sv[u * kD + F];
      if (!(x >= 0.f) || !std::isfinite(x))
        return fail(LOLA_ERR_STATE, "import: s of unit %zu has a negative or non-finite entry", u);
      sum += x;
    }
    if (std::fabs(sum - 2.0 * nfold) > 1e-3 * std::max(1.0, 2.0 * nfold))
      return fail(LOLA_ERR_STATE, "import: 1^T s = %.6g for unit %zu, expected 2 x %.0f folded pairs",
                  sum, u, nfold);
    for (size_t i = 0; i < (size_t)kD * d; ++i)
      if (!std::isfinite(hv[u * kD * d + i]))
        return fail(LOLA_ERR_STATE, "import: H of unit %zu has a non-finite entry", u);
  }
  return LOLA_OK;
}

}  // namespace

extern "C" {

const char* lola_strerror(int status) {
  switch (status) {
    case LOLA_OK: return "ok";
    case LOLA_ERR_INVALID_ARG: return "invalid argument";
    case LOLA_ERR_UNSUPPORTED: return "unsupported configuration";
    case LOLA_ERR_OUT_OF_MEMORY: return "out of device memory";
    case LOLA_ERR_HIP: return "HIP runtime error";
    case LOLA_ERR_STATE: return "invalid or poisoned state";
    case LOLA_ERR_WORKSPACE: return "workspace too small";
    default: return "unknown status";
  }
}

const char* lola_last_error(void) { return g_err.c_str(); }

int lola_state_init(const lola_config* cfg, const void* W, void* stream, lola_state** out) {
  if (!cfg || !W || !out) return fail(LOLA_ERR_INVALID_ARG, "cfg, W and out must be non-NULL");
  *out = nullptr;
  const lola_config& c = *cfg;
  if (c.batch < 1 || c.kv_heads < 1 || c.q_heads < 1 || c.q_heads % c.kv_heads ||
      c.window < 0 || c.cache < 0 || c.head_dim < 1 || c.feat_half < 1)
    return fail(LOLA_ERR_INVALID_ARG, "inconsistent configuration");
  if (c.dtype != LOLA_DTYPE_F32 && c.dtype != LOLA_DTYPE_BF16)
    return fail(LOLA_ERR_INVALID_ARG, "dtype must be LOLA_DTYPE_F32 or LOLA_DTYPE_BF16");
  const int g = c.q_heads / c.kv_heads;
  if (c.head_dim != 64 && c.head_dim != 128)
    return fail(LOLA_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", c.head_dim);
  if (c.feat_half != kM) return fail(LOLA_ERR_UNSUPPORTED, "feat_half must be %d", kM);
  if (g != 1 && g != 2 && g != 4)
    return fail(LOLA_ERR_UNSUPPORTED, "Hq/Hkv = %d (supported: 1, 2, 4)", g);
  if (c.window > (1 << 20) || c.cache > (1 << 20))
    return fail(LOLA_ERR_UNSUPPORTED, "window or cache too large");
  if (decode_lds_bytes(c.cache, c.window, c.head_dim, g, c.dtype == LOLA_DTYPE_F32) > kMaxLds)
    return fail(LOLA_ERR_UNSUPPORTED, "window + cache too large for the decode kernel's LDS");

  lola_state* st = new lola_state();
  memset(st, 0, sizeof *st);
  st->cfg = c;
  st->branches = LOLA_READ_ALL;
  st->order = LOLA_READ_BEFORE_UPDATE;
  st->spin_limit = kSpinLimit;
  st->fail_at = -1;
  st->overlap = -1;
  st->split = -1;
  st->force_k = 0;
  st->U = c.batch * c.kv_heads;
  st->g = g;
  st->d = c.head_dim;
  st->f32 = c.dtype == LOLA_DTYPE_F32;
  st->esz = st->f32 ? 4 : 2;
  st->last = (hipStream_t)stream;
  st->prof_pending = new std::vector<lola_state::Pending>();
  hipGetDevice(&st->device);
  scratch_setup(st->device);     // the no-allocation entry point's workspace on this device
  st->ncu = 0;
  if (hipDeviceGetAttribute(&st->ncu, hipDeviceAttributeMultiprocessorCount, st->device) != hipSuccess ||
      st->ncu < 1)
    st->ncu = 1;
  const size_t U = st->U, d = st->d, lam = c.cache, eta = c.window;
  auto alloc = [&](void** p, size_t bytes) -> bool {
    if (bytes == 0) bytes = 256;
    return hipMalloc(p, bytes) == hipSuccess;
  };
  bool ok = alloc((void**)&st->H, U * kD * d * 4) && alloc((void**)&st->s, U * kD * 4) &&
            alloc(&st->ring_k, U * eta * d * st->esz) && alloc(&st->ring_v, U * eta * d * st->esz) &&
            alloc(&st->W, (size_t)c.kv_heads * d * kM * st->esz) &&
            alloc(&st->WT, (size_t)c.kv_heads * d * kM * st->esz) &&
            alloc((void**)&st->dev_err, sizeof(int)) &&
            alloc((void**)&st->npos_dev, 2 * (size_t)c.batch * sizeof(long long)) &&
            alloc((void**)&st->pend, U * kPend * (kD + d) * 4) &&
            alloc((void**)&st->npend, U * 4);
  st->nseq = new int64_t[c.batch]();
  for (int b = 0; b < 2 && ok; ++b)
    ok = alloc(&st->cache_k[b], U * lam * d * st->esz) &&
         alloc(&st->cache_v[b], U * lam * d * st->esz) &&
         alloc((void**)&st->cache_pos[b], U * (lam ? lam : 1) * 4);
  if (!ok) {
    lola_state_free(st);
    return fail(LOLA_ERR_OUT_OF_MEMORY, "hipMalloc failed for the state");
  }
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipMemsetAsync(st->H, 0, U * kD * d * 4, s);
  if (e == hipSuccess) e = hipMemsetAsync(st->s, 0, U * kD * 4, s);
  for (int b = 0; b < 2 && e == hipSuccess; ++b)
    e = hipMemsetAsync(st->cache_pos[b], 0xFF, U * (lam ? lam : 1) * 4, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(st->W, W, (size_t)c.kv_heads * d * kM * st->esz, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess) e = launch_transpose_w(st->W, st->WT, c.kv_heads, (int)d, st->f32, s);
  if (e == hipSuccess) e = launch_zero_u32((unsigned*)st->dev_err, 1, s);
  if (e == hipSuccess) e = launch_zero_u32((unsigned*)st->npend, U, s);
  if (e != hipSuccess) {
    lola_state_free(st);
    return fail(LOLA_ERR_HIP, "state initialisation: %s", hipGetErrorString(e));
  }
  *out = st;
  return LOLA_OK;
}

int lola_state_free(lola_state* st) {
  if (!st) return LOLA_OK;
  hipStreamSynchronize(st->last);
  delete[] st->nseq;
  void* ps[] = {st->H, st->s, st->ring_k, st->ring_v, st->W, st->WT, st->dev_err, st->own_ws,
                st->npos_dev, st->pend, st->npend, st->ring_score, st->cache_score[0],
                st->cache_score[1],
                st->cache_k[0], st->cache_k[1], st->cache_v[0], st->cache_v[1],
                st->cache_pos[0], st->cache_pos[1]};
  for (void* p : ps)
    if (p) hipFree(p);
  if (st->prof_pending) {
    for (auto& pe : *st->prof_pending) { hipEventDestroy(pe.a); hipEventDestroy(pe.b); }
    delete st->prof_pending;
  }
  delete st;
  return LOLA_OK;
}

int64_t lola_state_tokens(const lola_state* st) { return st && !st->ragged ? st->n : -1; }

int lola_prefill_workspace_bytes(const lola_state* st, int T, int C, size_t* bytes) {
  if (!st || !bytes) return fail(LOLA_ERR_INVALID_ARG, "state and bytes must be non-NULL");
  if (T < 0 || C < 1) return fail(LOLA_ERR_INVALID_ARG, "T >= 0 and C >= 1 required");
  *bytes = (T == 0 || C == 1) ? 0 : ws_layout(st, T, C).total;
  return LOLA_OK;
}

int lola_decode_step(lola_state* st, const void* q, const void* k, const void* v, void* out,
                     int out_dtype, void* stream) {
  int rc = check_state(st);
  if (rc) return rc;
  if (!q || !k || !v || !out) return fail(LOLA_ERR_INVALID_ARG, "q, k, v, out must be non-NULL");
  if (out_dtype != LOLA_DTYPE_F32) return fail(LOLA_ERR_UNSUPPORTED, "out_dtype must be F32");
  for (int b = 0; b < st->cfg.batch; ++b)
    if (st->nseq[b] > (int64_t)0x7FFFFFF0) return fail(LOLA_ERR_UNSUPPORTED, "position overflow");
  if ((rc = check_read_config(st))) return rc;
  if (st->rule != LOLA_SCORE_SRE)
    return fail(LOLA_ERR_UNSUPPORTED, "decode with an accumulated scoring rule is not supported");
  if (st->ragged && st->cfg.cache + st->cfg.window > kDecodeOneChunkKeys)
    return fail(LOLA_ERR_UNSUPPORTED, "sequences at different positions with window + cache = %d "
                "> %d keys (the chunked decode kernel) are not supported",
                st->cfg.cache + st->cfg.window, kDecodeOneChunkKeys);
  hipStream_t s = (hipStream_t)stream;
  DecodeArgs a;
  a.q = q; a.k = k; a.v = v; a.WT = st->WT;
  a.H = st->H; a.s = st->s;
  a.pend = st->pend; a.npend = st->npend;
  a.ring_k = st->ring_k; a.ring_v = st->ring_v;
  a.cache_k = st->cache_k[st->cur]; a.cache_v = st->cache_v[st->cur];
  a.cache_pos = st->cache_pos[st->cur];
  a.out = (float*)out;
  a.n = st->n;
  a.lam = st->cfg.cache; a.eta = st->cfg.window; a.d = st->d; a.g = st->g;
  a.Hkv = st->cfg.kv_heads;
  decode_plan(a.lam, a.eta, st->d, st->g, st->f32, &a.kc);
  a.branches = st->branches;
  a.q_su = (long long)st->g * st->d; a.q_sh = st->d; a.kv_su = st->d;
  a.o_su = (long long)st->g * st->d; a.o_sh = st->d;
  const hipError_t e = decode_token(st, a, s);
  if (e != hipSuccess) return hip_fail(st, e, "decode launch");
  st->last = s;
  advance_positions(st);
  return LOLA_OK;
}

static int prefill_impl(lola_state* st, const void* q, const void* k, const void* v, int T,
                        int C, void* out, int out_dtype, void* ws, size_t ws_bytes,
                        int32_t* snap_pos, uint64_t* cand_keys, void* stream,
                        float* sre_map = nullptr, int32_t* fold_chunk = nullptr) {
  int rc = check_state(st);
  if (rc) return rc;
  if (T < 0 || C < 1) return fail(LOLA_ERR_INVALID_ARG, "T >= 0 and C >= 1 required");
  if (T == 0) return LOLA_OK;
  if (!q || !k || !v || !out) return fail(LOLA_ERR_INVALID_ARG, "q, k, v, out must be non-NULL");
  if (out_dtype != LOLA_DTYPE_F32) return fail(LOLA_ERR_UNSUPPORTED, "out_dtype must be F32");
  if ((rc = supported_C(st, C))) return rc;
  if (st->ragged)
    return fail(LOLA_ERR_UNSUPPORTED, "the sequences sit at different positions: prefill a new "
                "sequence in a state of its own and import it (lola_state_import_sequence)");
  if (st->order == LOLA_READ_AFTER_UPDATE && C != 1)
    return fail(LOLA_ERR_UNSUPPORTED, "read after update is token by token: C must be 1");
  if (st->rule != LOLA_SCORE_SRE && C == 1)
    return fail(LOLA_ERR_UNSUPPORTED, "an accumulated scoring rule needs C > 1");
  if ((rc = check_read_config(st))) return rc;
  if (st->n + T > (int64_t)0x7FFFFFF0) return fail(LOLA_ERR_UNSUPPORTED, "position overflow");
  const size_t NVs = (size_t)st->cfg.cache + st->cfg.window + T;
  if (NVs > (size_t)0x7FFFFFF0) return fail(LOLA_ERR_UNSUPPORTED, "T too large");
  hipStream_t s = (hipStream_t)stream;
  const int U = st->U, d = st->d, g = st->g;

  if (C == 1) {
    // token by token through the decode kernel, reading strided slices of
    // q [U, g, T, d], k / v [U, T, d] and writing out [U, g, T, d]
    DecodeArgs a;
    a.WT = st->WT; a.H = st->H; a.s = st->s;
    a.pend = st->pend; a.npend = st->npend;
    a.ring_k = st->ring_k; a.ring_v = st->ring_v;
    a.cache_k = st->cache_k[st->cur]; a.cache_v = st->cache_v[st->cur];
    a.cache_pos = st->cache_pos[st->cur];
    a.lam = st->cfg.cache; a.eta = st->cfg.window; a.d = d; a.g = g;
    a.Hkv = st->cfg.kv_heads;
    decode_plan(a.lam, a.eta, d, g, st->f32, &a.kc);
    a.branches = st->branches;
    a.q_su = (long long)g * T * d; a.q_sh = (long long)T * d; a.kv_su = (long long)T * d;
    a.o_su = a.q_su; a.o_sh = a.q_sh;
    for (int t = 0; t < T; ++t) {
      a.q = (const char*)q + (size_t)t * d * st->esz;
      a.k = (const char*)k + (size_t)t * d * st->esz;
      a.v = (const char*)v + (size_t)t * d * st->esz;
      a.out = (float*)out + (size_t)t * d;
      a.n = st->n;
      const hipError_t e = decode_token(st, a, s);
      if (e != hipSuccess) return hip_fail(st, e, "decode launch");
      set_uniform(st, st->n + 1);
    }
    st->last = s;
    return LOLA_OK;
  }

  // the chain reads H: the decode steps' held-back folds go in first
  if (hipError_t e = flush_pending(st, s); e != hipSuccess) return hip_fail(st, e, "flush");
  const WsLayout L = ws_layout(st, T, C);
  char* base = (char*)ws;
  if (!base) {
    if (st->own_ws_bytes < L.total) {
      hipStreamSynchronize(st->last);
      hipStreamSynchronize(s);
      if (st->own_ws) hipFree(st->own_ws);
      st->own_ws = nullptr;
      st->own_ws_bytes = 0;
      if (hipMalloc(&st->own_ws, L.total) != hipSuccess)
        return fail(LOLA_ERR_OUT_OF_MEMORY, "workspace of %zu bytes", L.total);
      st->own_ws_bytes = L.total;
    }
    base = (char*)st->own_ws;
  } else if (ws_bytes < L.total) {
    return fail(LOLA_ERR_WORKSPACE, "workspace %zu < required %zu bytes", ws_bytes, L.total);
  }

  const int lam = st->cfg.cache, eta = st->cfg.window;
  const int nch = (T + C - 1) / C;
  VirtRows vr;
  vr.cache_k = st->cache_k[st->cur];
  vr.cache_v = st->cache_v[st->cur];
  vr.cache_pos = st->cache_pos[st->cur];
  vr.ring_k = st->ring_k;
  vr.ring_v = st->ring_v;
  vr.in_k = k;
  vr.in_v = v;
  vr.n0 = st->n;
  vr.lam = lam;
  vr.eta = eta;
  vr.T = T;
  vr.d = d;
  const int gs0 = (int)std::min<int64_t>(lam, std::max<int64_t>(0, st->n - eta));
  const long long nend = st->n + T;
  const int gs_final = (int)std::min<long long>(lam, std::max<long long>(0, nend - eta));

  uint16_t* phi_hi = (uint16_t*)(base + L.phi_hi);
  uint16_t* phi_lo = (uint16_t*)(base + L.phi_lo);

  PhiArgs pa;
  pa.vr = vr; pa.W = st->W; pa.phi_hi = phi_hi; pa.phi_lo = phi_lo;
  pa.NV = (int)NVs; pa.Hkv = st->cfg.kv_heads; pa.gs0 = gs0;
  hipError_t e;
  { ProfScope ps(st, LOLA_KERNEL_PHI, s); e = launch_phi(pa, U, st->f32, s); }
  if (e != hipSuccess) return hip_fail(st, e, "phi launch");
  float* vscore = st->rule != LOLA_SCORE_SRE ? (float*)(base + L.vscore) : nullptr;
  if (vscore) {
    ScoreArgs sa;
    sa.vr = vr; sa.q = q; sa.W = st->W; sa.phi_hi = phi_hi; sa.phi_lo = phi_lo;
    sa.NV = (int)NVs; sa.g = g; sa.Hkv = st->cfg.kv_heads; sa.C = C; sa.rule = st->rule;
    sa.ring_score = st->ring_score; sa.vscore = vscore;
    e = launch_score(sa, U, st->f32, s);
    if (e != hipSuccess) return hip_fail(st, e, "score launch");
  }

  ChainArgs ca;
  ca.vr = vr; ca.phi_hi = phi_hi; ca.phi_lo = phi_lo;
  ca.H = st->H; ca.s = st->s;
  ca.snapHT = (uint16_t*)(base + L.snapHT);
  ca.snaps = (float*)(base + L.snaps);
  ca.snapG = (int32_t*)(base + L.snapG);
  ca.finalG = (int32_t*)(base + L.finalG);
  ca.NV = (int)NVs; ca.nch = nch; ca.C = C; ca.dbg_keys = cand_keys;
  ca.dbg_fold = fold_chunk;
  if (fold_chunk) {
    e = hipMemsetAsync(fold_chunk, 0xFF, (size_t)U * T * sizeof(int32_t), s);
    if (e != hipSuccess) return hip_fail(st, e, "debug reset");
  }
  const int k_ovl = overlap_workgroups(st, T, C, nch);
  ca.k = k_ovl                                                  ? k_ovl
         : st->force_k > 0 && (long long)U * st->force_k <= st->ncu ? st->force_k
                                                                 : chain_workgroups(U, st->ncu, d, lam, C);
  // k > 1: the candidate split where its LDS layout fits and (automatic
  // choice) a workgroup scores >= 2 tiles of 32 candidates per step: staging
  // the tiles once for all slabs then pays for holding all of H (folds over
  // all columns, a larger H^T rebuild).  Measured on MI355X, prefill call in
  // the one-launch schedule, column split -> candidate split: T = 32768
  // (4.5 tiles per workgroup) 3.30 -> 3.13 ms; 8 sequences of T = 8192 (10)
  // 2.95 -> 2.55 ms; Llama-shaped T = 4096 (0.6) 0.674 -> 0.705 ms
  auto pick_split = [&]() {
    ca.xs = ca.k > 1 && st->split != 0 && chain_split_lds_bytes(lam, C, d, st->f32) + 64 <= kMaxLds &&
                    (st->split == 1 || (lam + C + 31) / 32 >= 2 * ca.k)
                ? 1
                : 0;
  };
  pick_split();
  {
    // a forced workgroup count the split cannot use: the automatic one (the
    // column split needs k = 1, 2 or a multiple of d / 32; the candidate
    // split takes any k > 1)
    const int nslab = d / 32, k = ca.k;
    const bool ok = ca.xs ? k > 1 : (k == 1 || (k == 2 && nslab == 4) || k % nslab == 0);
    if (!ok && !k_ovl) {
      ca.k = chain_workgroups(U, st->ncu, d, lam, C);
      pick_split();
    } else if (!ok) {
      return fail(LOLA_ERR_INVALID_ARG, "chain workgroups per unit %d do not suit the work split", k);
    }
  }
  ca.xcd_group = (U % 8 == 0) ? 1 : 0;
  ca.xbuf = (uint64_t*)(base + L.xbuf);
  ca.err = st->dev_err;
  ca.j0 = 0;
  ca.j1 = nch;
  ca.xstep0 = 0;
  ca.spin_limit = st->spin_limit;
  ca.fail_at = st->fail_at;
  ca.vscore = vscore;
  ca.cscore = vscore ? st->cache_score[st->cur] : nullptr;
  ca.ready = k_ovl ? (int*)(base + L.ready) : nullptr;

  AttnArgs aa;
  aa.vr = vr; aa.q = q; aa.WT = st->WT;
  aa.snapHT = ca.snapHT; aa.snaps = ca.snaps; aa.snapG = ca.snapG;
  aa.out = (float*)out;
  aa.g = g; aa.Hkv = st->cfg.kv_heads; aa.nch = nch; aa.C = C;
  aa.ptile = attn_positions_per_block(C, g);
  aa.nblk = aa.ptile / 32;
  aa.ch0 = 0;
  aa.nch_launch = nch;
  aa.branches = st->branches;
  aa.err = st->dev_err;
  aa.ready = ca.ready;
  // writer workgroups per unit: one per slab group (d / 32 / SPW), or
  // min(k, d / 32) with the candidate split (the same counts)
  const int nslab = d / 32;
  aa.ready_need = ca.xs ? (ca.k >= nslab ? nslab : (nslab % ca.k == 0 ? ca.k : 1))
                        : (ca.k >= nslab ? nslab : (ca.k == 1 ? 1 : nslab / 2));
  aa.spin_limit = st->spin_limit;

  {
    // the exchange words (k > 1) and the published-snapshot counters (one
    // launch): zero before the chain starts
    FillSpan sp[2];
    int nsp = 0;
    if (ca.k > 1) sp[nsp++] = FillSpan{(uint32_t*)ca.xbuf, (size_t)U * 2 * (d / 32) * (lam + C) * 2, 0u};
    if (k_ovl) sp[nsp++] = FillSpan{(uint32_t*)ca.ready, (size_t)U, 0u};
    e = launch_fill_u32(sp, nsp, s);
    if (e != hipSuccess) return hip_fail(st, e, "exchange reset");
  }
  if (k_ovl) {
    { ProfScope ps(st, LOLA_KERNEL_OVERLAP, s); e = launch_overlap(ca, aa, U, st->f32, s); }
    if (e != hipSuccess) return hip_fail(st, e, "chain + read launch");
  } else {
    { ProfScope ps(st, LOLA_KERNEL_CHAIN, s); e = launch_chain(ca, U, st->f32, s); }
    if (e != hipSuccess) return hip_fail(st, e, "chain launch");
  }
  if (snap_pos) {
    e = launch_snappos(vr, ca.snapG, snap_pos, nch, C, U, st->dev_err, s);
    if (e != hipSuccess) return hip_fail(st, e, "debug launch");
  }
  if (sre_map) {
    SreMapArgs ma;
    ma.vr = vr; ma.phi_hi = phi_hi; ma.phi_lo = phi_lo; ma.NV = (int)NVs;
    ma.snapHT = ca.snapHT; ma.snaps = ca.snaps; ma.fold = fold_chunk; ma.out = sre_map;
    ma.nch = nch;
    ma.err = st->dev_err;
    e = launch_sre_map(ma, U, st->f32, s);
    if (e != hipSuccess) return hip_fail(st, e, "diagnostics launch");
  }

  if (!k_ovl) {
    { ProfScope ps(st, LOLA_KERNEL_ATTN, s); e = launch_attn(aa, U, st->f32, s); }
    if (e != hipSuccess) return hip_fail(st, e, "attention launch");
  }

  FinalizeArgs fa;
  fa.vr = vr;
  fa.finalG = ca.finalG;
  fa.new_cache_k = st->cache_k[1 - st->cur];
  fa.new_cache_v = st->cache_v[1 - st->cur];
  fa.new_cache_pos = st->cache_pos[1 - st->cur];
  fa.ring_k = st->ring_k;
  fa.ring_v = st->ring_v;
  fa.gs_final = gs_final;
  fa.err = st->dev_err;
  { ProfScope ps(st, LOLA_KERNEL_FINALIZE, s); e = launch_finalize(fa, U, st->f32, s); }
  if (e != hipSuccess) return hip_fail(st, e, "finalize launch");
  if (vscore) {
    ScoreWriteArgs wa;
    wa.vr = vr; wa.finalG = ca.finalG; wa.cscore_in = st->cache_score[st->cur];
    wa.vscore = vscore; wa.cscore_out = st->cache_score[1 - st->cur];
    wa.ring_score = st->ring_score; wa.gs_final = gs_final; wa.err = st->dev_err;
    e = launch_score_writeback(wa, U, s);
    if (e != hipSuccess) return hip_fail(st, e, "score write-back launch");
  }
  st->cur = 1 - st->cur;
  set_uniform(st, nend);
  st->last = s;
  return LOLA_OK;
}

int lola_prefill_chunk(lola_state* st, const void* q, const void* k, const void* v, int T,
                       int C, void* out, int out_dtype, void* ws, size_t ws_bytes,
                       void* stream) {
  return prefill_impl(st, q, k, v, T, C, out, out_dtype, ws, ws_bytes, nullptr, nullptr, stream);
}

int lola_prefill_chunk_noalloc(lola_state* st, const void* q, const void* k, const void* v,
                               int T, int C, void* out, int out_dtype, void* stream) {
  if (!st) return fail(LOLA_ERR_INVALID_ARG, "state is NULL");
  if (T < 0 || C < 1) return fail(LOLA_ERR_INVALID_ARG, "T >= 0 and C >= 1 required");
  const size_t need = (T == 0 || C == 1) ? 0 : ws_layout(st, T, C).total;
  if (need > kScratchBytes)
    return fail(LOLA_ERR_WORKSPACE, "this call needs %zu bytes of workspace; the static "
                "workspace of lola_prefill_chunk_noalloc holds %zu", need, kScratchBytes);
  int err = 0;
  void* ws = scratch_ptr_of(st->device, &err);
  if (!ws)
    return fail(LOLA_ERR_HIP, "no address of the static workspace on device %d (%s)", st->device,
                err >= 0 ? hipGetErrorString((hipError_t)err) : "not looked up");
  st->no_alloc_call = true;
  const int rc = prefill_impl(st, q, k, v, T, C, out, out_dtype, ws, kScratchBytes, nullptr,
                              nullptr, stream);
  st->no_alloc_call = false;
  return rc;
}

int lola_prefill_debug(lola_state* st, const void* q, const void* k, const void* v, int T,
                       int C, void* out, int out_dtype, void* ws, size_t ws_bytes,
                       int32_t* snap_pos, uint64_t* cand_keys, void* stream) {
  if (C == 1 && (snap_pos || cand_keys))
    return fail(LOLA_ERR_UNSUPPORTED, "debug export needs C > 1");
  return prefill_impl(st, q, k, v, T, C, out, out_dtype, ws, ws_bytes, snap_pos, cand_keys,
                      stream);
}

int lola_prefill_sre_map(lola_state* st, const void* q, const void* k, const void* v, int T,
                         int C, void* out, int out_dtype, void* ws, size_t ws_bytes,
                         float* sre_map, int32_t* fold_chunk, void* stream) {
  if (!sre_map || !fold_chunk)
    return fail(LOLA_ERR_INVALID_ARG, "sre_map and fold_chunk must be non-NULL");
  if (C == 1) return fail(LOLA_ERR_UNSUPPORTED, "the SRE diagnostics need C > 1");
  return prefill_impl(st, q, k, v, T, C, out, out_dtype, ws, ws_bytes, nullptr, nullptr, stream,
                      sre_map, fold_chunk);
}

int lola_set_read_branches(lola_state* st, int branches) {
  if (!st) return fail(LOLA_ERR_INVALID_ARG, "state must be non-NULL");
  if ((branches & ~LOLA_READ_ALL) || !(branches & LOLA_READ_WINDOW))
    return fail(LOLA_ERR_INVALID_ARG, "read branches %d: need a subset of %d with the window bit %d",
                branches, LOLA_READ_ALL, LOLA_READ_WINDOW);
  st->branches = branches;
  return LOLA_OK;
}

int lola_set_read_order(lola_state* st, int order) {
  if (!st) return fail(LOLA_ERR_INVALID_ARG, "state must be non-NULL");
  if (order != LOLA_READ_BEFORE_UPDATE && order != LOLA_READ_AFTER_UPDATE)
    return fail(LOLA_ERR_INVALID_ARG, "read order %d: need %d or %d", order,
                LOLA_READ_BEFORE_UPDATE, LOLA_READ_AFTER_UPDATE);
  st->order = order;
  return LOLA_OK;
}

int lola_set_scoring(lola_state* st, int rule) {
  if (!st) return fail(LOLA_ERR_INVALID_ARG, "state must be non-NULL");
  if (rule < LOLA_SCORE_SRE || rule > LOLA_SCORE_LOCAL_ATTN)
    return fail(LOLA_ERR_INVALID_ARG, "unknown scoring rule %d", rule);
  if (st->ragged || st->n != 0)
    return fail(LOLA_ERR_STATE, "the scoring rule is set on a state that holds no token "
                "(n = 0, after init or reset)");
  if (rule != LOLA_SCORE_SRE && !st->ring_score) {
    const size_t U = st->U, eta = st->cfg.window, lam = st->cfg.cache;
    auto alloc = [&](void** p, size_t bytes) -> bool {
      return hipMalloc(p, bytes ? bytes : 256) == hipSuccess;
    };
    if (!alloc((void**)&st->ring_score, U * eta * 4) ||
        !alloc((void**)&st->cache_score[0], U * lam * 4) ||
        !alloc((void**)&st->cache_score[1], U * lam * 4)) {
      for (float** p : {&st->ring_score, &st->cache_score[0], &st->cache_score[1]})
        if (*p) { hipFree(*p); *p = nullptr; }
      return fail(LOLA_ERR_OUT_OF_MEMORY, "hipMalloc failed for the scores");
    }
  }
  st->rule = rule;
  return LOLA_OK;
}

int lola_debug_set(lola_state* st, int key, long long value) {
  if (!st) return fail(LOLA_ERR_INVALID_ARG, "state must be non-NULL");
  switch (key) {
    case LOLA_DEBUG_SPIN_LIMIT:
      if (value < 0 || value > (1LL << 30))
        return fail(LOLA_ERR_INVALID_ARG, "spin limit %lld out of [0, 2^30]", value);
      st->spin_limit = value == 0 ? kSpinLimit : (int)value;   // 0: the default
      return LOLA_OK;
    case LOLA_DEBUG_CHAIN_FAIL_AT:
      if (value < -1 || value > (1LL << 30))
        return fail(LOLA_ERR_INVALID_ARG, "fail-at step %lld out of [-1, 2^30]", value);
      st->fail_at = (int)value;
      return LOLA_OK;
    case LOLA_DEBUG_OVERLAP:
      if (value < -1 || value > 1)
        return fail(LOLA_ERR_INVALID_ARG, "overlap %lld not in {-1, 0, 1}", value);
      st->overlap = (int)value;
      return LOLA_OK;
    case LOLA_DEBUG_CHAIN_WORKGROUPS:
      if (value < 0 || value > 64)
        return fail(LOLA_ERR_INVALID_ARG, "chain workgroups %lld not in [0, 64]", value);
      st->force_k = (int)value;
      return LOLA_OK;
    case LOLA_DEBUG_CHAIN_SPLIT:
      if (value < -1 || value > 1)
        return fail(LOLA_ERR_INVALID_ARG, "chain split %lld not in {-1, 0, 1}", value);
      st->split = (int)value;
      return LOLA_OK;
    default:
      return fail(LOLA_ERR_INVALID_ARG, "unknown debug key %d", key);
  }
}

int lola_state_reset(lola_state* st, void* stream) {
  if (!st) return fail(LOLA_ERR_INVALID_ARG, "state is NULL");
  hipStream_t s = (hipStream_t)stream;
  const size_t U = st->U, d = st->d, lam = st->cfg.cache;
  // H = 0, s = 0, both cache position buffers -1, the device flags and the
  // held-back fold counts 0: one launch
  const size_t cl = U * (lam ? lam : 1);
  const FillSpan sp[] = {{(uint32_t*)st->H, U * kD * d, 0u}, {(uint32_t*)st->s, U * kD, 0u},
                         {(uint32_t*)st->cache_pos[0], cl, ~0u}, {(uint32_t*)st->cache_pos[1], cl, ~0u},
                         {(uint32_t*)st->dev_err, 1, 0u}, {(uint32_t*)st->npend, U, 0u}};
  hipError_t e = launch_fill_u32(sp, 6, s);
  if (e != hipSuccess) return hip_fail(st, e, "reset");
  st->pend_maybe = false;
  set_uniform(st, 0);
  st->poisoned = false;
  st->last = s;
  return LOLA_OK;
}

int lola_state_check(lola_state* st, void* stream) {
  if (!st) return fail(LOLA_ERR_INVALID_ARG, "state is NULL");
  int flag = 0;
  hipError_t e = hipStreamSynchronize((hipStream_t)stream);
  if (e == hipSuccess) e = hipMemcpy(&flag, st->dev_err, sizeof(int), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(st, e, "check");
  if (flag) {
    st->poisoned = true;
    return fail(LOLA_ERR_STATE, "device fault flags 0x%x (bit 0: an SRE exchange between the "
                "workgroups of a unit did not complete; bit 1: a concurrent read gave up "
                "waiting for its chunk)", flag);
  }
  return st->poisoned ? fail(LOLA_ERR_STATE, "state is poisoned") : LOLA_OK;
}

int lola_profile(lola_state* st, int enable, double* ms, long long* launches) {
  if (!st) return fail(LOLA_ERR_INVALID_ARG, "state is NULL");
  for (auto& pe : *st->prof_pending) {
    hipError_t e = hipEventSynchronize(pe.b);
    float t = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&t, pe.a, pe.b);
    if (e != hipSuccess) return fail(LOLA_ERR_HIP, "profile: %s", hipGetErrorString(e));
    st->prof_ms[pe.kind] += t;
    st->prof_n[pe.kind] += 1;
    hipEventDestroy(pe.a);
    hipEventDestroy(pe.b);
  }
  st->prof_pending->clear();
  for (int k = 0; k < LOLA_KERNEL_COUNT; ++k) {
    if (ms) ms[k] = st->prof_ms[k];
    if (launches) launches[k] = st->prof_n[k];
    st->prof_ms[k] = 0.0;
    st->prof_n[k] = 0;
  }
  st->prof_on = enable != 0;
  return LOLA_OK;
}

int lola_state_export(const lola_state* st, lola_state_view* dst, void* stream) {
  if (!st || !dst || !dst->H || !dst->s || !dst->win_k || !dst->win_v || !dst->cache_pos ||
      !dst->cache_k || !dst->cache_v)
    return fail(LOLA_ERR_INVALID_ARG, "state and every view pointer must be non-NULL");
  if (st->ragged)
    return fail(LOLA_ERR_UNSUPPORTED, "the sequences sit at different positions: export them "
                "one by one (lola_state_export_sequence)");
  hipStream_t s = (hipStream_t)stream;
  const size_t U = st->U, d = st->d;
  const int lam = st->cfg.cache, eta = st->cfg.window;
  const int gs = (int)std::min<int64_t>(lam, std::max<int64_t>(0, st->n - eta));
  // the device keeps H^T [U, d, D] (plus held-back folds); the view holds H [U, D, d]
  hipError_t e = flush_pending(st, s);
  if (e == hipSuccess) e = launch_transpose_f32(st->H, dst->H, (int)U, (int)d, kD, s);
  if (e == hipSuccess) e = hipMemcpyAsync(dst->s, st->s, U * kD * 4, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess)
    e = launch_export(st->f32, st->U, st->ring_k, st->ring_v, st->cache_k[st->cur],
                      st->cache_v[st->cur], st->cache_pos[st->cur], dst->win_k, dst->win_v,
                      dst->cache_k, dst->cache_v, dst->cache_pos, st->n, eta, lam, gs, st->d, s);
  if (e != hipSuccess) return fail(LOLA_ERR_HIP, "export: %s", hipGetErrorString(e));
  dst->n = st->n;
  return LOLA_OK;
}

int lola_state_import(lola_state* st, const lola_state_view* src, void* stream) {
  if (!st || !src || !src->H || !src->s || !src->win_k || !src->win_v || !src->cache_pos ||
      !src->cache_k || !src->cache_v)
    return fail(LOLA_ERR_INVALID_ARG, "state and every view pointer must be non-NULL");
  if (src->n < 0 || src->n > (int64_t)0x7FFFFFF0) return fail(LOLA_ERR_STATE, "bad n");
  if (st->rule != LOLA_SCORE_SRE)
    return fail(LOLA_ERR_UNSUPPORTED, "the accumulated scores are not part of a state view");
  hipStream_t s = (hipStream_t)stream;
  const size_t U = st->U, d = st->d;
  const int lam = st->cfg.cache, eta = st->cfg.window;
  const int gs = (int)std::min<int64_t>(lam, std::max<int64_t>(0, src->n - eta));
  if (int rc = check_view(st, src, U, s)) return rc;
  // the state is replaced whole: the device fault flags and the held-back
  // decode folds of the old one go with it
  hipError_t e = launch_transpose_f32(src->H, st->H, (int)U, kD, (int)d, s);
  if (e == hipSuccess) e = launch_zero_u32((unsigned*)st->npend, U, s);
  if (e == hipSuccess) e = launch_zero_u32((unsigned*)st->dev_err, 1, s);
  if (e == hipSuccess) e = hipMemcpyAsync(st->s, src->s, U * kD * 4, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess)
    e = launch_import(st->f32, st->U, st->ring_k, st->ring_v, st->cache_k[st->cur],
                      st->cache_v[st->cur], st->cache_pos[st->cur], src->win_k, src->win_v,
                      src->cache_k, src->cache_v, src->cache_pos, src->n, eta, lam, gs, st->d, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(LOLA_ERR_HIP, "import: %s", hipGetErrorString(e));
  set_uniform(st, src->n);
  st->poisoned = false;
  st->last = s;
  return LOLA_OK;
}

int lola_state_import_sequence(lola_state* st, int b, const lola_state_view* src, void* stream) {
  int rc = check_state(st);
  if (rc) return rc;
  if (!src || !src->H || !src->s || !src->win_k || !src->win_v || !src->cache_pos ||
      !src->cache_k || !src->cache_v)
    return fail(LOLA_ERR_INVALID_ARG, "every view pointer must be non-NULL");
  if (b < 0 || b >= st->cfg.batch)
    return fail(LOLA_ERR_INVALID_ARG, "sequence slot %d out of range [0, %d)", b, st->cfg.batch);
  if (src->n < 0 || src->n > (int64_t)0x7FFFFFF0) return fail(LOLA_ERR_STATE, "bad n");
  if (st->rule != LOLA_SCORE_SRE)
    return fail(LOLA_ERR_UNSUPPORTED, "the accumulated scores are not part of a state view");
  hipStream_t s = (hipStream_t)stream;
  const int Hkv = st->cfg.kv_heads;
  const size_t d = st->d, u0 = (size_t)b * Hkv;
  const int lam = st->cfg.cache, eta = st->cfg.window;
  const int gs = (int)std::min<int64_t>(lam, std::max<int64_t>(0, src->n - eta));
  if (int rc = check_view(st, src, (size_t)Hkv, s)) return rc;
  const size_t es = st->esz;
  char* rk = (char*)st->ring_k + u0 * eta * d * es;
  char* rv = (char*)st->ring_v + u0 * eta * d * es;
  char* ck = (char*)st->cache_k[st->cur] + u0 * lam * d * es;
  char* cv = (char*)st->cache_v[st->cur] + u0 * lam * d * es;
  // every unit's held-back folds into H first (the slot's units are replaced)
  hipError_t e = flush_pending(st, s);
  if (e == hipSuccess) e = launch_transpose_f32(src->H, st->H + u0 * d * kD, Hkv, kD, (int)d, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(st->s + u0 * kD, src->s, (size_t)Hkv * kD * 4, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess)
    e = launch_import(st->f32, Hkv, rk, rv, ck, cv, st->cache_pos[st->cur] + u0 * lam, src->win_k,
                      src->win_v, src->cache_k, src->cache_v, src->cache_pos, src->n, eta, lam, gs,
                      st->d, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(st, e, "import sequence");
  st->nseq[b] = src->n;
  bool same = true;
  for (int i = 1; i < st->cfg.batch; ++i) same = same && st->nseq[i] == st->nseq[0];
  if (same) {
    set_uniform(st, st->nseq[0]);
  } else {
    // the positions decode reads next (a synchronous copy of the host array)
    st->ragged = true;
    st->n = -1;
    std::vector<long long> np(st->nseq, st->nseq + st->cfg.batch);
    e = hipMemcpy(st->npos_dev + (size_t)st->npos_cur * st->cfg.batch, np.data(),
                  np.size() * sizeof(long long), hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_fail(st, e, "import sequence positions");
  }
  st->last = s;
  return LOLA_OK;
}

int lola_state_export_sequence(const lola_state* st, int b, lola_state_view* dst, void* stream) {
  if (!st || !dst || !dst->H || !dst->s || !dst->win_k || !dst->win_v || !dst->cache_pos ||
      !dst->cache_k || !dst->cache_v)
    return fail(LOLA_ERR_INVALID_ARG, "state and every view pointer must be non-NULL");
  if (b < 0 || b >= st->cfg.batch)
    return fail(LOLA_ERR_INVALID_ARG, "sequence slot %d out of range [0, %d)", b, st->cfg.batch);
  hipStream_t s = (hipStream_t)stream;
  const int Hkv = st->cfg.kv_heads;
  const size_t d = st->d, u0 = (size_t)b * Hkv, es = st->esz;
  const int lam = st->cfg.cache, eta = st->cfg.window;
  const int64_t n = st->nseq[b];
  const int gs = (int)std::min<int64_t>(lam, std::max<int64_t>(0, n - eta));
  hipError_t e = flush_pending(st, s);
  if (e == hipSuccess) e = launch_transpose_f32(st->H + u0 * d * kD, dst->H, Hkv, (int)d, kD, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(dst->s, st->s + u0 * kD, (size_t)Hkv * kD * 4, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess)
    e = launch_export(st->f32, Hkv, (const char*)st->ring_k + u0 * eta * d * es,
                      (const char*)st->ring_v + u0 * eta * d * es,
                      (const char*)st->cache_k[st->cur] + u0 * lam * d * es,
                      (const char*)st->cache_v[st->cur] + u0 * lam * d * es,
                      st->cache_pos[st->cur] + u0 * lam, dst->win_k, dst->win_v, dst->cache_k,
                      dst->cache_v, dst->cache_pos, n, eta, lam, gs, st->d, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(LOLA_ERR_HIP, "export sequence: %s", hipGetErrorString(e));
  dst->n = n;
  return LOLA_OK;
}

int lola_state_positions(const lola_state* st, int64_t* out) {
  if (!st || !out) return fail(LOLA_ERR_INVALID_ARG, "state and out must be non-NULL");
  for (int b = 0; b < st->cfg.batch; ++b) out[b] = st->nseq[b];
  return LOLA_OK;
}

}  // extern "C"
