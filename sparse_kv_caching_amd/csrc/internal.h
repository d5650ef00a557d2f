// Internal interfaces between the C-ABI host runtime and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.h"
#include "lola.h"

namespace lola {

// Feature-map width: phi(x) = [softmax(x W), softmax(-x W)], W is d x kM.
constexpr int kM = 64;
constexpr int kD = 2 * kM;

// ---------------------------------------------------------------------------
// Virtual row space of one prefill call, per unit u = b * Hkv + h.
//
//   vi in [0, lam)                  slot vi of the cache at call start
//   vi in [lam, lam + eta + T)      position p = n0 - eta + (vi - lam):
//                                   p <  n0 -> window ring slot p % eta
//                                   p >= n0 -> input row p - n0
//
// Candidate order by virtual index is not position order for cache slots
// (decode leaves slots unordered), so every key also carries its position.
// ---------------------------------------------------------------------------
struct VirtRows {
  const void* cache_k;      // [U, lam, d]  (state dtype)
  const void* cache_v;
  const int32_t* cache_pos; // [U, lam], -1 = empty
  const void* ring_k;       // [U, eta, d]
  const void* ring_v;
  const void* in_k;         // [U, T, d]
  const void* in_v;
  long long n0;
  int lam, eta, T, d;

  __device__ __forceinline__ long long pos_of(int u, int vi) const {
    if (vi < lam) return cache_pos[(size_t)u * lam + vi];
    return n0 - eta + (vi - lam);
  }
  // byte offset of row vi of unit u in one of the three sources, elem = bytes
  __device__ __forceinline__ const char* row(const void* cache, const void* ring,
                                             const void* in, int u, int vi,
                                             int elem) const {
    size_t rb = (size_t)d * elem;
    if (vi < lam) return (const char*)cache + ((size_t)u * lam + vi) * rb;
    long long p = n0 - eta + (vi - lam);
    if (p < n0) return (const char*)ring + ((size_t)u * eta + (size_t)(p % eta)) * rb;
    return (const char*)in + ((size_t)u * T + (size_t)(p - n0)) * rb;
  }
  __device__ __forceinline__ const char* krow(int u, int vi, int elem) const {
    return row(cache_k, ring_k, in_k, u, vi, elem);
  }
  __device__ __forceinline__ const char* vrow(int u, int vi, int elem) const {
    return row(cache_v, ring_v, in_v, u, vi, elem);
  }
};

// ---------------------------------------------------------------------------
// K1: phi of every candidate row of the call -> hi/lo bf16 planes.
struct PhiArgs {
  VirtRows vr;
  const void* W;            // [Hkv, d, kM]
  uint16_t* phi_hi;         // [U, NV, kD]
  uint16_t* phi_lo;
  int NV;                   // lam + eta + T
  int Hkv;
  int gs0;                  // cache entries valid at call start
};

// K2: the serial SRE / top-lam / fold chain, one step per chunk.
struct ChainArgs {
  VirtRows vr;
  const uint16_t* phi_hi;
  const uint16_t* phi_lo;
  float* H;                 // [U, d, kD]  H^T (the device layout of H), in / out
  float* s;                 // [U, kD]
  uint16_t* snapHT;         // [U, nch, 2, d, kD]  H^T at chunk start, hi / lo
  float* snaps;             // [U, nch, kD]        s at chunk start
  int32_t* snapG;           // [U, nch, lam]       cache (virtual indices)
  int32_t* finalG;          // [U, lam]
  int NV, nch, C;
  uint64_t* dbg_keys;       // optional [U, nch, lam + C]: candidate keys per step
  int32_t* dbg_fold;        // optional [U, T]: the step that folded each call token (else untouched)
  // k workgroups per unit: 1, 2, or (d / 32) x CS with CS candidate groups;
  // every workgroup of the grid resident at once
  int k;
  // candidate split (k > 1): every workgroup holds all of H's columns and the
  // k workgroups are candidate groups; phi tiles are staged in LDS and shared
  // by the slabs' waves
  int xs;
  int xcd_group;            // U % 8 == 0: a unit's workgroups share a block residue mod 8
  uint64_t* xbuf;           // [U, 2, d / 32, lam + C]  tagged SRE parts per slab (k > 1), zeroed
  int* err;                 // device error flag: bit 0 = an exchange partner was lost
  int j0, j1;               // steps of this launch (a segment of the call's nch)
  int xstep0;               // exchange steps of the call before j0 (tags continue)
  int spin_limit;           // polls of one exchange word before its partner counts as lost
  int fail_at;              // debug: exchange step at which every workgroup gives up (-1: never)
  // accumulated scoring rules: the candidates are ranked by frozen scores
  // instead of SRE (no SRE products, no exchange); NULL for SRE
  const float* vscore;      // [U, eta + T] scores of the local rows (virtual index - lam)
  const float* cscore;      // [U, lam] scores of the cache slots at the call's start
  // concurrent read (NULL: none): the snapshots are written with coherent
  // stores, and each writer workgroup adds 1 to ready[u] once the snapshot
  // of a chunk is complete (writer workgroups per unit: d / 32 / SPW, or
  // min(k, d / 32) with the candidate split)
  int* ready;               // [U]
};

// K3: window + cache softmax attention merged with the linear read.
struct AttnArgs {
  VirtRows vr;
  const void* q;            // [B, Hq, T, d] == [U, g, T, d]
  const void* WT;           // [Hkv, kM, d]  W transposed
  const uint16_t* snapHT;
  const float* snaps;
  const int32_t* snapG;
  float* out;               // [U, g, T, d]
  int g, Hkv, nch, C, ptile, nblk;  // positions per WG, 32-position blocks per WG
  int ch0, nch_launch;      // chunks ch0 .. ch0 + nch_launch - 1 in this launch
  int branches;             // read mask, LOLA_READ_* bits (window always set)
  int* err;                 // device error flags: nonzero = the chain gave up, nothing to read
  // concurrent read (NULL: the snapshots are complete at launch): chunk j
  // of unit u may be read once ready[u] >= ready_need * (j + 1); the
  // snapshots are then read with coherent loads
  const int* ready;
  int ready_need;
  int spin_limit;           // polls of ready before the read gives up (sets err)
};

// Finalize: new cache rows / positions and window ring after a prefill call.
struct FinalizeArgs {
  VirtRows vr;
  const int32_t* finalG;    // [U, lam]
  void* new_cache_k;        // [U, lam, d]
  void* new_cache_v;
  int32_t* new_cache_pos;
  void* ring_k;             // written in place
  void* ring_v;
  int gs_final;
  const int* err;           // device error flags: nonzero = finalG was not written
};

// Decode step (C = 1) for every unit.
struct DecodeArgs {
  const void* q;            // [U, g, d]
  const void* k;            // [U, d]
  const void* v;
  const void* WT;           // [Hkv, kM, d]  W transposed, state dtype
  float* H;                 // [U, d, kD]  H^T
  float* s;                 // [U, kD]
  void* ring_k;
  void* ring_v;
  void* cache_k;            // current cache buffer, updated in place
  void* cache_v;
  int32_t* cache_pos;
  float* out;               // [U, g, d]
  long long n;
  int lam, eta, d, g, Hkv;
  int kc;                   // key rows per staged chunk (decode_plan)
  int branches;             // read mask, LOLA_READ_* bits (window always set)
  // 0: read, then update (the chunk schedule); 1: update only; 2: read only,
  // of a state that has just been updated (n counts the new token, which is
  // already in the window: no new pair, nothing scored or written)
  int phase;
  // ragged batches: position of each sequence [B] (NULL: every sequence at
  // n), and where to write the positions after this step (NULL: nowhere)
  const long long* npos;
  long long* npos_next;
  // element strides (one token): q / out [u][hd], k / v [u]
  long long q_su, q_sh, kv_su, o_su, o_sh;
  // deferred folds: H is the stored H plus, in order, the rank-one terms
  // phi v^T in pend [U][kPend][kD + d] (phi, then v; npend [U] of them);
  // NULL: every fold is written to H at once
  float* pend;
  int32_t* npend;
};

// Rank-one fold terms a unit may hold back between writes of its H: a
// decode step writes H only every kPend + 1 positions (staggered by unit) or
// when the list is full, else it appends its term (1 KB instead of 64 KB).
constexpr int kPend = 3;

// Accumulated cache scores of the local keys of a prefill call (the window
// at the call's start, then the call's keys): the alternative scoring rules.
struct ScoreArgs {
  VirtRows vr;
  const void* q;            // [U, g, T, d]
  const void* W;            // [Hkv, d, kM]
  const uint16_t* phi_hi;   // [U, NV, kD]
  const uint16_t* phi_lo;
  int NV, g, Hkv, C, rule;  // rule: LOLA_SCORE_*
  const float* ring_score;  // [U, eta] running scores of the window (slot p % eta)
  float* vscore;            // [U, eta + T] out: score of every local row
};

// The new cache's frozen scores and the window's running scores after a call.
struct ScoreWriteArgs {
  VirtRows vr;
  const int32_t* finalG;    // [U, lam]
  const float* cscore_in;   // [U, lam] cache scores at the call's start
  const float* vscore;      // [U, eta + T]
  float* cscore_out;        // [U, lam] scores of the new cache (its slot order)
  float* ring_score;        // [U, eta]
  int gs_final;
  const int* err;
};

// Diagnostics: SRE of the memories in the linear state at every chunk start.
struct SreMapArgs {
  VirtRows vr;
  const uint16_t* phi_hi;   // [U, NV, kD]
  const uint16_t* phi_lo;
  int NV;
  const uint16_t* snapHT;   // [U, nch, 2, d, kD]
  const float* snaps;       // [U, nch, kD]
  const int32_t* fold;      // [U, T] chunk that folded each call token, -1 none
  float* out;               // [U, nch, T]
  int nch;
  const int* err;           // device error flags: nonzero = the snapshots were not written
};

// Polls of one exchange word before the chain declares its partner lost.
constexpr int kSpinLimit = 1 << 22;
// Window + cache keys the one-chunk decode instance holds; more run through
// the chunked instance.
constexpr int kDecodeOneChunkKeys = 128;

// launchers (return hipError_t of the launch)
hipError_t launch_phi(const PhiArgs& a, int U, bool f32, hipStream_t st);
hipError_t launch_chain(const ChainArgs& a, int U, bool f32, hipStream_t st);
size_t chain_split_lds_bytes(int lam, int C, int d, bool f32);
size_t chain_lds_bytes(int lam, int C, int d, bool f32);
hipError_t launch_attn(const AttnArgs& a, int U, bool f32, hipStream_t st);
// The chain and the read of finished chunks in one launch: the chain's U * k
// workgroups come first in the grid (so they are all placed before any
// workgroup of the read), the read's workgroups (unit fastest, then position
// tile, then chunk) wait for their chunk's snapshot.  c.ready and a.ready
// point to the same zeroed counters.
hipError_t launch_overlap(const ChainArgs& c, const AttnArgs& a, int U, bool f32, hipStream_t st);
hipError_t launch_sre_map(const SreMapArgs& a, int U, bool f32, hipStream_t st);
hipError_t launch_score(const ScoreArgs& a, int U, bool f32, hipStream_t st);
size_t score_lds_bytes(int d);
hipError_t launch_score_writeback(const ScoreWriteArgs& a, int U, hipStream_t st);
size_t attn_lds_bytes(int d, int lam, int eta, int C, bool f32);
// the read's key table holds row addresses (the layout fits the LDS with
// them); the one-launch schedule needs it
bool attn_wide_table(int d, int lam, int eta, int C, bool f32);
int attn_positions_per_block(int C, int g);
hipError_t launch_finalize(const FinalizeArgs& a, int U, bool f32, hipStream_t st);
hipError_t launch_decode(const DecodeArgs& a, int U, bool f32, hipStream_t st);
// H += the held-back terms (in order, the same fma per element as the decode
// step's fold) and npend = 0, for every unit
hipError_t launch_flush_pending(float* H, const float* pend, int32_t* npend, int U, int d,
                                hipStream_t st);
hipError_t launch_export(bool f32, int U, const void* ring_k, const void* ring_v,
                         const void* cache_k, const void* cache_v, const int32_t* cache_pos,
                         void* win_k, void* win_v, void* out_ck, void* out_cv, int32_t* out_pos,
                         long long n, int eta, int lam, int gs, int d, hipStream_t st);
hipError_t launch_import(bool f32, int U, void* ring_k, void* ring_v, void* cache_k,
                         void* cache_v, int32_t* cache_pos, const void* win_k,
                         const void* win_v, const void* in_ck, const void* in_cv,
                         const int32_t* in_pos, long long n, int eta, int lam, int gs, int d,
                         hipStream_t st);
size_t decode_lds_bytes(int lam, int eta, int d, int g, bool f32);
void decode_plan(int lam, int eta, int d, int g, bool f32, int* kc);
hipError_t launch_transpose_w(const void* W, void* WT, int Hkv, int d, bool f32, hipStream_t st);
hipError_t launch_zero_u32(unsigned* p, size_t n, hipStream_t st);
// Several spans of 32-bit words, each set to its value, in one launch
// (empty spans are skipped; at most kMaxFill)
constexpr int kMaxFill = 8;
struct FillSpan {
  uint32_t* p;
  size_t n;
  uint32_t v;
};
hipError_t launch_fill_u32(const FillSpan* spans, int n, hipStream_t st);
// dst[b][c][r] = src[b][r][c] for b < batch, r < rows, c < cols (float32)
hipError_t launch_transpose_f32(const float* src, float* dst, int batch, int rows, int cols,
                                hipStream_t st);
hipError_t launch_snappos(const VirtRows& vr, const int32_t* snapG, int32_t* out, int nch,
                          int C, int U, const int* err, hipStream_t st);

}  // namespace lola
