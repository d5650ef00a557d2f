/*
 * lola.h -- C ABI of the LoLA chunkwise attention step (one layer) for AMD
 * Instinct MI355X (gfx950).
 *
 * The method (source: "LoLA: Low-Rank Linear Attention With Sparse Caching",
 * close-reading notes on arXiv:2505.23666v3, cited below as "LoLA notes"):
 * every (sequence, KV head) "unit" keeps three memories -- a sliding window
 * of the last eta key/value pairs, a sparse cache of at most lambda pairs, and
 * a linear-attention state H (D x d), s (D) (notes §2.1, §2.4).  Queries read
 * all three under one softmax normaliser (notes §2.5, Eq. (14)).  Pairs that
 * leave the window are scored, together with the cache, by the Self-Recall
 * Error ||H^T phi(k) / (phi(k)^T s) - v||^2 (notes §2.3, Eq. (10)); the lambda
 * highest stay cached and the rest are folded into H += phi(k) v^T,
 * s += phi(k) (notes §2.4, Eqs. (11)-(13)).  Prefill processes chunks of C
 * tokens that share the state at chunk start (notes §2.6, Eq. (15)).
 *
 * Feature map: phi(x) = [softmax(x W_h), softmax(-x W_h)], W_h a d x 64
 * matrix per KV head, so D = 128.
 *
 * Conventions
 *  - All tensor arguments are DEVICE pointers to contiguous row-major arrays,
 *    owned by the caller, read or written only by work enqueued on `stream`
 *    (a hipStream_t passed as void*; NULL = the null stream).  Calls return
 *    once the work is enqueued.
 *  - Element type of q, k, v, W and of the stored window/cache K/V is
 *    cfg->dtype (LOLA_DTYPE_F32 or LOLA_DTYPE_BF16, bf16 as raw 16-bit
 *    patterns).  H and s are float32.  Outputs are float32.
 *  - Every call returns a lola_status.  Argument errors leave the state
 *    unchanged.  A failure reported by HIP after work was enqueued marks the
 *    state poisoned: later calls return LOLA_ERR_STATE until
 *    lola_state_import() or lola_state_reset().  lola_last_error() gives a
 *    per-thread message.
 *  - Input ranges.  bf16 inputs: in the softmax branch of a prefill call V
 *    is multiplied in fp16 (by weights in [0, 2^8], fp32 accumulation), so
 *    |v| must stay below 65504 for y to stay finite, and values of magnitude
 *    below 2^-14 (fp16 subnormals) keep fewer significant bits there.  fp32
 *    inputs: every MFMA operand is split into fp16 hi + lo, so |q|, |k|, |v|
 *    and the phi, H and s entries must stay below 65504, and values below
 *    2^-14 lose relative precision (absolute error <= 2^-25 per split).
 *    H, s and the outputs are fp32.  The library does not scan the inputs
 *    for these ranges.
 */
#ifndef LOLA_H_
#define LOLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LOLA_OK = 0,
  LOLA_ERR_INVALID_ARG = 1,  /* null pointer, bad size, inconsistent config */
  LOLA_ERR_UNSUPPORTED = 2,  /* valid for the method, not for these kernels */
  LOLA_ERR_OUT_OF_MEMORY = 3,
  LOLA_ERR_HIP = 4,          /* a HIP runtime call failed */
  LOLA_ERR_STATE = 5,        /* poisoned state, or an import fails invariants */
  LOLA_ERR_WORKSPACE = 6     /* caller workspace smaller than required */
} lola_status;

typedef enum { LOLA_DTYPE_F32 = 0, LOLA_DTYPE_BF16 = 1 } lola_dtype;

typedef struct {
  int32_t batch;      /* B >= 1: sequences, all at the same position n */
  int32_t q_heads;    /* Hq; Hq % Hkv == 0; q-head j reads KV head j / (Hq/Hkv) */
  int32_t kv_heads;   /* Hkv >= 1 */
  int32_t head_dim;   /* d = d_k = d_v; supported: 64, 128 */
  int32_t feat_half;  /* m: phi has D = 2m features; supported: 64 */
  int32_t window;     /* eta >= 0: pairs kept in the sliding window */
  int32_t cache;      /* lambda >= 0: capacity of the sparse cache */
  int32_t dtype;      /* lola_dtype */
} lola_config;

typedef struct lola_state lola_state;

/* Create an empty state (n = 0, H = 0, s = 0, empty window and cache) on the
 * current HIP device.  W: device array [Hkv, d, m] in cfg->dtype, COPIED into
 * the state (the caller keeps ownership).  The library allocates and owns H
 * [B*Hkv, D, d], s [B*Hkv, D], the window ring [B*Hkv, eta, d] x2 and the
 * cache [B*Hkv, lambda, d] x2 plus positions (LoLA notes §2.7 state size).
 * Errors: INVALID_ARG, UNSUPPORTED (head_dim, feat_half, Hq/Hkv not in
 * {1,2,4}, sizes beyond the kernels' LDS budget), OUT_OF_MEMORY, HIP. */
int lola_state_init(const lola_config* cfg, const void* W, void* stream, lola_state** out);

/* Synchronise the state's last stream and release everything.  NULL: no-op. */
int lola_state_free(lola_state* st);

/* Tokens already processed (n); -1 while the sequences sit at different
 * positions (lola_state_positions). */
int64_t lola_state_tokens(const lola_state* st);

/* Bytes of workspace lola_prefill_chunk needs for (T, C).  0 for T == 0. */
int lola_prefill_workspace_bytes(const lola_state* st, int T, int C, size_t* bytes);

/* Process T new tokens with chunk length C (LoLA notes §2.6, Eq. (15)).
 * The serial chain of a call runs each unit on cooperating workgroups that
 * exchange partial SRE values through memory and must all be resident on
 * the GPU at once: the library sizes the grid to the device's compute units,
 * and other work sharing the GPU can delay them.  A wait that exceeds its
 * bound (see lola_debug_set) ends the chain with a device fault flag; every
 * later kernel of the call then returns without touching the state, and
 * lola_state_check() reports LOLA_ERR_STATE (the state must be reset or
 * imported).
 *   q   [B, Hq, T, d]    k, v  [B, Hkv, T, d]    (cfg->dtype)
 *   out [B, Hq, T, d]    float32 (out_dtype must be LOLA_DTYPE_F32)
 *   ws  device workspace of at least lola_prefill_workspace_bytes(T, C)
 *       bytes, or NULL to use a buffer the state owns (grown on demand;
 *       growing synchronises the stream).
 * Chunks start at the state's n; a last partial chunk is allowed.  Each
 * query reads the state as it was at the start of its chunk; the state is
 * then updated in place and n += T.  C == 1 processes token by token through
 * the decode kernel.  Other C: multiple of 32, at most 256.
 * Errors: INVALID_ARG, UNSUPPORTED (C), WORKSPACE, STATE, HIP. */
int lola_prefill_chunk(lola_state* st, const void* q, const void* k, const void* v, int T,
                       int C, void* out, int out_dtype, void* ws, size_t ws_bytes,
                       void* stream);

/* lola_prefill_chunk for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the workspace is a static device array of the library, 64 MiB
 * on every GPU it runs on, held until the process ends, so this call makes
 * no hipMalloc, hipFree or other allocating call (nor timing events of
 * lola_profile).  Arguments as lola_prefill_chunk, with no ws.
 * Every call on one GPU shares that GPU's array (it keeps the previous call's
 * contents; what must start at zero is cleared by a kernel of the call):
 * calls that overlap in time on one GPU -- other streams, other states, other
 * threads -- race and must be serialised by the caller.
 * Errors: as lola_prefill_chunk; WORKSPACE when lola_prefill_workspace_bytes
 * (T, C) exceeds 64 MiB (the state is then unchanged); HIP when the array's
 * address could not be found on the state's device. */
int lola_prefill_chunk_noalloc(lola_state* st, const void* q, const void* k, const void* v,
                               int T, int C, void* out, int out_dtype, void* stream);

/* lola_prefill_chunk plus a per-chunk record, for parity diagnostics:
 *   snap_pos  [B*Hkv, nch, lambda] int32: positions of the cache at the start
 *             of chunk j (in the chain's order, -1 padding), nch = ceil(T/C);
 *   cand_keys [B*Hkv, nch, lambda + C] uint64: for chunks whose candidates
 *             were scored, key (SRE float bits << 32) | (0xFFFFFFFF - position)
 *             of each candidate in candidate order; untouched otherwise.
 * Either may be NULL.  C must be > 1. */
int lola_prefill_debug(lola_state* st, const void* q, const void* k, const void* v, int T,
                       int C, void* out, int out_dtype, void* ws, size_t ws_bytes,
                       int32_t* snap_pos, uint64_t* cand_keys, void* stream);

/* lola_prefill_chunk plus SRE diagnostics (LoLA notes §4.4, Fig. 3, and
 * Eq. (26)), both outputs device memory and required:
 *   sre_map    [B*Hkv, nch, T] float32: for chunk j and the call's token p,
 *              the SRE (Eq. (10), squared) of (k_p, v_p) against the linear
 *              state H_j, s_j at the start of chunk j when an earlier chunk
 *              of this call folded p into it, else 0 (p in the window or the
 *              cache, or folded later);
 *   fold_chunk [B*Hkv, T] int32: the chunk whose update folded token p, -1
 *              if p was not folded during the call.
 * The SRE at first write of p is sre_map[u, fold_chunk[u, p] + 1, p], and the
 * relative SRE of Eq. (26) is sre_map[u, j, p] minus it, j > fold_chunk[u, p].
 * The map is fp32 from the chunk snapshots (hi/lo 16-bit planes of H_j).
 * C must be > 1.  Errors as lola_prefill_chunk, INVALID_ARG for NULL outputs. */
int lola_prefill_sre_map(lola_state* st, const void* q, const void* k, const void* v, int T,
                         int C, void* out, int out_dtype, void* ws, size_t ws_bytes,
                         float* sre_map, int32_t* fold_chunk, void* stream);

/* One token for every sequence: q [B, Hq, d], k, v [B, Hkv, d], out
 * [B, Hq, d] float32.  Exactly lola_prefill_chunk with T = 1, C = 1: the
 * query reads the state, then the pair leaving the window (if any) is scored
 * against the cache and the lowest-SRE candidate is folded (LoLA notes §2.4).
 * Storage: when window + cache <= 128 keys, a step may hold its fold term
 * (phi of the folded row and its value) in the state instead of rewriting H;
 * H is rewritten every fourth position, and any other call that reads or
 * replaces H (prefill, export, import, reset) first applies the held terms
 * in order.  The state every entry point observes is the one of a fold
 * applied at once, bit for bit.
 * Errors: INVALID_ARG, STATE, HIP; UNSUPPORTED while the sequences sit at
 * different positions (lola_state_import_sequence) and window + cache > 128
 * keys (that combination is not enabled). */
int lola_decode_step(lola_state* st, const void* q, const void* k, const void* v, void* out,
                     int out_dtype, void* stream);

/* Read branches (LoLA notes §4.8, Table 12: an ablation that hides memories
 * from the queries while the window, the cache, H and s are updated exactly
 * as before).  The read of Eq. (14) keeps the numerator and denominator terms
 * of the chosen memories only. */
enum {
  LOLA_READ_STATE = 1,    /* linear read H^T phi(q), phi(q)^T s */
  LOLA_READ_CACHE = 2,    /* keys of the sparse cache */
  LOLA_READ_WINDOW = 4,   /* local keys: window and the chunk's causal prefix */
  LOLA_READ_ALL = 7
};

/* Set the read-branch mask of the following prefill and decode calls
 * (default LOLA_READ_ALL).  The window bit must be set (every read then has
 * a positive normaliser).  Host-side only, takes effect at the next launch;
 * kept across lola_state_reset, not part of an exported state.
 * Errors: INVALID_ARG (NULL state, unknown bits, window bit clear). */
int lola_set_read_branches(lola_state* st, int branches);

/* Order of read and update for one token (LoLA notes §2.4-§2.6). */
enum {
  LOLA_READ_BEFORE_UPDATE = 0,  /* the chunk schedule: queries read the state as
                                   it is at chunk start (decode = C = 1) */
  LOLA_READ_AFTER_UPDATE = 1    /* the literal token recurrence: token t's query
                                   reads H_t, s_t, G_t and the window t-eta+1..t,
                                   after token t's pair has entered the window and
                                   the leaving pair was kept or folded (§2.5) */
};

/* Cache scoring rule (LoLA notes §4.5, Table 4: an ablation that replaces
 * the Self-Recall Error by other scores while everything else runs as
 * before).  The notes give the alternatives in words; with e = exp(q.k /
 * sqrt(d)) the exponential kernel and c = phi(q)^T phi(k) the feature
 * kernel of a (query, key) pair, a key's score is the sum of the rule's term
 * over every query head and every query that sees the key through the
 * sliding window (query t with chunk start n_t sees key i iff
 * max(0, n_t - eta) <= i <= t), frozen when the key leaves the window; the
 * cache keeps the lambda highest scores (ties: the older position). */
enum {
  LOLA_SCORE_SRE = 0,           /* ||H^T phi(k) / phi(k)^T s - v||^2 (the method) */
  LOLA_SCORE_KERNEL_SQ = 1,     /* sum (e - c)^2 */
  LOLA_SCORE_KERNEL_ABS = 2,    /* sum |e - c| */
  LOLA_SCORE_KERNEL_RATIO = 3,  /* sum c / e: keys the feature kernel overestimates */
  LOLA_SCORE_LOCAL_ATTN = 4     /* sum e: accumulated local attention */
};

/* Set the scoring rule of a state that holds no token yet (n = 0: fresh or
 * reset; kept across lola_state_reset).  The running scores of the window
 * and the frozen scores of the cache live in the state (allocated here).
 * With a rule other than LOLA_SCORE_SRE: prefill needs C > 1 and the read
 * order before update; decode, lola_state_import and
 * lola_state_import_sequence return UNSUPPORTED (the scores are not part of
 * the state view; lola_state_export writes the rest of the state);
 * lola_prefill_debug's cand_keys hold (score bits << 32) | (0xFFFFFFFF -
 * position).  The scores are fp32 sums; e must stay finite (q.k / sqrt(d)
 * below 88).
 * Errors: INVALID_ARG (NULL state, unknown rule), STATE (n > 0),
 * OUT_OF_MEMORY, HIP. */
int lola_set_scoring(lola_state* st, int rule);

/* Set the read order of the following decode calls and prefill calls with
 * C = 1 (default LOLA_READ_BEFORE_UPDATE).  With LOLA_READ_AFTER_UPDATE a
 * prefill with C > 1 returns UNSUPPORTED, and every token costs two decode
 * launches (update, then read).  With eta = 0 the window is empty after the
 * update; a call then needs a memory that is never empty (read branches with
 * the cache if lambda > 0, with the state if lambda = 0), else INVALID_ARG.
 * Host-side only; kept across lola_state_reset, not exported.
 * Errors: INVALID_ARG (NULL state, unknown order). */
int lola_set_read_order(lola_state* st, int order);

/* Start over: n = 0, H = 0, s = 0, empty window and cache (the memory and W
 * are kept).  Stream-ordered.  Clears a poisoned state. */
int lola_state_reset(lola_state* st, void* stream);

/* Wait for the state's work on `stream` and report faults the kernels
 * recorded on the device (an SRE exchange between the workgroups of a unit
 * that did not complete: LOLA_ERR_STATE, and the state is poisoned until
 * reset or import).  Errors: INVALID_ARG, HIP, STATE. */
int lola_state_check(lola_state* st, void* stream);

/* Kernel families whose launches can be timed. */
enum {
  LOLA_KERNEL_PHI = 0,       /* feature map of the candidate rows */
  LOLA_KERNEL_CHAIN = 1,     /* serial SRE / top-lambda / fold chain */
  LOLA_KERNEL_ATTN = 2,      /* chunk attention + linear read */
  LOLA_KERNEL_FINALIZE = 3,  /* cache / window write-back */
  LOLA_KERNEL_DECODE = 4,    /* decode step */
  LOLA_KERNEL_OVERLAP = 5,   /* chain and the read of finished chunks in one launch */
  LOLA_KERNEL_COUNT = 6
};

/* Per-kernel timing with HIP events recorded on the launch stream around
 * every launch while enabled.  Each call synchronises the recorded events,
 * writes the accumulated milliseconds and launch counts since the previous
 * call into ms[LOLA_KERNEL_COUNT] and launches[LOLA_KERNEL_COUNT] (either may
 * be NULL), resets them, and turns timing on (enable != 0) or off. */
int lola_profile(lola_state* st, int enable, double* ms, long long* launches);

/* Canonical state layout, all DEVICE pointers owned by the caller:
 *   H [B*Hkv, D, d] f32, s [B*Hkv, D] f32,
 *   win_k, win_v [B*Hkv, eta, d]: the last min(n, eta) pairs oldest first,
 *                                  rows beyond that zero,
 *   cache_pos [B*Hkv, lambda] int32 ascending, -1 padding; cache_k, cache_v
 *   [B*Hkv, lambda, d] in the same order (zero padding).
 * The cache holds min(lambda, max(0, n - eta)) pairs in every unit. */
typedef struct {
  int64_t n;
  float* H;
  float* s;
  void* win_k;
  void* win_v;
  int32_t* cache_pos;
  void* cache_k;
  void* cache_v;
} lola_state_view;

/* Write the state into `dst` (dst->n is set on return; stream-ordered).
 * UNSUPPORTED while the sequences sit at different positions (export them
 * one by one with lola_state_export_sequence). */
int lola_state_export(const lola_state* st, lola_state_view* dst, void* stream);

/* Replace the state with `src` (n = src->n).  Checks on the host what the
 * state's composition fixes (LoLA notes §2.7), and returns LOLA_ERR_STATE,
 * leaving the state unchanged, when one fails:
 *   - every unit's cache holds min(lambda, max(0, n - eta)) positions,
 *     ascending, non-negative and older than the window, then -1 padding;
 *   - s >= 0 and 1^T s = 2 x (max(0, n - eta) - cache count) to 1e-3
 *     relative (each half of phi sums to one, so a folded pair adds 2);
 *   - H is finite.
 * Clears a poisoned state and the device fault flags.  Synchronises stream. */
int lola_state_import(lola_state* st, const lola_state_view* src, void* stream);

/* Ragged batches.  Every memory of LoLA is per sequence and KV head (LoLA
 * notes §2.1, §2.4), so the sequences of one state may sit at different
 * positions: a serving loop prefills a new sequence in a state of its own
 * (batch 1, same configuration) and moves it into a free slot of the
 * batched decode state.
 *
 * lola_state_import_sequence copies `src`, a one-sequence state in the
 * lola_state_view layout with B = 1 (position src->n), into sequence slot
 * b; the checks of lola_state_import apply.  lola_state_export_sequence
 * writes slot b into a one-sequence view (dst->n = its position).  While the
 * positions differ, lola_decode_step advances every sequence by one token at
 * its own position (in either read order), lola_prefill_chunk and
 * lola_prefill_debug return UNSUPPORTED, lola_state_export returns
 * UNSUPPORTED and lola_state_tokens returns -1; lola_state_import and
 * lola_state_reset put every sequence at one position again.
 * lola_state_positions writes the B positions to host memory `out`.
 * Decode with positions that differ needs window + cache <= 128 keys
 * (UNSUPPORTED otherwise).
 * Import and export synchronise `stream`.
 * Errors: INVALID_ARG (NULL pointers, b out of range), STATE (bad cache
 * positions in src), HIP. */
int lola_state_import_sequence(lola_state* st, int b, const lola_state_view* src, void* stream);
int lola_state_export_sequence(const lola_state* st, int b, lola_state_view* dst, void* stream);
int lola_state_positions(const lola_state* st, int64_t* out);

/* Debug and schedule settings of a state (host-side, take effect at the next
 * launch; not exported, kept across lola_state_reset):
 *   LOLA_DEBUG_SPIN_LIMIT     polls of one exchange word of the chain before
 *                             its partner workgroup counts as lost, and of
 *                             the published-chunk counter by a concurrent
 *                             read (>= 1; 0 restores the default, 2^22);
 *   LOLA_DEBUG_CHAIN_FAIL_AT  every workgroup of the chain gives up at this
 *                             exchange step of a call, as if a partner were
 *                             lost (-1: never, the default);
 *   LOLA_DEBUG_OVERLAP        schedule of a chunked prefill call: 0 = the chain
 *                             over every chunk, then the read of every chunk;
 *                             1 = one launch in which the chain runs on half
 *                             of the compute units and the read of each chunk
 *                             starts as soon as the chain has published that
 *                             chunk's state (when the chain fits half of the
 *                             compute units, the call has >= 2 chunks and
 *                             the read's table of key row addresses fits its
 *                             LDS: window + cache + C up to about 4700 keys
 *                             at d = 128; otherwise as 0); -1 (default) = 1
 *                             for calls of >= 4 chunks, else 0.
 *                             Both schedules give bitwise the same results
 *                             (the chain's results do not depend on its
 *                             workgroup count).
 *   LOLA_DEBUG_CHAIN_SPLIT    how the chain's k > 1 workgroups of a unit share
 *                             the work: 0 = column slabs of H times groups of
 *                             candidates; 1 = groups of candidates only, every
 *                             workgroup holding all of H (when its LDS layout
 *                             fits; otherwise as 0); -1 (default) = 1 when a
 *                             workgroup scores >= 2 tiles of 32 candidates
 *                             per step, else 0.  Both give bitwise the same
 *                             results.
 *   LOLA_DEBUG_CHAIN_WORKGROUPS  the chain's workgroups per unit, k (1 .. 64;
 *                             0, the default: automatic).  Taken where the
 *                             whole chain grid fits the device (in the
 *                             one-launch schedule: U * k < the compute units)
 *                             and k suits the split (column split: k = 1, 2 or
 *                             a multiple of d / 32; candidate split: any k >
 *                             1); otherwise the automatic count, or
 *                             LOLA_ERR_INVALID_ARG from the prefill call when
 *                             the one-launch schedule has taken it.  Results
 *                             are bitwise the same for every k.
 * The first two exist to exercise the failure path: the chain sets its device
 * fault flag and ends, the later kernels of the call return untouched, and
 * lola_state_check() reports LOLA_ERR_STATE.
 * Errors: INVALID_ARG (NULL state, unknown key, value out of range). */
enum { LOLA_DEBUG_SPIN_LIMIT = 0, LOLA_DEBUG_CHAIN_FAIL_AT = 1, LOLA_DEBUG_OVERLAP = 2,
       LOLA_DEBUG_CHAIN_SPLIT = 3, LOLA_DEBUG_CHAIN_WORKGROUPS = 4 };
int lola_debug_set(lola_state* st, int key, long long value);

/* Text of a status code, and the last error detail of the calling thread. */
const char* lola_strerror(int status);
const char* lola_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LOLA_H_ */
