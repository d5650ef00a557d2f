"""Chunk-vectorised float64 oracle of LoLA's attention step for one layer.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What is computed, and where the pages say so
--------------------------------------------
A *unit* is one (sequence b, KV head h).  Every memory of LoLA is per unit:

* sliding window W: the most recent ``eta`` key/value pairs
  [LoLA notes §2.1 symbol table; §2.4 step 1];
* sparse global cache G: at most ``lam`` key/value pairs
  [LoLA notes §2.1; §2.4, Eq. (11)];
* linear state H (D x d_v) and s (D), which receive only the pairs that are
  *allocated* to them [LoLA notes §2.2, Eqs. (3)-(5) and the paragraph after].

Per chunk of c tokens starting at position n (chunk schedule: LoLA notes §2.6,
Eq. (15)):

1. **Read** (LoLA notes §2.5, Eq. (14)).  For query t the explicit keys are
   G plus every local position i with max(0, n - eta) <= i <= t, and

       y_t = (H^T phi(q_t) + sum_i a_ti v_i) / (phi(q_t)^T s + sum_i a_ti),
       a_ti = exp(q_t . k_i / sqrt(d_k)),

   one normaliser over all three memories, with H, s, G as at chunk start
   (chunk queries share the existing state, LoLA notes §2.6).
2. **Candidates** (LoLA notes §2.4 step 2; §2.6).  The tokens that leave the
   window, L = [max(0, n - eta), max(0, n + c - eta)), joined with the current
   cache: E = G u L.
3. **Keep all if few** (LoLA notes §2.4, after Eq. (13)): if |E| <= lam, G <- E
   and nothing is scored or folded.
4. **Score before write** (LoLA notes §2.3, Eq. (10); §2.4, Eqs. (11)-(13) and
   the before/after reading given there): each candidate's Self-Recall Error
   against the state as it is *before* this update,

       SRE(k, v | H, s) = || H^T phi(k) / (phi(k)^T s) - v ||^2 ,

   squared as in the LoLA summary's SRE section (the notes print the norm
   unsquared; the ranking is identical).  Keep the ``lam`` highest as the new
   G; fold the rest into H += sum phi(k) v^T, s += sum phi(k).
5. **Advance**: the window becomes the last ``eta`` positions; n += c.

Readings where the pages leave a step open:
eta counts past tokens kept between chunks and a query also sees its own
chunk's causal prefix (diagonal included); z = phi(k)^T s = 0 gives prediction
0 (the notes flag the H = 0, s = 0 division as unhandled); ties in the top-lam
order go to the older token (lower position); the read uses the state at chunk
start and decode is this same step with c = 1; with GQA, q-head j reads KV head
floor(j / g); every batch sequence is at the same n.

The feature map is phi(x) = [softmax(x W_h), softmax(-x W_h)] with one W_h
(d x m) per KV head, D = 2m (learned phi, R^{d_k} -> R^D with D = 2 d_k in the
notes §2.1 and §3.1; this fixed softmax form is the workload's).
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

F64 = np.float64

# Read branches of Eq. (14) (LoLA notes §4.8, Table 12: the ablation hides
# some memories from the queries while every update runs as before).  The
# window branch (local keys, including the chunk's causal prefix) is always
# read, as in every row of that table; it also keeps the normaliser positive.
BRANCH_STATE = 1      # H^T phi(q) and phi(q)^T s
BRANCH_SPARSE = 2     # the cache G
BRANCH_WINDOW = 4     # local positions max(0, n - eta) .. t
BRANCH_ALL = 7


# Cache scoring rules (LoLA notes §4.5, Table 4; the formulas of the notes'
# Appendix F are not on the pages, so these are readings of the table's
# words).  SRE is the method's rule; the other four score a key by what the
# local queries saw of it while it was in the sliding window, accumulated
# over those queries (and the query heads of its KV head) and frozen when it
# leaves the window.  With e = exp(q.k / sqrt(d)) the exponential kernel and
# c = phi(q)^T phi(k) the feature kernel of one (query, key) pair:
SCORE_SRE = "sre"                    # ||H^T phi(k) / phi(k)^T s - v||^2 (Eq. (10))
SCORE_KERNEL_SQ = "kernel_sq"        # sum (e - c)^2: squared kernel error
SCORE_KERNEL_ABS = "kernel_abs"      # sum |e - c|: absolute kernel error
SCORE_KERNEL_RATIO = "kernel_ratio"  # sum c / e: keys the feature kernel overestimates
SCORE_LOCAL_ATTN = "local_attn"      # sum e: accumulated local attention
SCORES = (SCORE_SRE, SCORE_KERNEL_SQ, SCORE_KERNEL_ABS, SCORE_KERNEL_RATIO, SCORE_LOCAL_ATTN)


def score_terms(rule: str, e: np.ndarray, c: np.ndarray) -> np.ndarray:
    """The per-(query, key) term that an accumulated rule adds to a key's
    score, from the exponential kernel e and the feature kernel c."""
    if rule == SCORE_KERNEL_SQ:
        return (e - c) ** 2
    if rule == SCORE_KERNEL_ABS:
        return np.abs(e - c)
    if rule == SCORE_KERNEL_RATIO:
        return c / e
    if rule == SCORE_LOCAL_ATTN:
        return e
    raise ValueError("not an accumulated scoring rule: %r" % rule)


def check_branches(branches: int) -> int:
    """A read-branch mask: bits BRANCH_*, with the window bit set."""
    b = int(branches)
    if b & ~BRANCH_ALL or not b & BRANCH_WINDOW:
        raise ValueError("read branches must be a subset of 7 that includes the window (4)")
    return b


# --------------------------------------------------------------------------- phi
def _softmax_last(u: np.ndarray) -> np.ndarray:
    """Softmax over the last axis.  Subtracting the row max first changes
    nothing mathematically; it only keeps exp finite."""
    e = np.exp(u - u.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def phi(x: np.ndarray, W: np.ndarray) -> np.ndarray:
    """phi(x) = [softmax(x W), softmax(-x W)] for rows x (..., d), W (d, m).

    Returns (..., 2m) in float64.  Each half sums to 1, so 1^T phi(x) = 2.
    """
    u = np.asarray(x, F64) @ np.asarray(W, F64)
    return np.concatenate([_softmax_last(u), _softmax_last(-u)], axis=-1)


def _phi_units(x: np.ndarray, Wu: np.ndarray) -> np.ndarray:
    """phi for per-unit rows: x (U, ..., d), Wu (U, d, m) -> (U, ..., 2m)."""
    U = x.shape[0]
    flat = x.reshape(U, -1, x.shape[-1])
    u = np.matmul(flat, Wu)                       # (U, rows, m)
    out = np.concatenate([_softmax_last(u), _softmax_last(-u)], axis=-1)
    return out.reshape(x.shape[:-1] + (out.shape[-1],))


# --------------------------------------------------------------------------- SRE
def sre(phk: np.ndarray, v: np.ndarray, H: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Self-Recall Error of candidates against a linear state.

    phk (U, E, D) features of the candidate keys, v (U, E, d) their values,
    H (U, D, d), s (U, D).  Returns (U, E):

        z = phi(k)^T s;  p = H^T phi(k) / z  (p = 0 when z = 0);
        SRE = sum_c (p_c - v_c)^2.

    [LoLA notes §2.3, Eq. (10); squared per the LoLA summary; the z = 0 rule
    is the reading of the notes' §2.6 remark that H = 0, s = 0 cannot be
    divided.]
    """
    phk = np.asarray(phk, F64)
    z = np.einsum("uef,uf->ue", phk, s)
    num = np.matmul(phk, H)                       # (U, E, d) = phi^T H per row
    safe = np.where(z > 0, z, 1.0)
    p = np.where((z > 0)[..., None], num / safe[..., None], 0.0)
    return ((p - np.asarray(v, F64)) ** 2).sum(axis=-1)


# ------------------------------------------------------------------- selection
def select_keep(scores: np.ndarray, pos: np.ndarray, lam: int) -> np.ndarray:
    """Top_lam membership per unit: keep the ``lam`` candidates that come first
    in the order (score descending, position ascending).

    [LoLA notes §2.4, Eq. (11) and the note after Eq. (13): Top_lam returns the
    highest-scoring set, capacity exactly lam; ties go to the older token.]
    scores, pos: (U, E).  Returns a boolean keep mask (U, E).
    """
    U, E = scores.shape
    keep = np.zeros((U, E), dtype=bool)
    if lam <= 0:
        return keep
    for u in range(U):
        order = np.lexsort((pos[u], -scores[u]))   # primary: -score, then pos
        keep[u, order[:lam]] = True
    return keep


def _given_keep(E_pos: np.ndarray, keep_pos, lam: int) -> np.ndarray:
    """Keep mask of an imposed kept set (see _update_chunk): exactly lam
    candidates of every unit."""
    keep = np.zeros(E_pos.shape, dtype=bool)
    for u in range(E_pos.shape[0]):
        want = np.asarray(sorted(keep_pos[u]), dtype=np.int64)
        keep[u] = np.isin(E_pos[u], want)
        if keep[u].sum() != lam or want.size != lam:
            raise ValueError("unit %d: the kept set must be %d of the candidates" % (u, lam))
    return keep


def boundary_gap(scores: np.ndarray, lam: int) -> np.ndarray:
    """Relative gap (SRE_(lam) - SRE_(lam+1)) / SRE_(lam) at the capacity
    boundary, per unit (scores sorted descending; inf if SRE_(lam) == 0)."""
    srt = -np.sort(-scores, axis=1)
    a, b = srt[:, lam - 1], srt[:, lam]
    with np.errstate(divide="ignore", invalid="ignore"):
        return np.where(a > 0, (a - b) / a, np.inf)


# ----------------------------------------------------------------------- state
@dataclass
class LolaState:
    """Per-layer state for U units (float64).

    n       tokens already processed (common to every unit)
    H, s    linear state (U, D, d) and (U, D)
    win_k/v window pairs (U, w, d), positions [n - w, n), w = min(n, eta)
    g_pos   cache positions (U, |G|), ascending; g_k/g_v (U, |G|, d)
    n_fold  tokens folded into H, s so far (common to every unit)
    """

    eta: int
    lam: int
    n: int
    H: np.ndarray
    s: np.ndarray
    win_k: np.ndarray
    win_v: np.ndarray
    g_pos: np.ndarray
    g_k: np.ndarray
    g_v: np.ndarray
    n_fold: int = 0
    rule: str = SCORE_SRE
    win_score: Optional[np.ndarray] = None   # (U, w) accumulated scores (other rules)
    g_score: Optional[np.ndarray] = None     # (U, |G|) frozen scores of the cache

    def copy(self) -> "LolaState":
        cp = lambda a: None if a is None else a.copy()
        return LolaState(self.eta, self.lam, self.n, self.H.copy(), self.s.copy(),
                         self.win_k.copy(), self.win_v.copy(), self.g_pos.copy(),
                         self.g_k.copy(), self.g_v.copy(), self.n_fold, self.rule,
                         cp(self.win_score), cp(self.g_score))


def new_state(U: int, d: int, D: int, eta: int, lam: int, rule: str = SCORE_SRE) -> LolaState:
    """Empty state: n = 0, H = 0, s = 0, no window, no cache; ``rule`` the
    cache scoring rule (SCORES)."""
    if rule not in SCORES:
        raise ValueError("unknown scoring rule %r" % rule)
    z = np.zeros
    acc = rule != SCORE_SRE
    return LolaState(eta, lam, 0, z((U, D, d)), z((U, D)), z((U, 0, d)), z((U, 0, d)),
                     z((U, 0), dtype=np.int64), z((U, 0, d)), z((U, 0, d)), 0, rule,
                     z((U, 0)) if acc else None, z((U, 0)) if acc else None)


def state_elements(d_k: int, d_v: int, D: int, eta: int, lam: int, t: int) -> int:
    """Persistent attention-state element count per head after t tokens:
    min{t (d_k + d_v), (eta + lam)(d_k + d_v) + D d_v + D}
    [LoLA notes §2.7, memory formula of Appendix B]."""
    return min(t * (d_k + d_v), (eta + lam) * (d_k + d_v) + D * d_v + D)


@dataclass
class ChunkLog:
    """What one chunk's update did (per unit arrays; ``sre`` is None when
    |E| <= lam and nothing was scored)."""

    n: int
    c: int
    cand_pos: np.ndarray
    sre: Optional[np.ndarray] = None
    keep: Optional[np.ndarray] = None
    gap: Optional[np.ndarray] = None


# ------------------------------------------------------------------------ read
def _read_chunk(st: LolaState, qc: np.ndarray, kc: np.ndarray, vc: np.ndarray,
                Wu: np.ndarray, branches: int = BRANCH_ALL) -> np.ndarray:
    """Eq. (14) for every query of the chunk, with the state at chunk start.

    qc (U, g, c, d); kc, vc (U, c, d).  Returns y (U, g, c, d).  ``branches``
    drops the terms of hidden memories from both numerator and denominator
    (LoLA notes §4.8, Table 12)."""
    U, g, c, d = qc.shape
    keys = np.concatenate([st.g_k, st.win_k, kc], axis=1)     # (U, nk, d)
    vals = np.concatenate([st.g_v, st.win_v, vc], axis=1)
    n_old = st.g_k.shape[1] + st.win_k.shape[1]
    logits = np.matmul(qc, keys[:, None].transpose(0, 1, 3, 2)) / np.sqrt(d)
    a = np.exp(logits)                                        # unshifted, Eq. (14)
    if not np.all(np.isfinite(a)):
        raise FloatingPointError("exp(q.k/sqrt(d)) overflowed in float64")
    causal = np.tril(np.ones((c, c), dtype=bool))             # t sees j <= t
    a[..., n_old:] *= causal
    if not branches & BRANCH_SPARSE:
        a[..., :st.g_k.shape[1]] = 0.0
    num = np.matmul(a, vals[:, None])
    den = a.sum(axis=-1)
    if branches & BRANCH_STATE:
        phq = _phi_units(qc, Wu)                              # (U, g, c, D)
        num = num + np.matmul(phq, st.H[:, None])
        den = den + np.einsum("ugtf,uf->ugt", phq, st.s)
    return num / den[..., None]


def _read_after(st: LolaState, qc: np.ndarray, Wu: np.ndarray,
                branches: int = BRANCH_ALL) -> np.ndarray:
    """Eq. (14) as the notes write it for one token (LoLA notes §2.5): the
    query of token t reads H_t, s_t, G_t and the window W_t *after* token t's
    update, so every key in W_t and G_t is visible (no causal part).
    qc (U, g, 1, d).  Returns y (U, g, 1, d)."""
    U, g, c, d = qc.shape
    nk = 0
    parts_k, parts_v = [], []
    if branches & BRANCH_SPARSE:
        parts_k.append(st.g_k)
        parts_v.append(st.g_v)
    parts_k.append(st.win_k)
    parts_v.append(st.win_v)
    keys = np.concatenate(parts_k, axis=1)
    vals = np.concatenate(parts_v, axis=1)
    logits = np.matmul(qc, keys[:, None].transpose(0, 1, 3, 2)) / np.sqrt(d)
    a = np.exp(logits)
    if not np.all(np.isfinite(a)):
        raise FloatingPointError("exp(q.k/sqrt(d)) overflowed in float64")
    num = np.matmul(a, vals[:, None])
    den = a.sum(axis=-1)
    if branches & BRANCH_STATE:
        phq = _phi_units(qc, Wu)
        num = num + np.matmul(phq, st.H[:, None])
        den = den + np.einsum("ugtf,uf->ugt", phq, st.s)
    return num / den[..., None]


# ---------------------------------------------------------------------- update
def _local_scores(st: LolaState, qc: np.ndarray, kc: np.ndarray, Wu: np.ndarray) -> np.ndarray:
    """The chunk's contribution to the accumulated scores of the local keys
    (window, then the chunk's own keys): for every query t of the chunk and
    every key i it sees through the window (positions max(0, n - eta) .. t),
    the rule's term of (q_t, k_i), summed over t and the g query heads.
    qc (U, g, c, d), kc (U, c, d).  Returns (U, w + c)."""
    U, g, c, d = qc.shape
    keys = np.concatenate([st.win_k, kc], axis=1)             # (U, nloc, d)
    w = st.win_k.shape[1]
    e = np.exp(np.matmul(qc, keys[:, None].transpose(0, 1, 3, 2)) / np.sqrt(d))
    if not np.all(np.isfinite(e)):
        raise FloatingPointError("exp(q.k/sqrt(d)) overflowed in float64")
    cfeat = np.matmul(_phi_units(qc, Wu), _phi_units(keys, Wu)[:, None].transpose(0, 1, 3, 2))
    terms = score_terms(st.rule, e, cfeat)                    # (U, g, c, nloc)
    vis = np.ones((c, w + c), dtype=bool)
    vis[:, w:] = np.tril(np.ones((c, c), dtype=bool))         # query t sees chunk keys <= t
    return (terms * vis).sum(axis=(1, 2))


def _update_chunk(st: LolaState, kc: np.ndarray, vc: np.ndarray, Wu: np.ndarray,
                  keep_pos=None, qc: Optional[np.ndarray] = None) -> ChunkLog:
    """Steps 2-5 of the chunk schedule (candidates, keep-all, SRE, fold,
    advance).  Mutates ``st``.

    ``keep_pos`` (per unit, lam positions of the candidates) replaces the
    top-lam selection of a scored update by a given kept set: another correct
    choice at a near-tie of the boundary (the compare rule's band), so that a
    run can continue along the cache another implementation chose."""
    U, c, d = kc.shape
    n, eta, lam = st.n, st.eta, st.lam
    w = st.win_k.shape[1]
    local_k = np.concatenate([st.win_k, kc], axis=1)          # positions n-w .. n+c-1
    local_v = np.concatenate([st.win_v, vc], axis=1)
    n_new = n + c
    w_new = min(n_new, eta)
    n_leave = w + c - w_new                                   # = |L|
    p0 = n - w
    leave_pos = np.broadcast_to(np.arange(p0, p0 + n_leave, dtype=np.int64), (U, n_leave))
    E_pos = np.concatenate([st.g_pos, leave_pos], axis=1)
    E_k = np.concatenate([st.g_k, local_k[:, :n_leave]], axis=1)
    E_v = np.concatenate([st.g_v, local_v[:, :n_leave]], axis=1)
    acc = st.rule != SCORE_SRE
    if acc:
        if qc is None:
            raise ValueError("the %r rule accumulates the queries' view of the keys" % st.rule)
        local_s = np.concatenate([st.win_score, np.zeros((U, c))], axis=1) + \
            _local_scores(st, qc, kc, Wu)
        E_score = np.concatenate([st.g_score, local_s[:, :n_leave]], axis=1)
        st.win_score = local_s[:, n_leave:].copy()
    st.win_k = local_k[:, n_leave:].copy()
    st.win_v = local_v[:, n_leave:].copy()
    log = ChunkLog(n=n, c=c, cand_pos=E_pos.copy())
    nE = E_pos.shape[1]
    if nE <= lam:
        st.g_pos, st.g_k, st.g_v = E_pos.copy(), E_k, E_v
        if acc:
            st.g_score = E_score.copy()
    else:
        phE = _phi_units(E_k, Wu)
        # SRE against the before-state, or the frozen accumulated scores
        scores = sre(phE, E_v, st.H, st.s) if not acc else E_score
        keep = select_keep(scores, E_pos, lam) if keep_pos is None else \
            _given_keep(E_pos, keep_pos, lam)
        fold = (~keep).astype(F64)
        st.H = st.H + np.matmul((phE * fold[..., None]).transpose(0, 2, 1), E_v)
        st.s = st.s + (phE * fold[..., None]).sum(axis=1)
        st.g_pos = E_pos[keep].reshape(U, lam)
        st.g_k = E_k[keep].reshape(U, lam, d)
        st.g_v = E_v[keep].reshape(U, lam, d)
        if acc:
            st.g_score = E_score[keep].reshape(U, lam)
        st.n_fold += nE - lam
        log.sre, log.keep = scores, keep
        log.gap = boundary_gap(scores, lam) if lam > 0 else None
    st.n = n_new
    return log


# ------------------------------------------------------------------ public API
def _as_units(q, k, v, W, Hkv):
    q = np.asarray(q, F64)
    k = np.asarray(k, F64)
    v = np.asarray(v, F64)
    B, Hq, T, d = q.shape
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    g = Hq // Hkv
    U = B * Hkv
    qu = q.reshape(B, Hkv, g, T, d).reshape(U, g, T, d)
    ku = k.reshape(U, T, d)
    vu = v.reshape(U, T, d)
    Wu = np.tile(np.asarray(W, F64), (B, 1, 1))               # unit b*Hkv+h -> W[h]
    return qu, ku, vu, Wu, (B, Hq, T, d)


def prefill(st: LolaState, q, k, v, W, C: int, *, outputs: bool = True,
            logs: Optional[List[ChunkLog]] = None,
            branches: int = BRANCH_ALL, order: str = "before",
            keep=None) -> Optional[np.ndarray]:
    """Process T new tokens with chunk length C (the last chunk may be short).

    q (B, Hq, T, d); k, v (B, Hkv, T, d); W (Hkv, d, m); ``st`` holds U = B*Hkv
    units and is updated in place.  Returns y (B, Hq, T, d) in float64, or None
    if ``outputs`` is False (the state trajectory does not depend on q).
    ``branches`` masks the read only (see check_branches); the state update is
    the same for every mask.  ``order``: "before" (the chunk schedule, LoLA
    notes §2.6: the chunk's queries read the state at chunk start) or "after"
    (the literal token recurrence, §2.4-§2.5: with C = 1, token t's query
    reads the state after token t's update).  ``keep``: for a call of one
    chunk (T <= C), the kept set to impose if its update is scored (per
    unit, lam positions; see _update_chunk).
    """
    if C < 1:
        raise ValueError("C must be >= 1")
    branches = check_branches(branches)
    if order not in ("before", "after"):
        raise ValueError("order must be 'before' or 'after'")
    if order == "after" and C != 1:
        raise ValueError("the read-after-update order is defined token by token (C = 1)")
    if order == "after" and st.rule != SCORE_SRE:
        raise ValueError("the accumulated scoring rules are defined for the chunk schedule")
    if order == "after" and outputs and st.eta == 0 and not (
            (st.lam > 0 and branches & BRANCH_SPARSE) or (st.lam == 0 and branches & BRANCH_STATE)):
        raise ValueError("eta = 0 reads no window after the update: keep a memory that is "
                         "never empty (the cache if lam > 0, else the state)")
    Hkv = np.asarray(W).shape[0]
    qu, ku, vu, Wu, shape = _as_units(q, k, v, W, Hkv)
    U, g, T, d = qu.shape
    if st.H.shape[0] != U:
        raise ValueError("state unit count does not match the inputs")
    if keep is not None and T > C:
        raise ValueError("an imposed kept set applies to a call of one chunk")
    y = np.zeros(qu.shape) if outputs else None
    t0 = 0
    while t0 < T:
        c = min(C, T - t0)
        sl = slice(t0, t0 + c)
        if outputs and order == "before":
            y[:, :, sl] = _read_chunk(st, qu[:, :, sl], ku[:, sl], vu[:, sl], Wu, branches)
        lg = _update_chunk(st, ku[:, sl], vu[:, sl], Wu, keep, qu[:, :, sl])
        if outputs and order == "after":
            y[:, :, sl] = _read_after(st, qu[:, :, sl], Wu, branches)
        if logs is not None:
            logs.append(lg)
        t0 += c
    if not outputs:
        return None
    B, Hq, T, d = shape
    return y.reshape(B, Hkv, g, T, d).reshape(B, Hq, T, d)


def decode_step(st: LolaState, q, k, v, W, *, logs=None,
                branches: int = BRANCH_ALL, order: str = "before") -> np.ndarray:
    """One token for every sequence: q (B, Hq, d), k, v (B, Hkv, d).
    Defined as prefill with T = 1, C = 1 (read, then update; or update, then
    read with order="after")."""
    y = prefill(st, np.asarray(q)[:, :, None], np.asarray(k)[:, :, None],
                np.asarray(v)[:, :, None], W, 1, logs=logs, branches=branches, order=order)
    return y[:, :, 0]


# ------------------------------------------------------------- SRE diagnostics
def sre_map(st: LolaState, k, v, W, C: int):
    """Self-Recall Error of the memories inside the linear state, chunk by
    chunk (the diagnostic of LoLA notes §4.4, Fig. 3, and Eq. (26)).

    Runs the chunk schedule on k, v (B, Hkv, T, d) from ``st`` (updated in
    place).  Returns

    * ``m`` (U, nch, T): m[u, j, p] = SRE(k_p, v_p | H_j, s_j) with H_j, s_j
      the state at the start of chunk j, for the call's tokens p folded into
      the state by an earlier chunk of the call; 0 for tokens not (yet) in the
      state (in the window or the cache: the notes show them as zero columns);
    * ``fold`` (U, T) int: the chunk whose update folded token p, -1 if it
      was not folded during the call.

    The SRE at first write of p is m[u, fold + 1, p] (the first state that
    holds it) and the relative SRE of Eq. (26) is m[u, j, p] minus it, for
    j > fold."""
    if st.rule != SCORE_SRE:
        raise ValueError("the SRE map describes the SRE rule")
    Hkv = np.asarray(W).shape[0]
    k = np.asarray(k, F64)
    v = np.asarray(v, F64)
    B, _, T, d = k.shape
    U = B * Hkv
    ku = k.reshape(U, T, d)
    vu = v.reshape(U, T, d)
    Wu = np.tile(np.asarray(W, F64), (B, 1, 1))
    n0 = st.n
    nch = (T + C - 1) // C
    m = np.zeros((U, nch, T))
    fold = np.full((U, T), -1, dtype=np.int64)
    phk = _phi_units(ku, Wu)                                  # (U, T, D)
    for j in range(nch):
        t0 = j * C
        for u in range(U):
            folded = np.nonzero((fold[u] >= 0) & (fold[u] < j))[0]
            if folded.size:
                m[u, j, folded] = sre(phk[u:u + 1, folded], vu[u:u + 1, folded],
                                      st.H[u:u + 1], st.s[u:u + 1])[0]
        lg = _update_chunk(st, ku[:, t0:t0 + C], vu[:, t0:t0 + C], Wu)
        if lg.keep is not None:
            for u in range(U):
                out = lg.cand_pos[u][~lg.keep[u]] - n0          # call-relative positions
                out = out[out >= 0]
                fold[u, out] = j
    return m, fold


# ------------------------------------------------------------ export / import
def export_state(st: LolaState) -> dict:
    """Canonical layout (per unit): n; H (U, D, d); s (U, D); window k/v oldest
    to newest (U, w, d); cache positions ascending (U, |G|) with its k/v."""
    d = dict(n=st.n, n_fold=st.n_fold, H=st.H.copy(), s=st.s.copy(),
             win_k=st.win_k.copy(), win_v=st.win_v.copy(),
             g_pos=st.g_pos.copy(), g_k=st.g_k.copy(), g_v=st.g_v.copy(), rule=st.rule)
    if st.rule != SCORE_SRE:
        d["win_score"], d["g_score"] = st.win_score.copy(), st.g_score.copy()
    return d


def import_state(d: dict, eta: int, lam: int) -> LolaState:
    """Inverse of :func:`export_state`; checks the bookkeeping invariants
    |W| = min(n, eta), |G| = min(lam, max(0, n - eta)), positions ascending
    and older than the window."""
    n = int(d["n"])
    U = d["H"].shape[0]
    w = d["win_k"].shape[1]
    gs = d["g_pos"].shape[1]
    if w != min(n, eta):
        raise ValueError("window length does not match n")
    if gs != min(lam, max(0, n - eta)):
        raise ValueError("cache size does not match n")
    gp = np.asarray(d["g_pos"], np.int64)
    if gs and (np.any(np.diff(gp, axis=1) <= 0) or np.any(gp >= n - w) or np.any(gp < 0)):
        raise ValueError("cache positions must be ascending and older than the window")
    n_fold = int(d.get("n_fold", max(0, n - eta) - gs))
    rule = d.get("rule", SCORE_SRE)
    ws = gsc = None
    if rule != SCORE_SRE:
        ws, gsc = np.array(d["win_score"], F64), np.array(d["g_score"], F64)
        if ws.shape != (U, w) or gsc.shape != (U, gs):
            raise ValueError("accumulated scores must match the window and the cache")
    return LolaState(eta, lam, n, np.array(d["H"], F64), np.array(d["s"], F64),
                     np.array(d["win_k"], F64), np.array(d["win_v"], F64), gp.copy(),
                     np.array(d["g_k"], F64), np.array(d["g_v"], F64), n_fold, rule, ws, gsc)
