"""Pins of the CPU oracle against what the pages and mathematics fix.

Each test names the plausible oracle mistakes it would catch.  Sizes are tiny
so the whole file runs in seconds on the CPU.
"""

import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import lola as O
from oracle.brute import BruteUnit, brute_prefill
from oracle.token_mode import token_trajectory

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _problem(B=1, Hq=2, Hkv=1, T=40, d=8, m=6, seed=0):
    q = _rand((B, Hq, T, d), seed)
    k = _rand((B, Hkv, T, d), seed + 1)
    v = _rand((B, Hkv, T, d), seed + 2)
    W = _rand((Hkv, d, m), seed + 3, 1 / math.sqrt(d))
    return q, k, v, W


def _run(q, k, v, W, eta, lam, C, logs=None):
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    st = O.new_state(B * Hkv, d, 2 * W.shape[2], eta, lam)
    y = O.prefill(st, q, k, v, W, C, logs=logs)
    return y, st


def _phi_lib(x, W):
    """phi from scipy's softmax (library routine), not the oracle's."""
    u = x @ W
    return np.concatenate([scipy.special.softmax(u, axis=-1),
                           scipy.special.softmax(-u, axis=-1)], axis=-1)


def _sdpa_causal(q, k, v):
    """Exact causal softmax attention via torch's library routine (fp64 CPU);
    GQA by repeating each KV head for its q-heads."""
    g = q.shape[1] // k.shape[1]
    kt = torch.from_numpy(np.repeat(k, g, axis=1))
    vt = torch.from_numpy(np.repeat(v, g, axis=1))
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), kt, vt, is_causal=True)
    return out.numpy()


# ---------------------------------------------------------------- phi
def test_phi_matches_library_softmax_and_halves():
    """Catches: wrong sign in the second half, softmax over the wrong axis,
    missing normalisation."""
    x = _rand((5, 7, 8), 1)
    W = _rand((8, 6), 2)
    f = O.phi(x, W)
    np.testing.assert_allclose(f, _phi_lib(x, W), rtol=1e-14, atol=1e-16)
    np.testing.assert_allclose(f[..., :6].sum(-1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(f[..., 6:].sum(-1), 1.0, rtol=1e-14)
    # phi(-x) swaps the halves
    g = O.phi(-x, W)
    np.testing.assert_allclose(g[..., :6], f[..., 6:], rtol=1e-13)


# ---------------------------------------------------------------- P-a, P-c
@pytest.mark.parametrize("C", [1, 5, 8, 40])
def test_window_covers_everything_is_softmax_attention(C):
    """P-a: eta >= T => nothing leaves the window, H = 0, G empty, and Eq. (14)
    is exact causal softmax attention (diagonal included).  Catches: causal
    mask off by one, wrong 1/sqrt(d) scale, a stray linear term, GQA head
    mapping."""
    q, k, v, W = _problem(Hq=4, Hkv=2, T=40)
    y, st = _run(q, k, v, W, eta=40, lam=3, C=C)
    np.testing.assert_allclose(y, _sdpa_causal(q, k, v), rtol=1e-11, atol=1e-13)
    assert st.g_pos.shape[1] == 0 and np.all(st.H == 0) and np.all(st.s == 0)


@pytest.mark.parametrize("C,eta", [(4, 6), (7, 6), (1, 3), (16, 5)])
def test_large_cache_is_softmax_attention(C, eta):
    """P-c: lam >= T - eta => every leaving token enters G, nothing is folded,
    output is exact softmax attention and G is exactly the leaving tokens.
    Catches: wrong candidate range, tokens dropped between window and cache."""
    T = 33
    q, k, v, W = _problem(T=T)
    y, st = _run(q, k, v, W, eta=eta, lam=T - eta, C=C)
    np.testing.assert_allclose(y, _sdpa_causal(q, k, v), rtol=1e-11, atol=1e-13)
    assert list(st.g_pos[0]) == list(range(0, T - eta))
    assert st.n_fold == 0 and np.all(st.s == 0)
    np.testing.assert_array_equal(st.win_k[0], k[0, 0, T - eta:])


# ---------------------------------------------------------------- P-b
@pytest.mark.parametrize("C,eta", [(4, 8), (8, 8), (5, 7), (1, 4), (12, 5)])
def test_no_cache_is_window_plus_linear_attention(C, eta):
    """P-b: lam = 0 => every token that has left the window is in H, s; the
    output is window softmax plus linear attention, one normaliser.  Closed
    form by prefix sums over positions.  Catches: dropped linear term, separate
    normalisers, H transposed (D != d here), state read after instead of
    before the chunk's own fold, wrong window start."""
    T, d, m = 37, 8, 6
    q, k, v, W = _problem(Hq=2, Hkv=1, T=T, d=d, m=m)
    y, _ = _run(q, k, v, W, eta=eta, lam=0, C=C)
    fk = _phi_lib(k[0, 0], W[0])                          # (T, D)
    outer = fk[:, :, None] * v[0, 0][:, None, :]          # (T, D, d)
    Hc = np.concatenate([np.zeros((1, 2 * m, d)), np.cumsum(outer, 0)])  # Hc[j] = sum_{i<j}
    sc = np.concatenate([np.zeros((1, 2 * m)), np.cumsum(fk, 0)])
    ref = np.zeros_like(y)
    for t in range(T):
        n = (t // C) * C                                  # chunk start
        lo = max(0, n - eta)
        for j in range(2):
            fq = _phi_lib(q[0, j, t], W[0])
            a = np.exp(k[0, 0, lo:t + 1] @ q[0, j, t] / math.sqrt(d))
            num = fq @ Hc[lo] + a @ v[0, 0, lo:t + 1]
            den = fq @ sc[lo] + a.sum()
            ref[0, j, t] = num / den
    np.testing.assert_allclose(y, ref, rtol=1e-11, atol=1e-13)


# ---------------------------------------------------------------- P-d, P-e
def test_sre_zero_for_single_stored_pair():
    """P-d: with one stored pair (k, v), H = phi v^T and s = phi, so
    H^T phi / (phi^T s) = v exactly: SRE = 0 for any k.  phi^T phi != 1 here,
    so a dropped normalisation fails."""
    rng = np.random.default_rng(5)
    for _ in range(5):
        f = rng.random(10) + 0.1
        v = rng.standard_normal(4)
        H = np.outer(f, v)[None]
        s = f[None]
        r = O.sre(f[None, None], v[None, None], H, s)
        assert abs(r[0, 0]) < 1e-24 + 1e-28 * v @ v


def test_sre_zero_for_orthogonal_features():
    """P-d: mutually orthogonal (one-hot) features make every stored pair
    perfectly recalled; a pair not stored has SRE = ||v - v_stored||^2."""
    D, d = 6, 3
    V = np.random.default_rng(7).standard_normal((D, d))
    E = np.eye(D)
    H = (E[:, :, None] * V[:, None, :]).sum(0)[None]      # sum_i e_i v_i^T
    s = E.sum(0)[None]
    r = O.sre(E[None], V[None], H, s)
    np.testing.assert_allclose(r, 0.0, atol=1e-28)
    # an unstored value under a stored feature: error is the plain distance
    r2 = O.sre(E[None, :1], (V[:1] + 2.0)[None], H, s)
    np.testing.assert_allclose(r2, [[4.0 * d]], rtol=1e-14)


def test_teaching_example_opposite_values():
    """P-e, the notes' teaching example (§2.4): two keys with the same features
    and values +1 and -1 written into one state read back 0, so each has
    SRE = 1.  In general identical features give p = (v1 + v2)/2 and
    SRE = ||v1 - v2||^2 / 4.  Golden values: tests/golden/teaching_example.json."""
    with open(os.path.join(GOLDEN, "teaching_example.json")) as fh:
        ex = json.load(fh)
    f = np.asarray(ex["phi"], float)
    vs = np.asarray(ex["values"], float)
    H = sum(np.outer(f, v) for v in vs)[None]
    s = (len(vs) * f)[None]
    r = O.sre(np.stack([f] * len(vs))[None], vs[None], H, s)
    np.testing.assert_allclose(r[0], ex["sre"], rtol=1e-14)
    rng = np.random.default_rng(3)
    v1, v2 = rng.standard_normal((2, 5))
    f = rng.random(8) + 0.05
    H = (np.outer(f, v1) + np.outer(f, v2))[None]
    r = O.sre(np.stack([f, f])[None], np.stack([v1, v2])[None], H, (2 * f)[None])
    np.testing.assert_allclose(r[0], [np.sum((v1 - v2) ** 2) / 4] * 2, rtol=1e-13)


def test_sre_zero_state_rule():
    """O5: H = 0, s = 0 => z = 0 => prediction 0 => SRE = ||v||^2."""
    v = np.random.default_rng(2).standard_normal((1, 4, 5))
    f = np.random.default_rng(3).random((1, 4, 6))
    r = O.sre(f, v, np.zeros((1, 6, 5)), np.zeros((1, 6)))
    np.testing.assert_allclose(r, (v ** 2).sum(-1), rtol=1e-15)


# ---------------------------------------------------------------- P-f
@pytest.mark.parametrize("seed", range(6))
def test_selection_equals_rank_counting(seed):
    """P-f: Top_lam by (score desc, position asc) equals O(n^2) rank counting
    (kept iff fewer than lam candidates come before it), ties included.
    Catches: keeping the lowest, ties to the newer token, over-keeping."""
    rng = np.random.default_rng(seed)
    U, E = 3, 25
    scores = rng.integers(0, 6, size=(U, E)).astype(float)   # many exact ties
    pos = np.stack([rng.permutation(100)[:E] for _ in range(U)])
    for lam in (0, 1, 7, 24):
        keep = O.select_keep(scores, pos, lam)
        for u in range(U):
            for e in range(E):
                better = np.sum((scores[u] > scores[u, e]) |
                                ((scores[u] == scores[u, e]) & (pos[u] < pos[u, e])))
                assert keep[u, e] == (better < lam)
        assert np.all(keep.sum(1) == lam)


def test_selection_prefers_high_sre_and_older_on_tie():
    scores = np.array([[1.0, 5.0, 5.0, 0.5, 3.0]])
    pos = np.array([[10, 40, 20, 30, 50]])
    keep = O.select_keep(scores, pos, 2)
    assert keep.tolist() == [[False, True, True, False, False]]
    keep = O.select_keep(scores, pos, 1)
    assert keep.tolist() == [[False, False, True, False, False]]   # 20 older than 40


# ---------------------------------------------------------------- P-g
@pytest.mark.parametrize("T,C,eta,lam", [
    (24, 4, 6, 5), (23, 5, 4, 3), (20, 1, 3, 2), (30, 8, 8, 8), (17, 6, 3, 0),
    (26, 9, 4, 4), (12, 4, 20, 3), (21, 3, 2, 30)])
def test_vectorised_equals_brute(T, C, eta, lam):
    """P-g: the chunk-vectorised form equals the scalar-loop form (different
    bookkeeping: position sets over the full history, rank counting),
    including C not dividing T and C > eta."""
    B, Hq, Hkv, d, m = 2, 4, 2, 5, 3
    q, k, v, W = _problem(B=B, Hq=Hq, Hkv=Hkv, T=T, d=d, m=m, seed=T * 7 + C)
    y, st = _run(q, k, v, W, eta, lam, C)
    units = [BruteUnit(d, W[u % Hkv], eta, lam) for u in range(B * Hkv)]
    yb = np.array(brute_prefill(units, q, k, v, C), dtype=float)
    np.testing.assert_allclose(y, yb, rtol=1e-12, atol=1e-14)
    for u in range(B * Hkv):
        assert list(st.g_pos[u]) == units[u].cache
        np.testing.assert_allclose(st.H[u], np.array(units[u].H), rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(st.s[u], np.array(units[u].s), rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- P-h
@pytest.mark.parametrize("eta,lam", [(3, 2), (1, 1), (4, 0), (2, 5)])
def test_c1_trajectory_is_token_recurrence(eta, lam):
    """P-h: with C = 1 the state after every token equals the notes' per-token
    recurrence (§2.4 steps 1-4: enter window, oldest leaves, score E against
    the before-state, keep top lam, write the rest).  Catches scoring against
    the after-state and off-by-one window eviction."""
    T, d, m = 30, 4, 3
    q, k, v, W = _problem(T=T, d=d, m=m, seed=11)
    traj = token_trajectory(k[0, 0], v[0, 0], W[0], eta, lam)
    st = O.new_state(1, d, 2 * m, eta, lam)
    for t in range(T):
        O.prefill(st, q[:, :, t:t + 1], k[:, :, t:t + 1], v[:, :, t:t + 1], W, 1)
        G, H, s = traj[t]
        assert set(st.g_pos[0].tolist()) == set(G)
        np.testing.assert_allclose(st.H[0], H, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(st.s[0], s, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- P-i
def test_decode_equals_prefill_t1_and_span_split():
    """P-i: decode is prefill with T = C = 1; prefill(A||B) equals prefill(A)
    then prefill(B) when |A| is a multiple of C; export/import resumes
    exactly."""
    T, C = 32, 4
    q, k, v, W = _problem(B=2, Hq=4, Hkv=2, T=T, seed=21)
    y, st = _run(q, k, v, W, 5, 4, C)
    st2 = O.new_state(4, 8, 12, 5, 4)
    ya = O.prefill(st2, q[:, :, :12], k[:, :, :12], v[:, :, :12], W, C)
    st3 = O.import_state(O.export_state(st2), 5, 4)
    yb = O.prefill(st3, q[:, :, 12:], k[:, :, 12:], v[:, :, 12:], W, C)
    np.testing.assert_allclose(np.concatenate([ya, yb], 2), y, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(st3.H, st.H, rtol=1e-13, atol=1e-15)
    assert np.array_equal(st3.g_pos, st.g_pos)
    # decode == C = 1 prefill
    y1, s1 = _run(q, k, v, W, 5, 4, 1)
    s4 = O.new_state(4, 8, 12, 5, 4)
    for t in range(T):
        yt = O.decode_step(s4, q[:, :, t], k[:, :, t], v[:, :, t], W)
        np.testing.assert_allclose(yt, y1[:, :, t], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(s4.H, s1.H, rtol=1e-13)


# ---------------------------------------------------------------- P-j
@pytest.mark.parametrize("C,eta,lam", [(4, 6, 5), (7, 3, 2), (1, 2, 3), (10, 10, 0)])
def test_mass_and_bookkeeping_invariants(C, eta, lam):
    """P-j: each phi half sums to 1, so 1^T s = 2 N_fold and
    1^T H = 2 sum_folded v^T; N_fold + |G| + |W| = n;
    |G| = min(lam, max(0, n - eta)).  Catches double counting, tokens lost or
    duplicated between memories."""
    T = 45
    q, k, v, W = _problem(B=1, Hq=2, Hkv=1, T=T, seed=31)
    logs = []
    y, st = _run(q, k, v, W, eta, lam, C, logs)
    folded = []
    for lg in logs:
        if lg.keep is not None:
            folded += lg.cand_pos[0][~lg.keep[0]].tolist()
    assert len(folded) == len(set(folded)) == st.n_fold
    np.testing.assert_allclose(st.s.sum(), 2 * st.n_fold, rtol=1e-13)
    vsum = v[0, 0, folded].sum(0) if folded else np.zeros(8)
    np.testing.assert_allclose(st.H[0].sum(0), 2 * vsum, rtol=1e-12, atol=1e-12)
    assert st.n_fold + st.g_pos.shape[1] + st.win_k.shape[1] == T
    assert st.g_pos.shape[1] == min(lam, max(0, T - eta))
    kept = set(st.g_pos[0].tolist())
    assert kept.isdisjoint(folded) and all(p < T - eta for p in kept)


# ---------------------------------------------------------------- P-k
def test_value_scaling_and_cache_permutation():
    """P-k: v -> alpha v gives y -> alpha y, H -> alpha H, SRE -> alpha^2 SRE,
    same membership; permuting the stored cache order leaves y unchanged."""
    q, k, v, W = _problem(T=40, seed=41)
    la, lb = [], []
    y1, s1 = _run(q, k, v, W, 6, 5, 4, la)
    y2, s2 = _run(q, k, 3.0 * v, W, 6, 5, 4, lb)
    np.testing.assert_allclose(y2, 3 * y1, rtol=1e-12)
    np.testing.assert_allclose(s2.H, 3 * s1.H, rtol=1e-12)
    assert np.array_equal(s1.g_pos, s2.g_pos)
    for a, b in zip(la, lb):
        if a.sre is not None:
            np.testing.assert_allclose(b.sre, 9 * a.sre, rtol=1e-12)
    st = O.new_state(1, 8, 12, 6, 5)
    O.prefill(st, q[:, :, :24], k[:, :, :24], v[:, :, :24], W, 4)
    sp = st.copy()
    perm = np.random.default_rng(0).permutation(sp.g_pos.shape[1])
    sp.g_pos, sp.g_k, sp.g_v = sp.g_pos[:, perm], sp.g_k[:, perm], sp.g_v[:, perm]
    ya = O.prefill(st.copy(), q[:, :, 24:28], k[:, :, 24:28], v[:, :, 24:28], W, 4)
    yb = O.prefill(sp, q[:, :, 24:28], k[:, :, 24:28], v[:, :, 24:28], W, 4)
    np.testing.assert_allclose(ya, yb, rtol=1e-13)


# ---------------------------------------------------------------- P-l
def test_state_size_formula_golden():
    """P-l: persistent elements per head, the notes' §2.7 formula, checked on
    the page's own arithmetic (ratio 6.39 at t = 4096, d_k = d_v = 128,
    D = 256, (eta, lam) = (256, 256)) and saturation at (eta + lam)."""
    with open(os.path.join(GOLDEN, "state_size.json")) as fh:
        ex = json.load(fh)
    full = ex["t"] * (ex["d_k"] + ex["d_v"])
    lola = O.state_elements(ex["d_k"], ex["d_v"], ex["D"], ex["eta"], ex["lam"], ex["t"])
    assert lola == ex["lola_elements"]
    assert round(full / lola, 2) == ex["ratio"]
    assert O.state_elements(128, 128, 256, 256, 256, 100) == 100 * 256


def test_oracle_state_matches_formula():
    """The oracle's state holds the formula's element count: while t <= eta +
    lam nothing is folded and every token is explicit (t (d_k + d_v)); once
    the budget is exceeded by more than the linear state's size, the state is
    (eta + lam)(d_k + d_v) + D d_v + D."""
    T, d, m, eta, lam = 40, 8, 6, 6, 5
    q, k, v, W = _problem(T=T, d=d, m=m)
    for t_end in (3, 9, 11, 30, 40):
        st = O.new_state(1, d, 2 * m, eta, lam)
        O.prefill(st, q[:, :1, :t_end], k[:, :, :t_end], v[:, :, :t_end], W, 4)
        explicit = (st.win_k.shape[1] + st.g_k.shape[1]) * 2 * d
        lin = st.H[0].size + st.s[0].size if st.n_fold > 0 else 0
        if t_end <= eta + lam:
            assert st.n_fold == 0 and explicit == t_end * 2 * d
        else:
            assert explicit + lin == (eta + lam) * 2 * d + 2 * m * d + 2 * m
        if t_end * 2 * d >= explicit + lin or t_end <= eta + lam:
            assert explicit + lin == O.state_elements(d, d, 2 * m, eta, lam, t_end)


# ---------------------------------------------------------------- P-m
def test_gqa_equals_replicated_kv_heads():
    """P-m: Hq = g * Hkv equals running each q-head against its own copy of
    its KV head (q-head j reads KV head floor(j / g))."""
    q, k, v, W = _problem(B=2, Hq=6, Hkv=2, T=30, seed=51)
    y, _ = _run(q, k, v, W, 5, 4, 3)
    kr, vr, Wr = np.repeat(k, 3, 1), np.repeat(v, 3, 1), np.repeat(W, 3, 0)
    yr, _ = _run(q, kr, vr, Wr, 5, 4, 3)
    np.testing.assert_allclose(y, yr, rtol=1e-13)


# ------------------------------------------------------ boundary gap (chunk log)
def test_boundary_gap_hand_values():
    """gamma = (SRE_(lam) - SRE_(lam+1)) / SRE_(lam) with SRE_(i) the i-th
    largest: values worked by hand, a tie at the boundary (0), and a zero
    lam-th value (inf)."""
    sc = np.array([[4.0, 9.0, 1.0, 7.0, 4.0]])
    assert O.boundary_gap(sc, 1)[0] == pytest.approx(2 / 9)      # 9 vs 7
    assert O.boundary_gap(sc, 2)[0] == pytest.approx(3 / 7)      # 7 vs 4
    assert O.boundary_gap(sc, 3)[0] == 0.0                      # 4 vs 4: a tie
    assert O.boundary_gap(sc, 4)[0] == pytest.approx(3 / 4)      # 4 vs 1
    assert O.boundary_gap(np.array([[0.0, 0.0, 0.0]]), 1)[0] == np.inf


@pytest.mark.parametrize("seed", range(4))
def test_boundary_gap_is_the_kept_minimum_against_the_folded_maximum(seed):
    """The lam-th largest SRE is the smallest kept one and the (lam+1)-th the
    largest folded one, for the membership select_keep gives (itself pinned
    by rank counting above).  Catches an off-by-one in either order statistic."""
    rng = np.random.default_rng(seed)
    U, E = 4, 30
    scores = rng.random((U, E)) + 0.1
    scores[:, :6] = scores[:, 6:12]                              # some exact ties
    pos = np.stack([rng.permutation(E) for _ in range(U)])
    for lam in (1, 5, 17, 29):
        keep = O.select_keep(scores, pos, lam)
        g = O.boundary_gap(scores, lam)
        for u in range(U):
            a, b = scores[u][keep[u]].min(), scores[u][~keep[u]].max()
            assert g[u] == pytest.approx((a - b) / a, rel=1e-14, abs=1e-300)


def test_identical_pairs_score_bitwise_equal():
    """Duplicate (k, v) pairs among the candidates get bitwise-equal SRE, so
    the tie rule (older position first) decides between them; the exact-tie
    stress inputs rely on this."""
    rng = np.random.default_rng(5)
    U, d, m = 2, 16, 8
    W = rng.standard_normal((d, m)) / np.sqrt(d)
    pool_k, pool_v = rng.standard_normal((5, d)), rng.standard_normal((5, d))
    idx = rng.integers(0, 5, size=97)
    k = np.broadcast_to(pool_k[idx], (U, 97, d))
    v = np.broadcast_to(pool_v[idx], (U, 97, d))
    ph = np.stack([O.phi(k[u], W) for u in range(U)])
    H, s = rng.random((U, 2 * m, d)), rng.random((U, 2 * m))
    sc = O.sre(ph, v, H, s)
    for u in range(U):
        for j in range(5):
            grp = sc[u][idx == j]
            assert np.all(grp == grp[0])


def test_imposed_kept_set():
    """Continuing along another kept set (an allowed choice at a near-tie):
    imposing the set the oracle itself selects reproduces its state bit for
    bit; imposing another set keeps the bookkeeping invariants and moves the
    swapped pairs between the cache and H, s."""
    q, k, v, W = _problem(B=1, Hq=2, Hkv=1, T=40, d=8, m=6, seed=3)
    eta, lam, C = 4, 5, 8
    st = O.new_state(1, 8, 12, eta, lam)
    O.prefill(st, q[:, :, :24], k[:, :, :24], v[:, :, :24], W, C)
    a, b = st.copy(), st.copy()
    logs = []
    ya = O.prefill(a, q[:, :, 24:32], k[:, :, 24:32], v[:, :, 24:32], W, C, logs=logs)
    lg = logs[0]
    assert lg.sre is not None
    own = [set(lg.cand_pos[0][lg.keep[0]].tolist())]
    yb = O.prefill(b, q[:, :, 24:32], k[:, :, 24:32], v[:, :, 24:32], W, C, keep=own)
    assert np.array_equal(ya, yb) and np.array_equal(a.H, b.H) and np.array_equal(a.g_pos, b.g_pos)
    # swap the weakest kept candidate with the strongest folded one
    order = np.lexsort((lg.cand_pos[0], -lg.sre[0]))
    alt = set(lg.cand_pos[0][order[:lam - 1]].tolist()) | {int(lg.cand_pos[0][order[lam]])}
    c = st.copy()
    O.prefill(c, q[:, :, 24:32], k[:, :, 24:32], v[:, :, 24:32], W, C, keep=[alt])
    assert set(c.g_pos[0].tolist()) == alt and c.n_fold == a.n_fold
    np.testing.assert_allclose(c.s.sum(), 2 * c.n_fold, rtol=1e-12)
    x, y = int(lg.cand_pos[0][order[lam - 1]]), int(lg.cand_pos[0][order[lam]])
    dH = O.phi(k[0, 0, x], W[0])[:, None] * v[0, 0, x] - O.phi(k[0, 0, y], W[0])[:, None] * v[0, 0, y]
    np.testing.assert_allclose(c.H[0] - a.H[0], dH, rtol=1e-10, atol=1e-12)
    with pytest.raises(ValueError):
        O.prefill(st.copy(), q[:, :, 24:32], k[:, :, 24:32], v[:, :, 24:32], W, C,
                  keep=[set(list(alt)[:2])])
