"""Pins of the oracle's read-branch masks (LoLA notes §4.8, Table 12: the
ablation hides memories from the queries; the memories themselves are updated
as before).

Each test names the plausible oracle mistakes it would catch.
"""

import math

import numpy as np
import pytest
import scipy.special

from oracle import lola as O
from oracle.brute import BruteUnit, brute_prefill


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _problem(B=1, Hq=2, Hkv=1, T=40, d=8, m=6, seed=0):
    q = _rand((B, Hq, T, d), seed)
    k = _rand((B, Hkv, T, d), seed + 1)
    v = _rand((B, Hkv, T, d), seed + 2)
    W = _rand((Hkv, d, m), seed + 3, 1 / math.sqrt(d))
    return q, k, v, W


def _chunkwise(q, k, v, W, eta, lam, C, branches):
    """Prefill chunk by chunk, recording the cache positions each chunk reads."""
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    st = O.new_state(B * Hkv, d, 2 * W.shape[2], eta, lam)
    ys, caches = [], []
    for t0 in range(0, T, C):
        sl = slice(t0, min(T, t0 + C))
        caches.append(st.g_pos.copy())
        ys.append(O.prefill(st, q[:, :, sl], k[:, :, sl], v[:, :, sl], W, C, branches=branches))
    return np.concatenate(ys, axis=2), caches, st


def _softmax_read(q, k, v, pos):
    """softmax(q . k_p / sqrt(d)) over the key positions `pos`, via scipy."""
    d = q.shape[-1]
    w = scipy.special.softmax(k[pos] @ q / math.sqrt(d))
    return w @ v[pos]


@pytest.mark.parametrize("C,eta,lam", [(4, 6, 5), (5, 3, 4), (1, 4, 2), (8, 8, 3)])
def test_window_only_is_sliding_window_softmax(C, eta, lam):
    """Mask 4 reads only the local keys: exact causal softmax attention over
    positions max(0, n - eta) .. t (n = chunk start).  Catches: cache keys or
    the linear terms leaking into the read, a window that starts one off, the
    causal prefix of the chunk dropped."""
    T = 31
    q, k, v, W = _problem(Hq=2, Hkv=1, T=T)
    y, _, _ = _chunkwise(q, k, v, W, eta, lam, C, branches=4)
    for t in range(T):
        n = (t // C) * C
        pos = np.arange(max(0, n - eta), t + 1)
        for j in range(2):
            np.testing.assert_allclose(y[0, j, t], _softmax_read(q[0, j, t], k[0, 0], v[0, 0], pos),
                                       rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("C,eta,lam", [(4, 6, 5), (5, 3, 4), (3, 2, 6)])
def test_sparse_and_window_is_softmax_over_cache_and_window(C, eta, lam):
    """Mask 6 hides H and s: exact softmax over the cache at chunk start
    together with the local keys.  Catches: the linear terms kept in the
    numerator or the denominator only, the cache read after the chunk's own
    update instead of before."""
    T = 33
    q, k, v, W = _problem(Hq=2, Hkv=1, T=T, seed=5)
    y, caches, _ = _chunkwise(q, k, v, W, eta, lam, C, branches=6)
    for t in range(T):
        n = (t // C) * C
        pos = np.concatenate([caches[t // C][0], np.arange(max(0, n - eta), t + 1)]).astype(int)
        for j in range(2):
            np.testing.assert_allclose(y[0, j, t], _softmax_read(q[0, j, t], k[0, 0], v[0, 0], pos),
                                       rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("branches", [4, 5, 6, 7])
@pytest.mark.parametrize("T,C,eta,lam", [(24, 4, 6, 5), (23, 5, 4, 3), (20, 1, 3, 2), (17, 6, 3, 0)])
def test_masked_vectorised_equals_brute(branches, T, C, eta, lam):
    """Every mask, the chunk-vectorised form against the scalar-loop form
    (which skips the hidden memories while it gathers the visible keys).
    Catches: the state mask (bit 1) mapped to the cache or the reverse, a
    mask applied to one GQA head only."""
    B, Hq, Hkv, d, m = 2, 4, 2, 5, 3
    q, k, v, W = _problem(B=B, Hq=Hq, Hkv=Hkv, T=T, d=d, m=m, seed=T * 3 + C)
    st = O.new_state(B * Hkv, d, 2 * m, eta, lam)
    y = O.prefill(st, q, k, v, W, C, branches=branches)
    units = [BruteUnit(d, W[u % Hkv], eta, lam) for u in range(B * Hkv)]
    yb = np.array(brute_prefill(units, q, k, v, C, branches=branches), dtype=float)
    np.testing.assert_allclose(y, yb, rtol=1e-12, atol=1e-14)


def test_masks_leave_the_updates_unchanged():
    """The ablation changes reads only: H, s, the cache and the window after a
    prefill and a few decode steps are bitwise the same for every mask.
    Catches: a mask that also skips the fold or the cache update."""
    q, k, v, W = _problem(B=1, Hq=4, Hkv=2, T=30, d=6, m=4, seed=9)
    ref = None
    for br in (7, 6, 5, 4):
        st = O.new_state(2, 6, 8, 5, 4)
        O.prefill(st, q, k, v, W, 4, branches=br)
        for i in range(3):
            O.decode_step(st, _rand((1, 4, 6), 40 + i), _rand((1, 2, 6), 50 + i),
                          _rand((1, 2, 6), 60 + i), W, branches=br)
        cur = (st.H, st.s, st.g_pos, st.g_k, st.win_k, st.n)
        if ref is None:
            ref = cur
            continue
        for a, b in zip(cur, ref):
            np.testing.assert_array_equal(a, b)


def test_full_mask_is_the_default_read():
    """Mask 7 reads every memory: it is the unmasked call.  Catches: a
    default that silently drops a branch."""
    q, k, v, W = _problem(Hq=2, Hkv=1, T=25, seed=11)
    st1 = O.new_state(1, 8, 12, 4, 3)
    st2 = O.new_state(1, 8, 12, 4, 3)
    np.testing.assert_array_equal(O.prefill(st1, q, k, v, W, 4),
                                  O.prefill(st2, q, k, v, W, 4, branches=7))


@pytest.mark.parametrize("bad", [0, 1, 2, 3, 8, 15, -1])
def test_invalid_masks_are_rejected(bad):
    """A mask without the window bit (the normaliser could vanish) or with
    unknown bits is an error."""
    with pytest.raises(ValueError):
        O.check_branches(bad)
