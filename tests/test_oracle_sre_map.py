"""Pins of the oracle's SRE diagnostics (LoLA notes §4.4, Fig. 3: the
Self-Recall Error of the memories inside the linear state at each chunk;
Eq. (26): relative to their first write).

Each test names the plausible oracle mistakes it would catch.
"""

import math

import numpy as np
import pytest

from oracle import lola as O
from oracle.brute import BruteUnit, brute_sre_map


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _kvw(T, d=5, m=3, seed=0, Hkv=1, B=1):
    k = _rand((B, Hkv, T, d), seed)
    v = _rand((B, Hkv, T, d), seed + 1)
    W = _rand((Hkv, d, m), seed + 2, 1 / math.sqrt(d))
    return k, v, W


@pytest.mark.parametrize("T,C,eta,lam", [(40, 4, 4, 3), (37, 5, 3, 0), (30, 1, 6, 2),
                                         (33, 8, 0, 4), (24, 3, 2, 30)])
def test_vectorised_equals_brute(T, C, eta, lam):
    """The vectorised map and fold chunks against the scalar-loop form (its
    own SRE, position sets and fold bookkeeping).  Catches: reading the state
    after the chunk's update instead of at its start, counting a token as in
    the state in the chunk that folds it, a wrong fold chunk."""
    k, v, W = _kvw(T, seed=T + C)
    st = O.new_state(1, 5, 6, eta, lam)
    m, fold = O.sre_map(st, k, v, W, C)
    u = BruteUnit(5, W[0], eta, lam)
    bm, bf = brute_sre_map(u, k[0, 0], v[0, 0], C)
    np.testing.assert_allclose(m[0], np.array(bm), rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(fold[0], np.array(bf))
    np.testing.assert_allclose(st.H[0], np.array(u.H), rtol=1e-12, atol=1e-14)


def test_single_stored_pair_is_recalled_exactly():
    """lam = 0, C = 1: token 0 is folded when it leaves the window; the first
    state that holds it holds nothing else, so its SRE there is 0 (one stored
    pair is recalled exactly, Eq. (10)).  Catches: a dropped normalisation,
    the entry placed one chunk off."""
    eta = 3
    k, v, W = _kvw(12, seed=4)
    m, fold = O.sre_map(O.new_state(1, 5, 6, eta, 0), k, v, W, 1)
    assert fold[0, 0] == eta                       # leaves at token eta
    assert abs(m[0, eta + 1, 0]) < 1e-24
    assert np.all(m[0, :eta + 1] == 0.0)           # not in the state before that
    assert m[0, eta + 2, 0] > 1e-6                 # a second pair now interferes


def test_constant_values_are_recalled_exactly():
    """With every v equal, H = (sum phi) v^T and s = sum phi, so every key
    reads back v: the whole map is 0 while tokens are folded.  Catches: H and
    s taken from different chunks, a missing division by z."""
    k, v, W = _kvw(30, seed=6)
    v[:] = v[:, :, :1]
    m, fold = O.sre_map(O.new_state(1, 5, 6, 4, 2), k, v, W, 3)
    assert (fold >= 0).sum() > 10
    assert np.abs(m).max() < 1e-24


def test_fold_chunks_match_the_chunk_logs_and_zero_outside_the_state():
    """fold[p] = j exactly for the tokens the chunk-j update leaves out of
    the cache; entries are non-zero only after that chunk."""
    k, v, W = _kvw(36, seed=8, Hkv=2, B=2)
    st = O.new_state(4, 5, 6, 5, 4)
    m, fold = O.sre_map(st, k, v, W, 4)
    st2 = O.new_state(4, 5, 6, 5, 4)
    logs = []
    O.prefill(st2, np.zeros((2, 2, 36, 5)), k, v, W, 4, outputs=False, logs=logs)
    for u in range(4):
        for j, lg in enumerate(logs):
            if lg.keep is None:
                continue
            out = set(lg.cand_pos[u][~lg.keep[u]].tolist())
            assert out == set(np.nonzero(fold[u] == j)[0].tolist())
        for j in range(m.shape[1]):
            inside = (fold[u] >= 0) & (fold[u] < j)
            assert np.all(m[u, j][~inside] == 0.0)
            assert np.all(m[u, j][inside] > 0.0)
    np.testing.assert_array_equal(st.H, st2.H)
