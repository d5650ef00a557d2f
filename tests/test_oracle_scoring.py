"""Pins of the oracle's alternative cache scoring rules (LoLA notes §4.5,
Table 4: the ablation replaces SRE by scores of the exponential kernel
e = exp(q.k/sqrt(d)) against the feature kernel c = phi(q)^T phi(k), or by
accumulated local attention; the notes give the rules in words, the formulas
are in the paper's Appendix F, not on the pages).  Reading: each rule sums
its term over the local queries (all query heads of the KV head) that see a
key through the window, and the sum is frozen when the key leaves it.

* the chunk-vectorised oracle equals the scalar-loop form (oracle/brute.py)
  on several schedules, for every rule;
* frozen scores make the cache the exact top-lambda (score desc, position
  asc) of every token that has left the window, at every chunk;
* with one (query, key) pair per key (g = 1, C = 1, eta = 0) the squared and
  the absolute kernel errors rank alike, so the caches agree; with more
  terms per key they are different rules (Table 4 reports different
  accuracies for them);
* the rules read no value and no state: other values leave the cache
  trajectory unchanged;
* decode is prefill with T = C = 1; the SRE map is refused.
"""

import math

import numpy as np
import pytest

from oracle import brute as Br
from oracle import lola as O

RULES = [O.SCORE_KERNEL_SQ, O.SCORE_KERNEL_ABS, O.SCORE_KERNEL_RATIO, O.SCORE_LOCAL_ATTN]


def _problem(B=1, Hq=2, Hkv=1, T=40, d=8, m=6, seed=0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, T, d))
    k = rng.standard_normal((B, Hkv, T, d))
    v = rng.standard_normal((B, Hkv, T, d))
    W = rng.standard_normal((Hkv, d, m)) / math.sqrt(d)
    return q, k, v, W


def _oracle(q, k, v, W, eta, lam, C, rule, logs=None):
    B, Hq, T, d = q.shape
    st = O.new_state(B * W.shape[0], d, 2 * W.shape[2], eta, lam, rule=rule)
    y = O.prefill(st, q, k, v, W, C, logs=logs)
    return y, st


@pytest.mark.parametrize("rule", RULES)
@pytest.mark.parametrize("T,C,eta,lam,Hq", [(30, 4, 6, 5, 2), (23, 5, 3, 4, 1), (20, 1, 2, 3, 2),
                                            (26, 7, 0, 4, 2), (24, 6, 5, 0, 1)])
def test_vectorised_equals_scalar_loops(rule, T, C, eta, lam, Hq):
    q, k, v, W = _problem(B=2, Hq=Hq, T=T, seed=T + C)
    y, st = _oracle(q, k, v, W, eta, lam, C, rule)
    units = [Br.BruteUnit(8, W[0], eta, lam, rule) for _ in range(2)]
    yb = np.array(Br.brute_prefill(units, q, k, v, C), dtype=float)
    np.testing.assert_allclose(y, yb, rtol=1e-11, atol=1e-13)
    for u, bu in enumerate(units):
        assert st.g_pos[u].tolist() == sorted(bu.cache)
        np.testing.assert_allclose(st.H[u], np.array(bu.H), rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(st.g_score[u], [bu.acc[p] for p in st.g_pos[u]], rtol=1e-11)
        w = st.win_k.shape[1]
        np.testing.assert_allclose(st.win_score[u], [bu.acc[p] for p in range(T - w, T)],
                                   rtol=1e-11)


@pytest.mark.parametrize("rule", RULES)
def test_cache_is_the_top_lambda_of_every_left_token(rule):
    q, k, v, W = _problem(B=1, Hq=2, T=60, seed=4)
    eta, lam, C = 5, 7, 4
    logs = []
    st = O.new_state(1, 8, 12, eta, lam, rule=rule)
    bu = Br.BruteUnit(8, W[0], eta, lam, rule)
    for t0 in range(0, 60, C):
        O.prefill(st, q[:, :, t0:t0 + C], k[:, :, t0:t0 + C], v[:, :, t0:t0 + C], W, C)
        Br.brute_prefill([bu], q[:, :, t0:t0 + C], k[:, :, t0:t0 + C], v[:, :, t0:t0 + C], C,
                         n0=t0)
        left = np.arange(max(0, st.n - eta))
        if left.size == 0:
            continue
        sc = np.array([bu.acc[int(p)] for p in left])
        keep = O.select_keep(sc[None], left[None], lam)[0]
        assert st.g_pos[0].tolist() == left[keep].tolist(), t0


def test_squared_and_absolute_errors_agree_with_one_term_per_key():
    q, k, v, W = _problem(B=1, Hq=1, T=50, seed=7)
    _, a = _oracle(q, k, v, W, 0, 9, 1, O.SCORE_KERNEL_SQ)
    _, b = _oracle(q, k, v, W, 0, 9, 1, O.SCORE_KERNEL_ABS)
    assert np.array_equal(a.g_pos, b.g_pos)
    np.testing.assert_allclose(a.g_score, b.g_score ** 2, rtol=1e-12)
    # more terms per key: the sums rank differently somewhere
    differ = False
    for seed in range(6):
        q, k, v, W = _problem(B=1, Hq=2, T=60, seed=seed)
        _, a = _oracle(q, k, v, W, 6, 5, 4, O.SCORE_KERNEL_SQ)
        _, b = _oracle(q, k, v, W, 6, 5, 4, O.SCORE_KERNEL_ABS)
        differ = differ or not np.array_equal(a.g_pos, b.g_pos)
    assert differ


@pytest.mark.parametrize("rule", RULES)
def test_rules_read_no_value_and_no_state(rule):
    q, k, v, W = _problem(B=1, Hq=2, T=48, seed=9)
    v2 = np.random.default_rng(99).standard_normal(v.shape) * 5.0
    _, a = _oracle(q, k, v, W, 4, 6, 4, rule)
    _, b = _oracle(q, k, v2, W, 4, 6, 4, rule)
    assert np.array_equal(a.g_pos, b.g_pos)
    np.testing.assert_array_equal(a.g_score, b.g_score)
    # the SRE rule does read the values
    _, c = _oracle(q, k, v, W, 4, 6, 4, O.SCORE_SRE)
    _, e = _oracle(q, k, v2, W, 4, 6, 4, O.SCORE_SRE)
    assert not np.array_equal(c.g_pos, e.g_pos)


@pytest.mark.parametrize("rule", RULES)
def test_decode_is_prefill_t1_and_export_round_trip(rule):
    q, k, v, W = _problem(B=1, Hq=2, T=30, seed=11)
    _, a = _oracle(q, k, v, W, 4, 5, 1, rule)
    b = O.new_state(1, 8, 12, 4, 5, rule=rule)
    for t in range(30):
        O.decode_step(b, q[:, :, t], k[:, :, t], v[:, :, t], W)
    assert np.array_equal(a.g_pos, b.g_pos)
    np.testing.assert_array_equal(a.g_score, b.g_score)
    np.testing.assert_array_equal(a.H, b.H)
    c = O.import_state(O.export_state(b), 4, 5)
    assert c.rule == rule
    np.testing.assert_array_equal(c.win_score, b.win_score)
    with pytest.raises(ValueError):
        O.sre_map(c, k, v, W, 4)
    with pytest.raises(ValueError):
        O.prefill(c, q[:, :, :1], k[:, :, :1], v[:, :, :1], W, 1, order="after")
