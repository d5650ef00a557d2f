"""Pins of the oracle's literal token mode: token t's query reads the
memories after token t's update (LoLA notes §2.4 steps 1-4, then §2.5 with
H_t, s_t, G_t and W_t = positions t - eta + 1 .. t).

Each test names the plausible oracle mistakes it would catch.
"""

import math

import numpy as np
import pytest
import torch

from oracle import lola as O
from oracle.token_mode import token_outputs


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _problem(Hq=2, T=30, d=6, m=4, seed=0):
    q = _rand((1, Hq, T, d), seed)
    k = _rand((1, 1, T, d), seed + 1)
    v = _rand((1, 1, T, d), seed + 2)
    W = _rand((1, d, m), seed + 3, 1 / math.sqrt(d))
    return q, k, v, W


def _after(q, k, v, W, eta, lam, branches=7):
    st = O.new_state(1, q.shape[-1], 2 * W.shape[2], eta, lam)
    return O.prefill(st, q, k, v, W, 1, order="after", branches=branches), st


def _sdpa_causal(q, k, v):
    g = q.shape[1] // k.shape[1]
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(np.repeat(k, g, axis=1)),
        torch.from_numpy(np.repeat(v, g, axis=1)), is_causal=True)
    return out.numpy()


@pytest.mark.parametrize("branches", [7, 5, 6])
@pytest.mark.parametrize("eta,lam", [(4, 3), (1, 2), (3, 0), (6, 10), (0, 3), (0, 0)])
def test_vectorised_equals_token_recurrence(eta, lam, branches):
    """The vectorised read-after-update against the deque form of the
    recurrence (its own scores, window and Top_lam).  Catches: reading the
    window before the leaving pair is moved out, the leaving pair still read
    as a window key, H or G taken before the update, eta = 0 mishandled."""
    if eta == 0 and not ((lam > 0 and branches & 2) or (lam == 0 and branches & 1)):
        pytest.skip("no memory left to read")
    q, k, v, W = _problem(seed=eta * 10 + lam)
    y, _ = _after(q, k, v, W, eta, lam, branches)
    yt = token_outputs(q[0], k[0, 0], v[0, 0], W[0], eta, lam, branches)
    np.testing.assert_allclose(y[0], yt, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("eta,lam", [(30, 2), (40, 0), (3, 30), (1, 29)])
def test_no_fold_is_causal_softmax(eta, lam):
    """eta >= T or lam >= T: nothing is folded, G_t u W_t holds every
    position <= t, and the read is exact causal softmax attention (torch's
    library routine).  Catches: a key dropped or read twice when it moves
    from the window to the cache."""
    q, k, v, W = _problem(Hq=2, T=30)
    y, st = _after(q, k, v, W, eta, lam)
    np.testing.assert_allclose(y, _sdpa_causal(q, k, v), rtol=1e-11, atol=1e-13)
    assert np.all(st.s == 0)


@pytest.mark.parametrize("eta", [1, 3, 5])
def test_no_cache_closed_form(eta):
    """lam = 0: the pair leaving at token t (position t - eta) is in H_t before
    the query reads, the window is t - eta + 1 .. t.  Closed form by prefix
    sums.  Catches: an off-by-one between the fold and the read, H_t - 1 read
    instead of H_t."""
    T, d, m = 27, 6, 4
    q, k, v, W = _problem(Hq=2, T=T, d=d, m=m, seed=3)
    y, _ = _after(q, k, v, W, eta, 0)
    u = k[0, 0] @ W[0]
    fk = np.concatenate([np.exp(u - u.max(-1, keepdims=True)), np.exp(-u + u.min(-1, keepdims=True))], -1)
    fk[:, :m] /= fk[:, :m].sum(-1, keepdims=True)
    fk[:, m:] /= fk[:, m:].sum(-1, keepdims=True)
    Hc = np.concatenate([np.zeros((1, 2 * m, d)), np.cumsum(fk[:, :, None] * v[0, 0][:, None], 0)])
    sc = np.concatenate([np.zeros((1, 2 * m)), np.cumsum(fk, 0)])
    for t in range(T):
        lo = max(0, t - eta + 1)                   # window start; positions < lo are in H
        for j in range(2):
            uq = q[0, j, t] @ W[0]
            fq = np.concatenate([np.exp(uq - uq.max()), np.exp(-uq + uq.min())])
            fq[:m] /= fq[:m].sum()
            fq[m:] /= fq[m:].sum()
            a = np.exp(k[0, 0, lo:t + 1] @ q[0, j, t] / math.sqrt(d))
            ref = (fq @ Hc[lo] + a @ v[0, 0, lo:t + 1]) / (fq @ sc[lo] + a.sum())
            np.testing.assert_allclose(y[0, j, t], ref, rtol=1e-11, atol=1e-13)


def test_order_does_not_change_the_state():
    """Only the read moves: the state after every token is the same for both
    orders.  Catches: the after-order updating twice or skipping an update."""
    q, k, v, W = _problem(T=25, seed=7)
    _, sa = _after(q, k, v, W, 4, 3)
    sb = O.new_state(1, 6, 8, 4, 3)
    O.prefill(sb, q, k, v, W, 1)
    for a, b in zip((sa.H, sa.s, sa.g_pos, sa.win_k, sa.n), (sb.H, sb.s, sb.g_pos, sb.win_k, sb.n)):
        np.testing.assert_array_equal(a, b)


def test_after_order_needs_token_steps_and_a_readable_memory():
    q, k, v, W = _problem(T=8)
    with pytest.raises(ValueError):
        O.prefill(O.new_state(1, 6, 8, 4, 3), q, k, v, W, 4, order="after")
    with pytest.raises(ValueError):   # eta = 0, lam = 0, state hidden: nothing to read
        O.prefill(O.new_state(1, 6, 8, 0, 0), q, k, v, W, 1, order="after", branches=6)
