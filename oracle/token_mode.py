"""The per-token recurrence of LoLA, as the notes state it, for one unit.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

LoLA notes §2.4 ("一次单 token 更新的核心过程"): a new pair enters the window;
once the window holds more than eta pairs its oldest pair becomes a candidate;
E_t = G_{t-1} u {leaving pair}; every candidate is scored by SRE against the
state *before* the update and the lam highest form G_t (all kept when there are
fewer than lam); the rest, S_t = E_t \\ G_t, are written into H and s
(Eqs. (11)-(13)).

The state trajectory pins that the chunk schedule with C = 1 follows this
recurrence exactly; the outputs of the literal token mode (each query reads
the memories after its own token's update, LoLA notes §2.5) pin the
read-after-update order of the vectorised form.  The window is a deque of
positions and the scores come from a direct transcription of Eq. (10) with
numpy float64 vectors, independent of the other two forms.
"""

from __future__ import annotations

import math
from collections import deque
from typing import List, Tuple

import numpy as np


def _phi(x: np.ndarray, W: np.ndarray) -> np.ndarray:
    u = x @ W
    a = np.exp(u - u.max())
    b = np.exp(-u - (-u).max())
    return np.concatenate([a / a.sum(), b / b.sum()])


def _token_steps(k: np.ndarray, v: np.ndarray, W: np.ndarray, eta: int, lam: int):
    """The recurrence token by token; yields (t, G, window, H, s) after the
    update of token t (G and the window as positions)."""
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    W = np.asarray(W, np.float64)
    T, d = k.shape
    D = 2 * W.shape[1]
    H = np.zeros((D, d))
    s = np.zeros(D)
    window: deque = deque()
    G: set = set()
    for t in range(T):
        window.append(t)                          # step 1: enter the window
        if len(window) > eta:
            leaving = window.popleft()
            E = G | {leaving}                     # step 2
            if len(E) <= lam:
                G = E
            else:
                def score(p):                     # Eq. (10) on the before-state
                    f = _phi(k[p], W)
                    z = f @ s
                    pred = (f @ H) / z if z > 0 else np.zeros(d)
                    return float(np.sum((pred - v[p]) ** 2))
                ranked = sorted(E, key=lambda p: (-score(p), p))
                G = set(ranked[:lam])             # step 3: Top_lam
                for p in ranked[lam:]:            # step 4: write S_t
                    f = _phi(k[p], W)
                    H = H + np.outer(f, v[p])
                    s = s + f
        yield t, G, tuple(window), H, s


def token_trajectory(k: np.ndarray, v: np.ndarray, W: np.ndarray, eta: int, lam: int
                     ) -> List[Tuple[frozenset, np.ndarray, np.ndarray]]:
    """k, v (T, d); W (d, m).  Returns, after each token t, the tuple
    (cache positions, H copy, s copy)."""
    return [(frozenset(G), H.copy(), s.copy()) for _, G, _, H, s in _token_steps(k, v, W, eta, lam)]


def token_outputs(q: np.ndarray, k: np.ndarray, v: np.ndarray, W: np.ndarray, eta: int,
                  lam: int, branches: int = 7) -> np.ndarray:
    """The literal token mode: every query reads the memories *after* its
    own token's update, LoLA notes §2.5 (y_t with H_t, s_t, G_t and W_t, the
    window holding positions t - eta + 1 .. t).  q (g, T, d) for the q-heads
    of one unit; k, v (T, d).  ``branches`` hides memories as in the
    read-branch ablation (LoLA notes §4.8): bit 1 H and s, bit 2 G, bit 4 the
    window.  Returns y (g, T, d)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g, T, d = q.shape
    y = np.zeros((g, T, d))
    for t, G, window, H, s in _token_steps(k, v, W, eta, lam):
        keys = (sorted(G) if branches & 2 else []) + (list(window) if branches & 4 else [])
        for j in range(g):
            a = np.array([math.exp(float(q[j, t] @ k[p]) / math.sqrt(d)) for p in keys])
            num = (a @ v[keys]) if keys else np.zeros(d)
            den = float(a.sum()) if keys else 0.0
            if branches & 1:
                f = _phi(q[j, t], np.asarray(W, np.float64))
                num = num + f @ H
                den = den + float(f @ s)
            y[j, t] = num / den
    return y
