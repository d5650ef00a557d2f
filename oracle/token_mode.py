"""The per-token recurrence of LoLA, as the notes state it, for one unit.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

LoLA notes §2.4 ("一次单 token 更新的核心过程"): a new pair enters the window;
once the window holds more than eta pairs its oldest pair becomes a candidate;
E_t = G_{t-1} u {leaving pair}; every candidate is scored by SRE against the
state *before* the update and the lam highest form G_t (all kept when there are
fewer than lam); the rest, S_t = E_t \\ G_t, are written into H and s
(Eqs. (11)-(13)).

Only the state trajectory is produced here; it is used to pin that the chunk
schedule with C = 1 follows this recurrence exactly.  The window is a deque of
positions and the scores come from a direct transcription of Eq. (10) with
numpy float64 vectors, independent of the other two forms.
"""

from __future__ import annotations

from collections import deque
from typing import List, Tuple

import numpy as np


def _phi(x: np.ndarray, W: np.ndarray) -> np.ndarray:
    u = x @ W
    a = np.exp(u - u.max())
    b = np.exp(-u - (-u).max())
    return np.concatenate([a / a.sum(), b / b.sum()])


def token_trajectory(k: np.ndarray, v: np.ndarray, W: np.ndarray, eta: int, lam: int
                     ) -> List[Tuple[frozenset, np.ndarray, np.ndarray]]:
    """k, v (T, d); W (d, m).  Returns, after each token t, the tuple
    (cache positions, H copy, s copy)."""
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    W = np.asarray(W, np.float64)
    T, d = k.shape
    D = 2 * W.shape[1]
    H = np.zeros((D, d))
    s = np.zeros(D)
    window: deque = deque()
    G: set = set()
    out = []
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
        out.append((frozenset(G), H.copy(), s.copy()))
    return out
