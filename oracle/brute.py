"""Scalar-loop form of LoLA's attention step, for tiny shapes only.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

This is the same method as :mod:`oracle.lola` written a second, independent
way: plain Python floats and loops, the whole token history kept as lists, the
window and cache held as *sets of positions* into that history rather than as
arrays of pairs, and membership decided by counting how many candidates beat
each one (a candidate is kept iff fewer than lam others come before it in the
order SRE descending, position ascending).  Sources, as in the vectorised form:
LoLA notes §2.2 Eqs. (3)-(5), §2.3 Eq. (10), §2.4 Eqs. (11)-(13), §2.5
Eq. (14), §2.6 Eq. (15).

Use it only for T <= a few hundred, d <= 16: it is O(T * (eta + lam) * d) pure
Python per unit.
"""

from __future__ import annotations

import math
from typing import List, Sequence


def _phi_row(x: Sequence[float], W: Sequence[Sequence[float]]) -> List[float]:
    d, m = len(W), len(W[0])
    u = [sum(x[i] * W[i][j] for i in range(d)) for j in range(m)]
    hi = max(u)
    ep = [math.exp(uj - hi) for uj in u]
    lo = min(u)
    en = [math.exp(lo - uj) for uj in u]          # exp(-u_j - max(-u))
    sp, sn = sum(ep), sum(en)
    return [e / sp for e in ep] + [e / sn for e in en]


def _rule_term(rule: str, e: float, c: float) -> float:
    """One (query, key) term of an accumulated scoring rule (LoLA notes §4.5,
    Table 4): e the exponential kernel, c the feature kernel."""
    if rule == "kernel_sq":
        return (e - c) * (e - c)
    if rule == "kernel_abs":
        return abs(e - c)
    if rule == "kernel_ratio":
        return c / e
    if rule == "local_attn":
        return e
    raise ValueError(rule)


class BruteUnit:
    """One (sequence, KV head) unit with its own history and memories.

    ``rule``: "sre", or an accumulated rule whose per-position scores live in
    ``acc``: every query that sees a position through the window adds its
    term while the position is in the window."""

    def __init__(self, d: int, W, eta: int, lam: int, rule: str = "sre"):
        self.d = d
        self.W = [list(map(float, row)) for row in W]
        self.D = 2 * len(self.W[0])
        self.eta, self.lam = eta, lam
        self.hist_k: List[List[float]] = []
        self.hist_v: List[List[float]] = []
        self.cache: List[int] = []                # positions, ascending
        self.H = [[0.0] * d for _ in range(self.D)]
        self.s = [0.0] * self.D
        self.folded: List[int] = []
        self.rule = rule
        self.acc = {}                              # position -> accumulated score

    # -- the accumulated rules: query q (of token t, chunk start n) adds its
    # term to every position it sees through the window
    def accumulate(self, q: Sequence[float], t: int, n: int) -> None:
        fq = _phi_row(q, self.W)
        for p in range(max(0, n - self.eta), t + 1):
            k = self.hist_k[p]
            e = math.exp(sum(q[i] * k[i] for i in range(self.d)) / math.sqrt(self.d))
            fk = _phi_row(k, self.W)
            c = sum(fq[i] * fk[i] for i in range(self.D))
            self.acc[p] = self.acc.get(p, 0.0) + _rule_term(self.rule, e, c)

    # -- Eq. (14), state at chunk start; `branches` (bit 1 state, 2 cache,
    # 4 window) leaves out the hidden memories (LoLA notes §4.8, Table 12)
    def read(self, q: Sequence[float], t: int, n: int, branches: int = 7) -> List[float]:
        d, D = self.d, self.D
        num, den = [0.0] * d, 0.0
        if branches & 1:
            fq = _phi_row(q, self.W)
            num = [sum(fq[i] * self.H[i][c] for i in range(D)) for c in range(d)]
            den = sum(fq[i] * self.s[i] for i in range(D))
        visible = []
        if branches & 2:
            visible += list(self.cache)
        if branches & 4:
            visible += list(range(max(0, n - self.eta), t + 1))
        for p in visible:
            a = math.exp(sum(q[i] * self.hist_k[p][i] for i in range(d)) / math.sqrt(d))
            den += a
            for c in range(d):
                num[c] += a * self.hist_v[p][c]
        return [x / den for x in num]

    # -- Eq. (10), squared
    def sre_of(self, p: int) -> float:
        f = _phi_row(self.hist_k[p], self.W)
        z = sum(f[i] * self.s[i] for i in range(self.D))
        err = 0.0
        for c in range(self.d):
            pred = (sum(f[i] * self.H[i][c] for i in range(self.D)) / z) if z > 0 else 0.0
            err += (pred - self.hist_v[p][c]) ** 2
        return err

    # -- Eqs. (11)-(13) over the chunk's leaving tokens
    def update(self, n: int, c: int) -> None:
        leaving = list(range(max(0, n - self.eta), max(0, n + c - self.eta)))
        cand = sorted(self.cache + leaving)
        if len(cand) <= self.lam:
            self.cache = cand
            return
        if self.rule == "sre":
            score = {p: self.sre_of(p) for p in cand}   # all against the before-state
        else:
            score = {p: self.acc[p] for p in cand}      # frozen since p left the window
        kept, out = [], []
        for p in cand:
            better = sum(1 for o in cand
                         if score[o] > score[p] or (score[o] == score[p] and o < p))
            (kept if better < self.lam else out).append(p)
        for p in out:
            f = _phi_row(self.hist_k[p], self.W)
            for i in range(self.D):
                self.s[i] += f[i]
                for cc in range(self.d):
                    self.H[i][cc] += f[i] * self.hist_v[p][cc]
        self.folded.extend(out)
        self.cache = kept


def brute_prefill(units: List[BruteUnit], q, k, v, C: int, n0: int = 0, branches: int = 7):
    """Run T tokens through every unit with chunk length C.

    units: B*Hkv BruteUnit, unit b*Hkv + h for sequence b, KV head h.
    q (B, Hq, T, d), k, v (B, Hkv, T, d) as nested sequences or arrays.
    n0: tokens the units have already seen.  Returns y as nested lists
    [B][Hq][T][d].  ``branches``: read mask (see BruteUnit.read).
    """
    B, Hq, T = len(q), len(q[0]), len(q[0][0])
    Hkv = len(k[0])
    g = Hq // Hkv
    y = [[[None] * T for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hkv):
            u = units[b * Hkv + h]
            t0 = 0
            while t0 < T:
                c = min(C, T - t0)
                n = n0 + t0
                for t in range(t0, t0 + c):
                    u.hist_k.append([float(x) for x in k[b][h][t]])
                    u.hist_v.append([float(x) for x in v[b][h][t]])
                for t in range(t0, t0 + c):
                    for j in range(g):
                        y[b][h * g + j][t] = u.read([float(x) for x in q[b][h * g + j][t]],
                                                    n0 + t, n, branches)
                if u.rule != "sre":
                    for t in range(t0, t0 + c):
                        for j in range(g):
                            u.accumulate([float(x) for x in q[b][h * g + j][t]], n0 + t, n)
                u.update(n, c)
                t0 += c
    return y


def brute_sre_map(unit: BruteUnit, k, v, C: int):
    """The SRE of every memory in the linear state at each chunk start
    (LoLA notes §4.4, Fig. 3): for one unit, k, v (T, d) the call's tokens.
    Returns (map [nch][T], fold [T]) as nested lists, with the conventions of
    ``oracle.lola.sre_map``: 0 for tokens not in the state, fold = the chunk
    whose update wrote the token, -1 if none."""
    T = len(k)
    n0 = len(unit.hist_k)
    nch = (T + C - 1) // C
    m = [[0.0] * T for _ in range(nch)]
    fold = [-1] * T
    for j in range(nch):
        t0 = j * C
        for p in range(T):
            if 0 <= fold[p] < j:
                m[j][p] = unit.sre_of(n0 + p)
        c = min(C, T - t0)
        for t in range(t0, t0 + c):
            unit.hist_k.append([float(x) for x in k[t]])
            unit.hist_v.append([float(x) for x in v[t]])
        before = set(unit.folded)
        unit.update(n0 + t0, c)
        for p in set(unit.folded) - before:
            if p >= n0:
                fold[p - n0] = j
    return m, fold
