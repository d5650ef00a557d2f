"""Seeded synthetic inputs for the LoLA attention step.

This module holds no part of the method's arithmetic: it only draws random
numbers, rounds them to the storage dtype and plants repeated keys.  Both the
HIP path (through tests and the benchmark) and the CPU oracle receive the
arrays it returns, bit for bit.

Recipe:

* ``numpy.random.default_rng(seed)`` (PCG64) draws q, k, v ~ N(0, 1) in float32,
  in that order, shapes q (B, Hq, T, d), k and v (B, Hkv, T, d).  bf16
  workloads round them to bf16 with round-to-nearest-even.
* The feature-map weights W (Hkv, d, m) ~ N(0, 1/d) come from
  ``default_rng(seed + 100)`` and are rounded to the same dtype.
* Planted pairs stand in for needle-in-a-haystack probes: for N planted pairs
  the last N positions' queries copy an earlier key of the same KV head,
  q[b, j, T - N + i] = k[b, floor(j / g), p_i] for every q-head j.  The planted
  positions lie in [0, P) with P = floor((T - N) / C) * C - eta, so they have
  left the window by the time they are probed.  ``plant="random"`` draws them
  without replacement (per sequence) from the same generator after v;
  ``plant="uniform"`` takes p_i = floor((i + 1/2) P / N).
* Decode steps draw fresh q (B, Hq, d), k, v (B, Hkv, d) from
  ``default_rng([seed, 1_000_000 + step])``.
* Parity stress inputs (``keys`` other than "iid"; the workloads above are
  all "iid") replace k and v: the centres or pairs come from
  ``default_rng([seed, 7])``, each token's choice and noise from
  ``default_rng([seed, 8])``:
  "clustered": per (sequence, KV head) 16 centres c_j ~ N(0, 1) and 16 value
  rows m_j ~ N(0, 1); token t takes a uniform cluster z_t and
  k_t = c_{z_t} + 0.1 n_t, v_t = m_{z_t} + 0.1 n'_t (n, n' ~ N(0, 1)), so the
  values are predictable from the keys;
  "pool": per (sequence, KV head) 6 pairs (k, v) ~ N(0, 1), and token t takes
  pair p_t uniform in 0..5: exact duplicate pairs, so candidates tie exactly.
  Decode steps of these workloads draw their k, v the same way, the choice
  and noise from ``default_rng([seed, 2_000_000 + step])``.
"""

from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Dict, Optional

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    m: int            # features per half; D = 2m
    T: int
    eta: int
    lam: int
    C: int
    dtype: str        # "bf16" or "f32"
    seed: int
    planted: int = 0
    plant: str = "none"
    decode_steps: int = 0
    keys: str = "iid"     # "iid", or the stress structures "clustered", "pool"

    @property
    def D(self) -> int:
        return 2 * self.m

    @property
    def g(self) -> int:
        return self.Hq // self.Hkv

    @property
    def units(self) -> int:
        return self.B * self.Hkv

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    # 1 head, head dim 64, fp32, 8 planted pairs
    "tiny_fp32": Workload("tiny_fp32", 1, 1, 1, 64, 64, 512, 64, 64, 64, "f32", 0, 8, "random"),
    # Llama-3-8B-shaped layer: 32 q heads / 8 KV heads, head dim 128
    "llama8b_4k": Workload("llama8b_4k", 1, 32, 8, 128, 64, 4096, 256, 256, 64, "bf16", 1),
    # batch 8, T = 8192, 32 planted pairs per sequence
    "batched_8k": Workload("batched_8k", 8, 32, 8, 128, 64, 8192, 512, 512, 128, "bf16", 2, 32,
                           "random"),
    # decode: state from a 4096-token prefill (C = eta = 64), then 1024 steps
    "decode_b64": Workload("decode_b64", 64, 32, 8, 128, 64, 4096, 64, 64, 64, "bf16", 3,
                           decode_steps=1024),
    # long context: T = 32768, lam = 2048, 64 planted pairs spread uniformly
    "long_32k": Workload("long_32k", 1, 32, 8, 128, 64, 32768, 256, 2048, 256, "bf16", 4, 64,
                         "uniform"),
}


# ----------------------------------------------------------------- rounding
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns the
    16-bit patterns as uint16."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Inputs:
    """Arrays in storage form plus exact float64 views for the oracle.

    ``q``, ``k``, ``v``, ``W`` are uint16 bf16 patterns (bf16 workloads) or
    float32; ``*_f64`` are their exact float64 values."""

    wl: Workload
    q: Optional[np.ndarray]
    k: np.ndarray
    v: np.ndarray
    W: np.ndarray
    planted_pos: np.ndarray        # (B, N) int64

    def f64(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        if a is None:
            return None
        if self.wl.dtype == "bf16":
            return bf16_to_f32(a).astype(np.float64)
        return a.astype(np.float64)


def _store(wl: Workload, x: np.ndarray) -> np.ndarray:
    return bf16_bits(x) if wl.dtype == "bf16" else np.ascontiguousarray(x, np.float32)


def planted_positions(wl: Workload, rng: Optional[np.random.Generator]) -> np.ndarray:
    N = wl.planted
    if N == 0:
        return np.zeros((wl.B, 0), np.int64)
    P = ((wl.T - N) // wl.C) * wl.C - wl.eta
    if P < N:
        raise ValueError("workload too short to plant %d pairs" % N)
    if wl.plant == "uniform":
        p = np.floor((np.arange(N) + 0.5) * P / N).astype(np.int64)
        return np.broadcast_to(p, (wl.B, N)).copy()
    return np.stack([np.sort(rng.choice(P, size=N, replace=False)) for _ in range(wl.B)]
                    ).astype(np.int64)


def _structure(wl: Workload):
    """Centres (or pairs) of a stress structure: (Hk, Hv), each (B, Hkv, n, d)."""
    rng = np.random.default_rng([wl.seed, 7])
    n = 16 if wl.keys == "clustered" else 6
    return (rng.standard_normal((wl.B, wl.Hkv, n, wl.d), dtype=np.float32),
            rng.standard_normal((wl.B, wl.Hkv, n, wl.d), dtype=np.float32))


def _structured_kv(wl: Workload, rng: np.random.Generator, T: int):
    """k, v (B, Hkv, T, d) float32 of a stress structure."""
    ck, cv = _structure(wl)
    n = ck.shape[2]
    z = rng.integers(0, n, size=(wl.B, wl.Hkv, T))
    bi = np.arange(wl.B)[:, None, None]
    hi = np.arange(wl.Hkv)[None, :, None]
    k, v = ck[bi, hi, z], cv[bi, hi, z]
    if wl.keys == "clustered":
        k = k + np.float32(0.1) * rng.standard_normal(k.shape, dtype=np.float32)
        v = v + np.float32(0.1) * rng.standard_normal(v.shape, dtype=np.float32)
    elif wl.keys != "pool":
        raise ValueError("unknown key structure %r" % wl.keys)
    return np.ascontiguousarray(k), np.ascontiguousarray(v)


def make_inputs(wl: Workload, with_q: bool = True) -> Inputs:
    """Draw the prefill inputs of a workload (see the module docstring).

    ``with_q=False`` skips storing q (the state trajectory does not read it);
    the generator still draws it so k and v stay the same."""
    rng = np.random.default_rng(wl.seed)
    q = rng.standard_normal((wl.B, wl.Hq, wl.T, wl.d), dtype=np.float32)
    k = rng.standard_normal((wl.B, wl.Hkv, wl.T, wl.d), dtype=np.float32)
    v = rng.standard_normal((wl.B, wl.Hkv, wl.T, wl.d), dtype=np.float32)
    pp = planted_positions(wl, rng)
    W = np.random.default_rng(wl.seed + 100).standard_normal(
        (wl.Hkv, wl.d, wl.m), dtype=np.float32) * np.float32(1.0 / np.sqrt(wl.d))
    if wl.keys != "iid":
        k, v = _structured_kv(wl, np.random.default_rng([wl.seed, 8]), wl.T)
    ks = _store(wl, k)
    del k
    vs = _store(wl, v)
    del v
    qs = None
    if with_q:
        qs = _store(wl, q)
        N, g = wl.planted, wl.g
        for b in range(wl.B):
            for i in range(N):
                for h in range(wl.Hkv):
                    qs[b, h * g:(h + 1) * g, wl.T - N + i] = ks[b, h, pp[b, i]]
    del q
    return Inputs(wl, qs, ks, vs, _store(wl, W), pp)


def decode_inputs(wl: Workload, step: int):
    """Fresh (q, k, v) for decode step ``step``: q (B, Hq, d), k, v (B, Hkv, d),
    in storage form."""
    rng = np.random.default_rng([wl.seed, 1_000_000 + step])
    q = rng.standard_normal((wl.B, wl.Hq, wl.d), dtype=np.float32)
    k = rng.standard_normal((wl.B, wl.Hkv, wl.d), dtype=np.float32)
    v = rng.standard_normal((wl.B, wl.Hkv, wl.d), dtype=np.float32)
    if wl.keys != "iid":
        k, v = _structured_kv(wl, np.random.default_rng([wl.seed, 2_000_000 + step]), 1)
        k, v = k[:, :, 0], v[:, :, 0]
    return _store(wl, q), _store(wl, k), _store(wl, v)


def to_f64(wl: Workload, a: np.ndarray) -> np.ndarray:
    """Exact float64 value of a storage-form array."""
    if wl.dtype == "bf16":
        return bf16_to_f32(a).astype(np.float64)
    return np.asarray(a, np.float64)
