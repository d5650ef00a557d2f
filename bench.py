#!/usr/bin/env python3
"""Benchmark of the LoLA attention step for one layer on one MI355X.

A step is one lola_prefill_chunk call over the whole workload (every chunk,
every stage: phi, the SRE/top-lambda/fold chain, chunk attention with the
linear read, state write-back) from an empty state, inputs resident in HBM.
Default workload: the Llama-3-8B-shaped layer (B = 1, 32 q / 8 KV heads,
d = 128, T = 4096, eta = lambda = 256, C = 64).  The same run also times the
decode workload (64 sequences, state from a 4096-token prefill, decode steps
of fresh tokens) and the float64 CPU oracle on the host.

Prints one JSON line (see the keys below).  --gpus N with N > 1 is refused:
this build runs on a single GPU.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


# ---------------------------------------------------------------- work model
def prefill_work(wl):
    """Algorithmic flops of one prefill call from an empty state, by kernel.

    Each contraction counted once (2 M N K): attention q.k and p.v over the
    keys each query actually sees (cache, window, causal prefix), the linear
    read phi(q)^T [H | s], phi = x W for every q row and k row, SRE
    phi(k)^T [H | s] for every scored candidate, and the fold phi(k) v^T for
    every folded token.  Exponentials, selection and the split-precision
    extra passes are not counted."""
    d, D, m, g, U = wl.d, wl.D, wl.m, wl.g, wl.units
    attn = lin = sre = fold = 0
    n = 0
    gs = 0
    for t0 in range(0, wl.T, wl.C):
        c = min(wl.C, wl.T - t0)
        lo = max(0, n - wl.eta)
        keys = sum(gs + (t - lo + 1) for t in range(n, n + c))   # visible keys, summed
        attn += 4 * d * keys * g
        lin += c * g * 2 * D * (d + 1)
        nL = max(0, n + c - wl.eta) - lo
        nE = gs + nL
        if nE > wl.lam:
            sre += nE * 2 * D * (d + 1)
            fold += (nE - wl.lam) * 2 * D * (d + 1)
            gs = wl.lam
        else:
            gs = nE
        n += c
    phi_q = wl.T * g * 2 * d * m
    phi_k = wl.T * 2 * d * m
    per_unit = dict(phi=phi_k, chain=sre + fold, attn=attn + lin + phi_q, finalize=0)
    return {k: v * U for k, v in per_unit.items()}


def decode_bytes_per_step(wl):
    """Algorithmic HBM bytes of one decode step (steady state, one fold per
    unit): read H, s, window and cache K/V, cache positions, q/k/v and W;
    write H, s, the output, one ring slot and one cache slot."""
    d, D, g, U, esz = wl.d, wl.D, wl.g, wl.units, 2
    rd = D * d * 4 + D * 4 + 2 * wl.eta * d * esz + 2 * wl.lam * d * esz + wl.lam * 4 \
        + g * d * esz + 2 * d * esz + (wl.Hkv * d * wl.m * esz) // wl.B
    wr = D * d * 4 + D * 4 + g * d * 4 + 2 * d * esz + 2 * d * esz + 4
    return (rd + wr) * U


def kernel_source_hash(name):
    p = os.path.join(ROOT, "sparse_kv_caching_amd", "csrc", name)
    h = hashlib.sha256()
    for f in (name, "common.h", "internal.h"):
        with open(os.path.join(ROOT, "sparse_kv_caching_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(kernel_file, kernel_name, workload):
    """HBM bytes per launch from a committed counter summary, if it was taken
    on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic_%s_%s.txt" % (kernel_name, workload))
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if "=" in line and not line.startswith("#"):
                k, v = line.strip().split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("src_sha") != kernel_source_hash(kernel_file):
        return None
    try:
        return float(kv["bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ------------------------------------------------------------------ helpers
def to_dev(arr, dtype):
    import numpy as np
    import torch
    arr = np.ascontiguousarray(arr)
    if dtype == "bf16":
        return torch.from_numpy(arr.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(arr).cuda()


def cpu_baseline(wl, budget_s=20.0):
    """Time the float64 oracle (as it stands) on the host: the whole workload
    if one unit-sequence estimate fits the budget, else a leading subset of
    KV heads; scaled to tokens/s."""
    import numpy as np
    from oracle import lola as O
    from sparse_kv_caching_amd.workloads import make_inputs
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    sub = wl.scaled(B=1)
    inp = make_inputs(sub)
    q, k, v, W = inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.f64("W")
    # first: one KV head, to size the sample
    heads = 1
    t = time.perf_counter()
    st = O.new_state(heads, wl.d, wl.D, wl.eta, wl.lam)
    O.prefill(st, q[:, :wl.g], k[:, :1], v[:, :1], W[:1], wl.C)
    one = time.perf_counter() - t
    heads = int(max(1, min(wl.Hkv, budget_s // max(one, 1e-3))))
    # the sample (repeated until about half the budget has passed when one
    # run is short, so the timing is not a fraction of a second)
    reps, el = 0, 0.0
    while reps == 0 or el < 0.5 * budget_s:
        t = time.perf_counter()
        st = O.new_state(heads, wl.d, wl.D, wl.eta, wl.lam)
        O.prefill(st, q[:, :wl.g * heads], k[:, :heads], v[:, :heads], W[:heads], wl.C)
        el += time.perf_counter() - t
        reps += 1
    # tokens/s of the whole layer: each run did heads/Hkv of one sequence
    value = reps * wl.T * (heads / wl.Hkv) / el
    return dict(value=value, unit="tokens/s", cores=threads, kind="oracle",
                sample="%d of %d KV heads (with their %d q-heads each) of one sequence, "
                       "T=%d, full chunk schedule, %d run(s); %.1f s" % (heads, wl.Hkv, wl.g, wl.T,
                                                                       reps, el))


# -------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama8b_4k")
    ap.add_argument("--decode-steps", type=int, default=1024)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the LoLA step of one layer shards by "
              "(sequence, KV head) units with no communication; --gpus %d is not "
              "supported by this build" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_kv_caching_amd.lola import LolaLayer
    from sparse_kv_caching_amd.workloads import WORKLOADS, make_inputs

    torch.cuda.set_device(0)
    wl = WORKLOADS[args.workload]
    print("[bench] workload %s: generating inputs" % wl.name, file=sys.stderr, flush=True)
    inp = make_inputs(wl)
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    q, k, v = to_dev(inp.q, wl.dtype), to_dev(inp.k, wl.dtype), to_dev(inp.v, wl.dtype)
    layer = LolaLayer(batch=wl.B, q_heads=wl.Hq, kv_heads=wl.Hkv, head_dim=wl.d, window=wl.eta,
                      cache=wl.lam, W=to_dev(inp.W, wl.dtype), dtype=tdt)
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    ws = torch.empty(layer.workspace_bytes(wl.T, wl.C), dtype=torch.uint8, device="cuda")

    def step():
        layer.reset()
        layer.prefill(q, k, v, wl.C, out=out, ws=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print("[bench] warmup done; timing %d steps" % args.steps, file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    ms_step = el / args.steps * 1e3
    value = wl.B * wl.T / (el / args.steps)

    # per-kernel durations, HIP events on the launch stream (separate pass)
    layer.profile(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    prof = layer.profile(False)
    work = prefill_work(wl)
    kernels = {}
    for name, (ms, cnt) in prof.items():
        if cnt:
            avg = ms / cnt
            kernels[name] = dict(avg_ms=round(avg, 5), launches_per_step=cnt // args.steps,
                                 gflop=round(work.get(name, 0) / 1e9, 3),
                                 tflops=round(work.get(name, 0) / (avg * 1e-3) / 1e12, 2))
    dom = max(kernels, key=lambda n: kernels[n]["avg_ms"] * kernels[n]["launches_per_step"])
    ach = work[dom] / (kernels[dom]["avg_ms"] * 1e-3) / 1e12
    kfile = {"phi": "phi.hip", "chain": "chain.hip", "attn": "attn.hip",
             "finalize": "state.hip"}[dom]
    roofline = dict(bound="mfma", achieved=round(ach, 3), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                    frac=round(ach / PEAK_BF16_TFLOPS, 5), kernel=dom,
                    traffic=read_traffic(kfile, dom, wl.name))
    total_work = sum(work.values())
    result = {
        "metric": "LoLA prefill tokens/s per layer + decode us/token; % MFMA/HBM roofline",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q/k/v, PCG64; bf16)",
        "config": {"workload": wl.name, "B": wl.B, "Hq": wl.Hq, "Hkv": wl.Hkv, "d": wl.d,
                   "D": wl.D, "T": wl.T, "eta": wl.eta, "lam": wl.lam, "C": wl.C},
        "roofline": roofline,
        "end_to_end_mfma_frac": round(total_work / (ms_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 5),
        "kernels": kernels,
    }
    layer.free()
    del q, k, v, out, ws

    # ------------------------------------------------------------ decode
    if not args.no_decode:
        result["decode"] = bench_decode(args.decode_steps)

    # ------------------------------------------------------- CPU oracle
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(result))


def bench_decode(steps):
    """Decode workload: 64 sequences, 32 q / 8 KV heads, state from a
    4096-token prefill (eta = lambda = 64, C = 64), then `steps` decode steps
    of fresh seeded tokens.  Reports us per step (all 64 sequences advance one
    token), tokens/s and the decode kernel's HBM roofline."""
    import torch
    from sparse_kv_caching_amd.lola import LolaLayer
    from sparse_kv_caching_amd.workloads import WORKLOADS, make_inputs
    wl = WORKLOADS["decode_b64"]
    print("[bench] decode: building the prefill state", file=sys.stderr, flush=True)
    inp = make_inputs(wl, with_q=False)
    k, v = to_dev(inp.k, "bf16"), to_dev(inp.v, "bf16")
    del inp.k, inp.v
    layer = LolaLayer(batch=wl.B, q_heads=wl.Hq, kv_heads=wl.Hkv, head_dim=wl.d, window=wl.eta,
                      cache=wl.lam, W=to_dev(inp.W, "bf16"), dtype=torch.bfloat16)
    # the state does not depend on q: the prefill's queries are zeros
    q0 = torch.zeros((wl.B, wl.Hq, wl.T, wl.d), dtype=torch.bfloat16, device="cuda")
    layer.prefill(q0, k, v, wl.C)
    torch.cuda.synchronize()
    del q0, k, v
    snap = layer.export()
    gen = torch.Generator(device="cuda").manual_seed(wl.seed)
    nw = 16
    total = steps + nw
    qs = torch.randn((total, wl.B, wl.Hq, wl.d), generator=gen, device="cuda").to(torch.bfloat16)
    ks = torch.randn((total, wl.B, wl.Hkv, wl.d), generator=gen, device="cuda").to(torch.bfloat16)
    vs = torch.randn((total, wl.B, wl.Hkv, wl.d), generator=gen, device="cuda").to(torch.bfloat16)
    out = torch.empty((wl.B, wl.Hq, wl.d), dtype=torch.float32, device="cuda")

    def run(i0, i1):
        for i in range(i0, i1):
            layer.decode(qs[i], ks[i], vs[i], out=out)

    run(0, nw)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(nw, total)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    us = el / steps * 1e6
    layer.import_(snap)
    layer.profile(True)
    run(nw, total)
    torch.cuda.synchronize()
    ms, cnt = layer.profile(False)["decode"]
    avg_us = ms / cnt * 1e3
    b = decode_bytes_per_step(wl)
    gbs = b / (avg_us * 1e-6) / 1e9
    # cold variant: the 67 MB state fits the 256 MB Infinity Cache, so the
    # steady state above may be served partly from it; here 1 GiB is read
    # between steps (outside the decode launches' event brackets), so every
    # step reads the state from HBM.  (A read, not a write: written lines
    # would still be dirty in the caches and their write-back would be
    # charged to the decode step.)
    layer.import_(snap)
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    sink = torch.zeros((), dtype=torch.float32, device="cuda")
    n_cold = min(64, steps)
    layer.profile(True)
    for i in range(nw, nw + n_cold):
        torch.sum(flush, dim=0, out=sink)
        layer.decode(qs[i], ks[i], vs[i], out=out)
    torch.cuda.synchronize()
    ms_c, cnt_c = layer.profile(False)["decode"]
    cold_us = ms_c / cnt_c * 1e3
    cold_gbs = b / (cold_us * 1e-6) / 1e9
    del flush
    layer.free()
    return dict(workload=wl.name, B=wl.B, Hq=wl.Hq, Hkv=wl.Hkv, d=wl.d, eta=wl.eta, lam=wl.lam,
                prefill_T=wl.T, steps=steps, us_per_step=round(us, 3),
                us_per_token=round(us, 3), tokens_per_s=round(wl.B / (us * 1e-6), 1),
                kernel_avg_us=round(avg_us, 3),
                roofline=dict(bound="hbm", achieved=round(gbs, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                              frac=round(gbs / PEAK_HBM_GBS, 4), bytes_per_step=b,
                              traffic=read_traffic("decode.hip", "decode", wl.name)),
                cold=dict(steps=n_cold, kernel_avg_us=round(cold_us, 3),
                          achieved=round(cold_gbs, 1), frac=round(cold_gbs / PEAK_HBM_GBS, 4),
                          flush_bytes_read_between_steps=1 << 30))


if __name__ == "__main__":
    main()
