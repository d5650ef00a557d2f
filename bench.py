#!/usr/bin/env python3
"""Benchmark of the LoLA attention step for one layer on one MI355X.

A prefill step is one lola_prefill_chunk call over a whole workload (every
chunk, every stage: phi, the SRE/top-lambda/fold chain, chunk attention with
the linear read, state write-back) from an empty state, inputs resident in
HBM.  The headline line is the largest single-GPU prefill workload by work:
the long-context layer (B = 1, 32 q / 8 KV heads, d = 128, T = 32768,
eta = 256, lambda = 2048, C = 256).  The same run times the batched
(B = 8, T = 8192, eta = lambda = 512, C = 128) and Llama-shaped (B = 1,
T = 4096, eta = lambda = 256, C = 64) prefills, the decode workload (64
sequences, state from a 4096-token prefill, then decode steps of fresh
tokens, warm and after a cache-evicting read), and the float64 CPU oracle on
the host.

Prints one JSON line.  --gpus N with N > 1 is refused: this build runs on a
single GPU.
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
HEADLINE = "long_32k"
EXTRA = ("batched_8k", "llama8b_4k")


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


# ---------------------------------------------------------------- work model
def prefill_work(wl):
    """Algorithmic flops of one prefill call from an empty state, by kernel.

    Each contraction counted once (2 M N K): attention q.k and p.v over the
    keys each query actually sees (cache, window, causal prefix), the linear
    read phi(q)^T [H | s] on chunks whose state holds folded pairs, phi = x W
    for every q row and k row, SRE phi(k)^T [H | s] for every scored
    candidate, and the fold phi(k) v^T for every folded token.  Exponentials,
    selection and the split-precision extra passes are not counted."""
    d, D, m, g, U = wl.d, wl.D, wl.m, wl.g, wl.units
    attn = lin = sre = fold = 0
    n = 0
    gs = 0
    nfold = 0
    for t0 in range(0, wl.T, wl.C):
        c = min(wl.C, wl.T - t0)
        lo = max(0, n - wl.eta)
        keys = sum(gs + (t - lo + 1) for t in range(n, n + c))   # visible keys, summed
        attn += 4 * d * keys * g
        if nfold > 0:
            lin += c * g * 2 * D * (d + 1)
        nL = max(0, n + c - wl.eta) - lo
        nE = gs + nL
        if nE > wl.lam:
            sre += nE * 2 * D * (d + 1)
            fold += (nE - wl.lam) * 2 * D * (d + 1)
            nfold += nE - wl.lam
            gs = wl.lam
        else:
            gs = nE
        n += c
    phi_q = wl.T * g * 2 * d * m
    phi_k = wl.T * 2 * d * m
    # (the concurrent schedule runs the chain and the read in one launch)
    per_unit = dict(phi=phi_k, chain=sre + fold, attn=attn + lin + phi_q, finalize=0,
                    overlap=sre + fold + attn + lin + phi_q)
    return {k: v * U for k, v in per_unit.items()}


def decode_bytes_per_step(wl):
    """Algorithmic HBM bytes of one decode step (steady state, one fold per
    unit), as the state's storage precision defines them: read H, s, window
    and cache K/V, cache positions, q/k/v and W (amortised over the units);
    write H, s, the output, one ring slot and one cache slot (with its
    position)."""
    d, D, g, U, esz = wl.d, wl.D, wl.g, wl.units, 2
    rd = D * d * 4 + D * 4 + 2 * wl.eta * d * esz + 2 * wl.lam * d * esz + wl.lam * 4 \
        + (g + 2) * d * esz + (wl.Hkv * d * wl.m * esz) // wl.B // wl.Hkv
    wr = D * d * 4 + D * 4 + g * d * 4 + 2 * d * esz + 2 * d * esz + 4
    return (rd + wr) * U


def kernel_source_hash(name):
    from sparse_kv_caching_amd.traffic import kernel_source_hash as ksh
    return ksh(name)


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


KFILE = {"phi": "phi.hip", "chain": "chain.hip", "attn": "attn.hip", "finalize": "state.hip",
         "overlap": "fused.hip",
         "decode": "decode.hip"}


# ------------------------------------------------------------------ helpers
def to_dev(arr, dtype):
    import numpy as np
    import torch
    arr = np.ascontiguousarray(arr)
    if dtype == "bf16":
        return torch.from_numpy(arr.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(arr).cuda()


def blas_info():
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            i = info[0]
            return dict(library=i.get("internal_api"), version=i.get("version"),
                        threads=i.get("num_threads"), arch=i.get("architecture"))
    except Exception:
        pass
    return dict(library="unknown", threads=len(os.sched_getaffinity(0)))


def cpu_baseline(wl, budget_s=12.0, threads=None):
    """Time the float64 oracle (as it stands) on the host: a leading subset of
    KV heads of the first sequence, sized to the budget and repeated until
    about half of it has passed; scaled to tokens/s of the whole layer."""
    from oracle import lola as O
    from sparse_kv_caching_amd.workloads import make_inputs
    ctx = None
    if threads is not None:
        from threadpoolctl import threadpool_limits
        ctx = threadpool_limits(limits=threads, user_api="blas")
    try:
        sub = wl.scaled(B=1)
        inp = make_inputs(sub)
        q, k, v, W = inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.f64("W")
        t = time.perf_counter()
        st = O.new_state(1, wl.d, wl.D, wl.eta, wl.lam)
        O.prefill(st, q[:, :wl.g], k[:, :1], v[:, :1], W[:1], wl.C)
        one = time.perf_counter() - t
        heads = int(max(1, min(wl.Hkv, budget_s // max(one, 1e-3))))
        reps, el = 0, 0.0
        while reps == 0 or el < 0.5 * budget_s:
            t = time.perf_counter()
            st = O.new_state(heads, wl.d, wl.D, wl.eta, wl.lam)
            O.prefill(st, q[:, :wl.g * heads], k[:, :heads], v[:, :heads], W[:heads], wl.C)
            el += time.perf_counter() - t
            reps += 1
        value = reps * wl.T * (heads / wl.Hkv) / el
        used = threads if threads is not None else blas_info().get("threads")
        return dict(value=round(value, 1), unit="tokens/s", cores=used, kind="oracle",
                    sample="%d of %d KV heads (with their %d q-heads each) of one sequence, "
                           "T=%d, full chunk schedule, %d run(s) in %.1f s; scaled to the "
                           "workload's B*T tokens" % (heads, wl.Hkv, wl.g, wl.T, reps, el))
    finally:
        if ctx is not None:
            ctx.unregister()


# ------------------------------------------------------------------ prefill
def bench_prefill(wl, steps, warmup):
    """Time `steps` prefill calls of workload wl; per-kernel event timing in
    a second pass.  Returns the measurement dict."""
    import torch
    from sparse_kv_caching_amd.lola import LolaLayer
    from sparse_kv_caching_amd.workloads import make_inputs

    log("workload %s: generating inputs" % wl.name)
    inp = make_inputs(wl)
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    q, k, v = to_dev(inp.q, wl.dtype), to_dev(inp.k, wl.dtype), to_dev(inp.v, wl.dtype)
    layer = LolaLayer(batch=wl.B, q_heads=wl.Hq, kv_heads=wl.Hkv, head_dim=wl.d, window=wl.eta,
                      cache=wl.lam, W=to_dev(inp.W, wl.dtype), dtype=tdt)
    del inp
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    ws = torch.empty(layer.workspace_bytes(wl.T, wl.C), dtype=torch.uint8, device="cuda")

    def step():
        layer.reset()
        layer.prefill(q, k, v, wl.C, out=out, ws=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    layer.check()
    log("%s: timing %d steps" % (wl.name, steps))
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    ms_step = el / steps * 1e3
    value = wl.B * wl.T / (el / steps)

    # per-kernel durations: HIP events on the launch stream around each
    # launch (a separate pass; the kernels here last tens of us to ms)
    layer.profile(True)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    prof = layer.profile(False)
    layer.check()
    work = prefill_work(wl)
    kernels = {}
    for name, (ms, cnt) in prof.items():
        if cnt:
            avg = ms / cnt
            kernels[name] = dict(avg_ms=round(avg, 5), launches_per_step=cnt // steps,
                                 gflop=round(work.get(name, 0) / 1e9, 3),
                                 tflops=round(work.get(name, 0) / (avg * 1e-3) / 1e12, 2),
                                 frac=round(work.get(name, 0) / (avg * 1e-3) / 1e12
                                            / PEAK_BF16_TFLOPS, 5))
    dom = max(kernels, key=lambda n: kernels[n]["avg_ms"] * kernels[n]["launches_per_step"])
    ach = work[dom] / (kernels[dom]["avg_ms"] * 1e-3) / 1e12
    roofline = dict(bound="mfma", achieved=round(ach, 3), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                    frac=round(ach / PEAK_BF16_TFLOPS, 5), kernel=dom,
                    traffic=read_traffic(KFILE[dom], dom, wl.name))
    total = sum(v for k, v in work.items() if k != "overlap")
    layer.free()
    del q, k, v, out, ws
    torch.cuda.empty_cache()
    return dict(value=round(value, 1), unit="tokens/s", ms_per_step=round(ms_step, 4),
                config={"workload": wl.name, "B": wl.B, "Hq": wl.Hq, "Hkv": wl.Hkv, "d": wl.d,
                        "D": wl.D, "T": wl.T, "eta": wl.eta, "lam": wl.lam, "C": wl.C},
                roofline=roofline, kernels=kernels,
                gflop_per_step=round(total / 1e9, 2),
                end_to_end_mfma_frac=round(total / (ms_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 5))


# ------------------------------------------------------------------- decode
def bench_decode(steps):
    """Decode workload: 64 sequences, 32 q / 8 KV heads, state from a
    4096-token prefill (eta = lambda = 64, C = 64), then `steps` decode steps
    of fresh seeded tokens.

    Warm: one event pair around `steps` back-to-back launches (no per-launch
    brackets).  Cold: 1 GiB is read between steps (outside the decode's
    events), so the state (67 MB, which fits the 256 MB Infinity Cache) comes
    from HBM; each cold step is bracketed by its own event pair, whose
    overhead is measured on warm steps bracketed the same way and taken off.
    The HBM claim is the cold one."""
    import torch
    from sparse_kv_caching_amd.lola import LolaLayer
    from sparse_kv_caching_amd.workloads import WORKLOADS, make_inputs
    wl = WORKLOADS["decode_b64"]
    log("decode: building the prefill state")
    inp = make_inputs(wl, with_q=False)
    k, v = to_dev(inp.k, "bf16"), to_dev(inp.v, "bf16")
    layer = LolaLayer(batch=wl.B, q_heads=wl.Hq, kv_heads=wl.Hkv, head_dim=wl.d, window=wl.eta,
                      cache=wl.lam, W=to_dev(inp.W, "bf16"), dtype=torch.bfloat16)
    del inp
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
    log("decode: timing %d steps" % steps)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    run(nw, total)
    e1.record()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    us = el / steps * 1e6
    warm_us = e0.elapsed_time(e1) * 1e3 / steps          # one event pair around the launches
    # per-launch brackets on warm steps (their overhead, for the cold steps)
    layer.import_(snap)
    layer.profile(True)
    run(nw, total)
    torch.cuda.synchronize()
    ms_b, cnt_b = layer.profile(False)["decode"]
    bracket_us = ms_b / cnt_b * 1e3
    overhead = max(0.0, bracket_us - warm_us)
    layer.import_(snap)
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    sink = torch.zeros((), dtype=torch.float32, device="cuda")
    n_cold = min(128, steps)
    layer.profile(True)
    for i in range(nw, nw + n_cold):
        torch.sum(flush, dim=0, out=sink)
        layer.decode(qs[i], ks[i], vs[i], out=out)
    torch.cuda.synchronize()
    ms_c, cnt_c = layer.profile(False)["decode"]
    cold_bracket_us = ms_c / cnt_c * 1e3
    cold_us = cold_bracket_us - overhead
    layer.check()
    del flush
    layer.free()
    b_alg = decode_bytes_per_step(wl)
    b_meas = read_traffic("decode.hip", "decode", wl.name)

    def rate(b, t_us):
        return None if b is None else round(b / (t_us * 1e-6) / 1e9, 1)

    cold_alg = rate(b_alg, cold_us)
    return dict(workload=wl.name, B=wl.B, Hq=wl.Hq, Hkv=wl.Hkv, d=wl.d, eta=wl.eta, lam=wl.lam,
                prefill_T=wl.T, steps=steps, us_per_step=round(us, 3),
                us_per_token=round(us, 3), tokens_per_s=round(wl.B / (us * 1e-6), 1),
                warm_kernel_us=round(warm_us, 3),
                roofline=dict(bound="hbm", achieved=cold_alg, peak=PEAK_HBM_GBS, unit="GB/s",
                              frac=round(cold_alg / PEAK_HBM_GBS, 4), kernel="decode",
                              variant="cold: 1 GiB read between steps",
                              kernel_us=round(cold_us, 3), bytes_per_step=b_alg,
                              bytes_counted="algorithmic: state at storage precision, H and s "
                                            "read and written every step",
                              traffic=b_meas,
                              achieved_on_traffic=rate(b_meas, cold_us)),
                warm=dict(kernel_us=round(warm_us, 3), achieved=rate(b_alg, warm_us),
                          frac=round(rate(b_alg, warm_us) / PEAK_HBM_GBS, 4),
                          achieved_on_traffic=rate(b_meas, warm_us)),
                cold=dict(steps=n_cold, kernel_us=round(cold_us, 3),
                          bracketed_us=round(cold_bracket_us, 3),
                          bracket_overhead_us=round(overhead, 3),
                          flush_bytes_read_between_steps=1 << 30))


# -------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--extra", default=",".join(EXTRA),
                    help="comma-separated further prefill workloads ('' for none)")
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
    from sparse_kv_caching_amd.workloads import WORKLOADS

    torch.cuda.set_device(0)
    head = bench_prefill(WORKLOADS[args.workload], args.steps, args.warmup)
    result = {
        "metric": "LoLA prefill tokens/s per layer + decode us/token; % MFMA/HBM roofline",
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q/k/v, PCG64, planted repeated keys; bf16)",
        "config": head["config"],
        "roofline": head["roofline"],
        "end_to_end_mfma_frac": head["end_to_end_mfma_frac"],
        "gflop_per_step": head["gflop_per_step"],
        "kernels": head["kernels"],
    }
    extra = [w for w in args.extra.split(",") if w]
    result["prefill_configs"] = {}
    for name in extra:
        result["prefill_configs"][name] = bench_prefill(WORKLOADS[name], args.steps, args.warmup)
    if not args.no_decode:
        result["decode"] = bench_decode(args.decode_steps)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        result["cpu_baseline"] = cpu_baseline(WORKLOADS[args.workload])
        for name in extra:
            result["prefill_configs"][name]["cpu_baseline"] = cpu_baseline(WORKLOADS[name])
        result["cpu_single_thread"] = {
            name: cpu_baseline(WORKLOADS[name], budget_s=8.0, threads=1)
            for name in ("tiny_fp32", "llama8b_4k")}
        result["cpu_blas"] = blas_info()
    print(json.dumps(result))


if __name__ == "__main__":
    main()
