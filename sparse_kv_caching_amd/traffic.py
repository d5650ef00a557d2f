"""HBM traffic of the library's kernels from rocprofv3 counters.

Two modes:

``run``       executes one workload's kernels for counter collection (run it
              under ``rocprofv3 --pmc FETCH_SIZE`` and again under
              ``--pmc WRITE_SIZE``, one counter per run):

                python3 -m sparse_kv_caching_amd.traffic run --workload llama8b_4k
                python3 -m sparse_kv_caching_amd.traffic run --workload decode_b64

              A prefill workload runs two prefill calls (the second is the one
              measured); the decode workload runs its 4096-token prefill and
              then decode steps.  Both end with an elementwise copy of
              256 MiB (``torch.neg`` into a preallocated tensor), whose
              counters calibrate the scale: bytes = counter * 1024 * factor
              with factor = copy bytes / (copy counter * 1024).

``counters``  prints one kernel's SQ / TCC counters (any number of
              ``--pmc`` folders of the same run command) with per-wave and
              per-cycle ratios.

``summarize`` reads the two rocprofv3 output folders and writes
              ``profiles/traffic_<kernel>_<workload>.txt`` with the measured
              bytes per launch (the average over the measured launches), the
              calibration factors, the algorithmic bytes where they are
              defined, and the hash of the kernel's sources (``bench.py``
              only uses a summary whose hash matches the current sources).
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_kv_caching_amd", "csrc")
COPY_BYTES = 256 << 20

# kernel -> (source file, symbol prefix in the rocprofv3 kernel name)
KERNELS = {
    "phi": ("phi.hip", "lola::phi_kernel"),
    "chain": ("chain.hip", "lola::chain_kernel"),
    "attn": ("attn.hip", "lola::attn_kernel"),
    "decode": ("decode.hip", "lola::decode_kernel"),
    "overlap": ("fused.hip", "lola::overlap_kernel"),
}


def kernel_source_hash(fname: str) -> str:
    """Hash of a kernel's sources: its file, the bodies it includes
    (``*_impl.h``: both for the fused chain + attention kernel) and the shared
    headers."""
    files = [fname]
    if fname == "fused.hip":
        files += ["chain_impl.h", "attn_impl.h"]
    else:
        impl = fname.replace(".hip", "_impl.h")
        if os.path.exists(os.path.join(CSRC, impl)):
            files.append(impl)
    h = hashlib.sha256()
    for f in files + ["common.h", "internal.h"]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# ------------------------------------------------------------------- run
def _run(args):
    import numpy as np
    import torch

    sys.path.insert(0, ROOT)
    from sparse_kv_caching_amd.lola import LolaLayer
    from sparse_kv_caching_amd.workloads import WORKLOADS, make_inputs

    def to_dev(arr):
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).cuda().view(torch.bfloat16)

    torch.cuda.set_device(0)
    wl = WORKLOADS[args.workload]
    print("[traffic] %s" % wl.name, flush=True)
    if wl.decode_steps:
        inp = make_inputs(wl, with_q=False)
        layer = LolaLayer(batch=wl.B, q_heads=wl.Hq, kv_heads=wl.Hkv, head_dim=wl.d,
                          window=wl.eta, cache=wl.lam, W=to_dev(inp.W), dtype=torch.bfloat16)
        q0 = torch.zeros((wl.B, wl.Hq, wl.T, wl.d), dtype=torch.bfloat16, device="cuda")
        layer.prefill(q0, to_dev(inp.k), to_dev(inp.v), wl.C)
        gen = torch.Generator(device="cuda").manual_seed(wl.seed)
        out = torch.empty((wl.B, wl.Hq, wl.d), dtype=torch.float32, device="cuda")
        for _ in range(args.steps):
            q = torch.randn((wl.B, wl.Hq, wl.d), generator=gen, device="cuda").to(torch.bfloat16)
            k = torch.randn((wl.B, wl.Hkv, wl.d), generator=gen, device="cuda").to(torch.bfloat16)
            v = torch.randn((wl.B, wl.Hkv, wl.d), generator=gen, device="cuda").to(torch.bfloat16)
            layer.decode(q, k, v, out=out)
    else:
        inp = make_inputs(wl)
        layer = LolaLayer(batch=wl.B, q_heads=wl.Hq, kv_heads=wl.Hkv, head_dim=wl.d,
                          window=wl.eta, cache=wl.lam, W=to_dev(inp.W), dtype=torch.bfloat16)
        if args.overlap is not None:
            from sparse_kv_caching_amd.lola import DEBUG_OVERLAP
            layer.debug_set(DEBUG_OVERLAP, args.overlap)
        q, k, v = to_dev(inp.q), to_dev(inp.k), to_dev(inp.v)
        for _ in range(2):
            layer.reset()
            layer.prefill(q, k, v, wl.C)
    torch.cuda.synchronize()
    a = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    torch.neg(a, out=b)
    torch.cuda.synchronize()
    layer.free()
    print("[traffic] done", flush=True)


# ------------------------------------------------------------- summarize
def _read_counter(folder: str, counter: str):
    """{kernel name: [value per dispatch in dispatch order]} from a rocprofv3
    counter_collection.csv (values in KiB for FETCH_SIZE / WRITE_SIZE)."""
    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no counter_collection.csv under %s" % folder)
    per = defaultdict(dict)
    for path in files:
        with open(path) as fh:
            for row in csv.DictReader(fh):
                if row.get("Counter_Name") != counter:
                    continue
                did = int(row.get("Dispatch_Id") or row.get("Correlation_Id") or 0)
                name = row.get("Kernel_Name", "")
                per[name][did] = per[name].get(did, 0.0) + float(row["Counter_Value"])
    return {k: [v[i] for i in sorted(v)] for k, v in per.items()}


def _pick(counts, prefix):
    vals = []
    for name, v in counts.items():
        if name.startswith(prefix) or ("%s<" % prefix) in name or prefix in name:
            vals.extend(v)
    return vals


def _summarize(args):
    fetch = _read_counter(args.fetch, "FETCH_SIZE")
    write = _read_counter(args.write, "WRITE_SIZE")
    fname, prefix = KERNELS[args.kernel]
    fv, wv = _pick(fetch, prefix), _pick(write, prefix)
    if not fv or not wv:
        raise SystemExit("kernel %s not found in the counter files" % prefix)
    # measured launches: the last `--last` dispatches of the kernel
    fv, wv = fv[-args.last:], wv[-args.last:]
    cf = [v for k, vs in fetch.items() if "neg" in k.lower() for v in vs]
    cw = [v for k, vs in write.items() if "neg" in k.lower() for v in vs]
    if not cf or not cw:
        raise SystemExit("calibration copy kernel not found")
    f_fac = COPY_BYTES / (cf[-1] * 1024.0)
    w_fac = COPY_BYTES / (cw[-1] * 1024.0)
    fb = sum(fv) / len(fv) * 1024.0 * f_fac
    wb = sum(wv) / len(wv) * 1024.0 * w_fac
    out = os.path.join(ROOT, "profiles", "traffic_%s_%s.txt" % (args.kernel, args.workload))
    sched = "" if args.overlap is None else " --overlap %d" % args.overlap
    with open(out, "w") as fh:
        fh.write("# HBM traffic of %s on the %s workload%s (rocprofv3 PMC, MI355X)\n"
                 % (prefix, args.workload,
                    ", sequential schedule (the kernel launched alone)" if args.overlap == 0 else ""))
        fh.write("# commands (repository root = $REPO, on PYTHONPATH; one counter per run):\n")
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            fh.write("#   cd /tmp && export TMPDIR=/tmp && timeout -s KILL 120 rocprofv3 --pmc %s "
                     "--output-format csv -d $REPO/gpurun_out/<dir> -o run -- python3 -m "
                     "sparse_kv_caching_amd.traffic run --workload %s%s\n" % (c, args.workload, sched))
        fh.write("#   python3 -m sparse_kv_caching_amd.traffic summarize --workload %s --kernel %s "
                 "--fetch <fetch dir> --write <write dir> --last %d\n"
                 % (args.workload, args.kernel, args.last))
        fh.write("# calibration: torch.neg over %d bytes reads %.1f KiB and writes %.1f KiB\n"
                 % (COPY_BYTES, cf[-1], cw[-1]))
        fh.write("kernel = %s\n" % args.kernel)
        fh.write("workload = %s\n" % args.workload)
        fh.write("src_sha = %s\n" % kernel_source_hash(fname))
        fh.write("launches = %d\n" % len(fv))
        fh.write("fetch_kib_per_launch = %.1f\n" % (sum(fv) / len(fv)))
        fh.write("write_kib_per_launch = %.1f\n" % (sum(wv) / len(wv)))
        fh.write("fetch_factor = %.4f\n" % f_fac)
        fh.write("write_factor = %.4f\n" % w_fac)
        fh.write("fetch_bytes_per_launch = %.0f\n" % fb)
        fh.write("write_bytes_per_launch = %.0f\n" % wb)
        fh.write("bytes_per_launch = %.0f\n" % (fb + wb))
        if args.algorithmic:
            fh.write("algorithmic_bytes_per_launch = %d\n" % args.algorithmic)
    print(open(out).read())


def _counters(args):
    """SQ / TCC counters of one kernel (its last `--last` launches, averaged)
    from several rocprofv3 --pmc folders, with per-wave and per-cycle ratios."""
    fname, prefix = KERNELS[args.kernel]
    vals = {}
    for folder in args.dirs:
        files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
        for path in files:
            per = defaultdict(lambda: defaultdict(float))
            with open(path) as fh:
                for row in csv.DictReader(fh):
                    if prefix not in row.get("Kernel_Name", ""):
                        continue
                    did = int(row.get("Dispatch_Id") or row.get("Correlation_Id") or 0)
                    per[row["Counter_Name"]][did] += float(row["Counter_Value"])
            for name, byd in per.items():
                last = [byd[d] for d in sorted(byd)][-args.last:]
                vals[name] = sum(last) / len(last)
    print("[%s, %s, source %s]" % (prefix, args.workload, kernel_source_hash(fname)))
    for k in sorted(vals):
        print("%s = %.6g" % (k, vals[k]))
    w = vals.get("SQ_WAVES")
    if w:
        for k in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_INSTS_VMEM_RD"):
            if k in vals:
                print("per_wave_%s = %.1f" % (k[9:].lower(), vals[k] / w))
    wc = vals.get("SQ_WAVE_CYCLES")
    if wc:
        for k in ("SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU",
                  "SQ_ACTIVE_INST_LDS"):
            if k in vals:
                print("%s_fraction_of_wave_cycles = %.3f" % (k[3:].lower(), vals[k] / wc))
    if "TCC_HIT_sum" in vals and "TCC_MISS_sum" in vals:
        h, m = vals["TCC_HIT_sum"], vals["TCC_MISS_sum"]
        print("l2_hit_rate = %.3f" % (h / max(h + m, 1.0)))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="mode", required=True)
    r = sub.add_parser("run")
    r.add_argument("--workload", required=True)
    r.add_argument("--steps", type=int, default=16)
    r.add_argument("--overlap", type=int, default=None, choices=(-1, 0, 1),
                   help="prefill schedule (LOLA_DEBUG_OVERLAP); default: the library's choice")
    s = sub.add_parser("summarize")
    s.add_argument("--workload", required=True)
    s.add_argument("--kernel", required=True, choices=sorted(KERNELS))
    s.add_argument("--fetch", required=True)
    s.add_argument("--write", required=True)
    s.add_argument("--last", type=int, default=1)
    s.add_argument("--algorithmic", type=int, default=0)
    s.add_argument("--overlap", type=int, default=None,
                   help="the prefill schedule of the runs (recorded in the summary's commands)")
    c = sub.add_parser("counters")
    c.add_argument("--workload", required=True)
    c.add_argument("--kernel", required=True, choices=sorted(KERNELS))
    c.add_argument("--dirs", nargs="+", required=True)
    c.add_argument("--last", type=int, default=1)
    args = ap.parse_args()
    if args.mode == "run":
        _run(args)
    elif args.mode == "counters":
        _counters(args)
    else:
        _summarize(args)


if __name__ == "__main__":
    main()
