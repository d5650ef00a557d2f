"""Per-workload kernel durations from a rocprofv3 kernel trace.

``rocprofv3 --kernel-trace --stats`` aggregates each kernel over the whole
run; ``bench.py`` runs several prefill workloads one after the other, so its
per-kernel statistics mix them.  This splits the trace
(``<dir>/run_kernel_trace.csv``) by workload: every prefill call launches the
φ kernel first, so the φ dispatches, in time order, are cut into consecutive
segments of the given call counts (one per workload, in the order
``bench.py`` runs them), and each dispatch of a prefill kernel (φ, chain,
attention, the chain and read in one launch, finalize) takes the workload of
the segment its start time falls in.  Every other kernel is reported over
the whole run.

    python3 -m sparse_kv_caching_amd.kstats <dir>/run_kernel_trace.csv \
        --segments long_32k:12,batched_8k:12,llama8b_4k:12,decode_b64:1

prints a Markdown table (calls, average / min / max in microseconds).  With
``--last N`` it adds, for the prefill kernels of each segment, the average of
the segment's last N calls (``bench.py`` times its last N calls of a workload
with HIP events, so that column is the one to set beside its figures).
"""

from __future__ import annotations

import argparse
import csv
from collections import defaultdict

PREFILL = ("lola::phi_kernel", "lola::chain_kernel", "lola::attn_kernel",
           "lola::overlap_kernel", "lola::finalize_cache_kernel", "lola::finalize_ring_kernel")


def _family(name: str) -> str:
    for p in PREFILL:
        if p in name:
            return p
    return ""


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("trace")
    ap.add_argument("--segments", required=True,
                    help="workload:calls,... in the order the prefill workloads ran")
    ap.add_argument("--last", type=int, default=0,
                    help="also average each segment's last N calls of a prefill kernel")
    args = ap.parse_args()
    segs = []
    for item in args.segments.split(","):
        w, n = item.split(":")
        segs.append((w, int(n)))
    rows = []
    with open(args.trace) as fh:
        for r in csv.DictReader(fh):
            t0, t1 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
            rows.append((t0, r["Kernel_Name"], (t1 - t0) / 1e3))
    rows.sort()
    # segment start times from the phi dispatches
    phi_t = [t0 for t0, name, _ in rows if "lola::phi_kernel" in name]
    starts, i = [], 0
    for w, n in segs:
        if i >= len(phi_t):
            break
        starts.append((phi_t[i], w))
        i += n
    groups = defaultdict(list)        # (label, kernel name) -> durations
    for t0, name, us in rows:
        label = "whole run"
        if _family(name):
            label = "before the first segment"
            for ts, w in starts:
                if t0 >= ts:
                    label = w
        short = name.split("(")[0].replace("void ", "")
        groups[(label, short)].append(us)
    order = ["before the first segment"] + [w for w, _ in segs] + ["whole run"]
    n = args.last
    if n:
        print("| Workload | Kernel | Calls | Avg (us) | Avg of the last %d (us) | Min (us) | Max (us) |" % n)
        print("|---|---|---|---|---|---|---|")
    else:
        print("| Workload | Kernel | Calls | Avg (us) | Min (us) | Max (us) |")
        print("|---|---|---|---|---|---|")
    for label in order:
        items = sorted(((k, v) for k, v in groups.items() if k[0] == label),
                       key=lambda kv: -sum(kv[1]))
        for (lab, name), v in items:
            if n:
                tail = "%.1f" % (sum(v[-n:]) / len(v[-n:])) if lab in dict(segs) and len(v) >= n else "-"
                print("| %s | `%s` | %d | %.1f | %s | %.1f | %.1f |"
                      % (lab, name, len(v), sum(v) / len(v), tail, min(v), max(v)))
            else:
                print("| %s | `%s` | %d | %.1f | %.1f | %.1f |"
                      % (lab, name, len(v), sum(v) / len(v), min(v), max(v)))


if __name__ == "__main__":
    main()
