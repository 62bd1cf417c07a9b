"""Summaries of rocprofv3 output databases (rocpd SQLite files).

    python -m sparse_kv_refresh_amd.rocprof_summary stats  <run_results.db> [--steps K --warmup W]
    python -m sparse_kv_refresh_amd.rocprof_summary traffic <fetch.db> <write.db> --kernel NAME
        [--config c2_layer] [--skip-first N] [--out FILE]

`stats` prints the per-kernel launch count, total and average duration from a
`--kernel-trace` run.  Given the run's W warm-up and K timed steps, a kernel
launched a whole number of times per step is summarised over its dispatches
of the last K steps only; other kernels (copies, fills) over all of them.  `traffic` turns two `--pmc FETCH_SIZE` / `--pmc
WRITE_SIZE` runs into HBM bytes per launch of one kernel; each counter is
scaled by what it reads for a plain 1 GiB device-to-device copy captured in
the same run (bench.py --copy-calibration), so counter quirks of the chip
cancel out.
"""
from __future__ import annotations

import argparse
import collections
import hashlib
import json
import os
import re
import sqlite3
import sys

COPY_BYTES = 1 << 30

KIND_PATTERNS = {
    "gemm_qkv": r"gemm_bf16_\w*kernel<\(?wamc::GemmEpi\)?0|gemm_bf16_\w*kernel<0",
    "gemm_out_resid": r"gemm_bf16_\w*kernel<\(?wamc::GemmEpi\)?1|gemm_bf16_\w*kernel<1",
    "gemm_down_resid": r"gemm_bf16_\w*kernel<\(?wamc::GemmEpi\)?3|gemm_bf16_\w*kernel<3",
    "gemm_up_gelu": r"gemm_bf16_\w*kernel<\(?wamc::GemmEpi\)?2|gemm_bf16_\w*kernel<2",
    "attention": "attn_bf16_kernel",
    "score_pass1": "score_pass1_bf16",
    "score_pass2": "score_pass2_bf16",
    "select": "select_topk_kernel",
    "gather": "gather_kernel",
    "gather_ln": "gather_ln_kernel",
    "ln_mod": "ln_mod_kernel",
}
KERNEL_SOURCE = {"gemm_qkv": "gemm.hip", "gemm_out_resid": "gemm.hip", "gemm_up_gelu": "gemm.hip",
                 "gemm_down_resid": "gemm.hip", "attention": "attention.hip", "score_pass1": "score.hip",
                 "score_pass2": "score.hip", "select": "select.hip", "gather": "rows.hip", "gather_ln": "rows.hip", "ln_mod": "rows.hip"}


def kernel_stats(db: str):
    con = sqlite3.connect(db)
    rows = con.execute("select name, total_calls, total_duration, average from top_kernels").fetchall()
    return [(n, int(c), float(t), float(a)) for n, c, t, a in rows]


def kernel_stats_timed(db: str, steps: int, warmup: int):
    """Per kernel name: count, total and mean duration in microseconds of its
    dispatches in the last `steps` of `warmup + steps` steps, by start time
    (the kernels view holds ns)."""
    con = sqlite3.connect(db)
    per = collections.defaultdict(list)
    for n, dur in con.execute("select name, duration from kernels order by start"):
        per[n].append(float(dur))
    out = []
    for n, ds in per.items():
        if len(ds) % (steps + warmup) == 0:
            ds = ds[-(len(ds) // (steps + warmup)) * steps:]
        out.append((n, len(ds), sum(ds) / 1e3, sum(ds) / len(ds) / 1e3))
    return sorted(out, key=lambda r: -r[2])


def counters(db: str, name: str):
    con = sqlite3.connect(db)
    out = collections.defaultdict(list)
    for kn, cn, v, dispatch in con.execute(
            "select kernel_name, counter_name, value, dispatch_id from counters_collection order by dispatch_id"):
        if cn == name:
            out[kn].append(float(v))
    return out


def copy_factor(vals: dict, counter: str) -> float:
    copies = [v for kn, vs in vals.items() if "copyBuffer" in kn for v in vs]
    big = max(copies) if copies else 0.0
    if big <= 0:
        raise SystemExit(f"no calibration copy found for {counter}")
    return COPY_BYTES / (big * 1024.0)


def source_hash(fname: str) -> str:
    """Hash of a kernel's source file together with the shared headers it
    includes (every csrc/*.h, in name order), so that a change to either
    marks the counters taken before it as stale."""
    d = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
    h = hashlib.sha256()
    for name in [fname] + sorted(n for n in os.listdir(d) if n.endswith(".h")):
        with open(os.path.join(d, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("stats")
    a.add_argument("db")
    a.add_argument("--steps", type=int, default=0, help="timed steps of the run")
    a.add_argument("--warmup", type=int, default=0, help="warm-up steps of the run, before the timed ones")
    b = sub.add_parser("traffic")
    b.add_argument("fetch_db")
    b.add_argument("write_db")
    b.add_argument("--kernel", required=True)
    b.add_argument("--config", default="c2_layer")
    b.add_argument("--skip-first", type=int, default=1, help="launches dropped as warm-up")
    b.add_argument("--occurrence", type=int, default=0,
                   help="for kernels launched more than once per step: which launch of each step")
    b.add_argument("--per-step", type=int, default=1, help="launches of this kernel per step")
    b.add_argument("--out")
    args = ap.parse_args(argv)

    if args.cmd == "stats":
        # the rocpd top_kernels view reports durations in microseconds
        print(f"{'kernel':90s} {'calls':>6s} {'total_us':>11s} {'avg_us':>9s}")
        rows = kernel_stats_timed(args.db, args.steps, args.warmup) if args.steps > 0 else kernel_stats(args.db)
        for n, c, t, av in rows:
            print(f"{n[:90]:90s} {c:6d} {t:11.1f} {av:9.2f}")
        return

    pat = KIND_PATTERNS[args.kernel]
    res = {}
    for key, db, cname in (("fetch", args.fetch_db, "FETCH_SIZE"), ("write", args.write_db, "WRITE_SIZE")):
        vals = counters(db, cname)
        f = copy_factor(vals, cname)
        launches = [v for kn, vs in vals.items() if re.search(pat, kn) for v in vs]
        launches = launches[args.skip_first * args.per_step:]
        launches = launches[args.occurrence::args.per_step]
        if not launches:
            raise SystemExit(f"no launches of {pat} in {db}")
        kib = sum(launches) / len(launches)
        res[key] = {"raw_kib_per_launch": kib, "copy_factor": f, "bytes_per_launch": kib * 1024.0 * f,
                    "launches": len(launches)}
    src = KERNEL_SOURCE[args.kernel]
    rec = {"kernel": args.kernel, "config": args.config, "counter_runs": res,
           "hbm_bytes_per_launch": res["fetch"]["bytes_per_launch"] + res["write"]["bytes_per_launch"],
           "source_file": src, "source_sha256_16": source_hash(src)}
    text = json.dumps(rec, indent=1)
    if args.out:
        with open(args.out, "w") as fh:
            fh.write(text + "\n")
    print(text)


if __name__ == "__main__":
    main(sys.argv[1:])
