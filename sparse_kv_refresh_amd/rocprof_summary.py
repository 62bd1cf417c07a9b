"""Summaries of rocprofv3 output databases (rocpd SQLite files).

    python -m sparse_kv_refresh_amd.rocprof_summary stats  <run_results.db> [--steps K --warmup W]
    python -m sparse_kv_refresh_amd.rocprof_summary traffic <fetch.db> <write.db> --kernel NAME
        [--config c2_layer] [--skip-first N] [--out FILE]
    python -m sparse_kv_refresh_amd.rocprof_summary sq <run_results.db>

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
    "gemm_qkv": r"gemm_bf16_\w*kernel<(\(wamc::GemmEpi\))?0[,>]",
    "gemm_out_resid": r"gemm_bf16_\w*kernel<(\(wamc::GemmEpi\))?1[,>]",
    "gemm_down_resid": r"gemm_bf16_\w*kernel<(\(wamc::GemmEpi\))?3[,>]",
    "gemm_up_gelu": r"gemm_bf16_\w*kernel<(\(wamc::GemmEpi\))?2[,>]",
    "attention": "attn_bf16_kernel",
    "score_pass1": "score_pass1_bf16",
    "score_pass2": "score_pass2_bf16",
    "select": "select_topk_kernel",
    "gather": "gather_kernel",
    "gather_ln": "gather_ln_kernel",
    "ln_mod": "ln_mod_kernel",
}
# Split-K launches of a projection run a second kernel (the reduction of the
# f32 planes, with the epilogue and, after a residual, the LayerNorm that
# follows); a launch of the kind is the pair.
SECOND_PATTERNS = {
    "gemm_qkv": r"gemm_parts_(resid_ln_kernel<\d+, |epilogue_kernel<)(\(wamc::GemmEpi\))?0[,>]",
    "gemm_out_resid": r"gemm_parts_(resid_ln_kernel<\d+, |epilogue_kernel<)(\(wamc::GemmEpi\))?1[,>]",
    "gemm_up_gelu": r"gemm_parts_(resid_ln_kernel<\d+, |epilogue_kernel<)(\(wamc::GemmEpi\))?2[,>]",
    "gemm_down_resid": r"gemm_parts_(resid_ln_kernel<\d+, |epilogue_kernel<)(\(wamc::GemmEpi\))?3[,>]",
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


SQ_COUNTERS = ("SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_VALU",
               "SQ_ACTIVE_INST_LDS")


def sq_summary(db: str):
    """Per kernel name, from one `--pmc SQ_WAVES SQ_WAVE_CYCLES ...` run:
    launches, waves per launch and the shares of all resident wave-cycles
    spent waiting on anything, waiting on a dependency, and issuing VALU and
    LDS instructions (each counter summed over the launches, so the shares
    weight launches by their wave-cycles)."""
    vals = {cn: counters(db, cn) for cn in SQ_COUNTERS}
    out = []
    for kn, cyc in vals["SQ_WAVE_CYCLES"].items():
        tot = sum(cyc)
        if tot <= 0:
            continue
        share = {cn: sum(vals[cn].get(kn, [0.0])) / tot for cn in SQ_COUNTERS[2:]}
        waves = vals["SQ_WAVES"].get(kn, [0.0])
        out.append((kn, len(cyc), sum(waves) / max(len(waves), 1), share, tot))
    return sorted(out, key=lambda r: -r[4])


MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "GRBM_GUI_ACTIVE")


def mfma_summary(db: str, chunks: int, last: int, simds: int, xcds: int):
    """Per kernel kind, from one `--pmc SQ_VALU_MFMA_BUSY_CYCLES
    SQ_INSTS_VALU_MFMA_MOPS_BF16 GRBM_GUI_ACTIVE` run of `chunks` steps: the
    mean of each counter per launch over the launches of the last `last`
    steps, the MFMA busy share and the bf16 MFMA flops executed (MOPS x 512).
    As stored per dispatch, the MFMA busy cycles are summed over all SIMDs
    and GRBM_GUI_ACTIVE over the XCDs (divided by the XCD count it matches
    the traced kernel duration at 2.4 GHz), so the busy share is
    busy / (active / xcds * simds)."""
    vals = {c: counters(db, c) for c in MFMA_COUNTERS}
    out = {}
    for kind, pat in KIND_PATTERNS.items():
        per = {cname: [v for kn, vs in table.items() if re.search(pat, kn) for v in vs]
               for cname, table in vals.items()}
        n = min(len(v) for v in per.values())
        if n == 0 or n % chunks:
            continue
        drop = n - (n // chunks) * last
        mean = {c: sum(v[drop:n]) / (n - drop) for c, v in per.items()}
        launches = n - drop
        if kind in SECOND_PATTERNS:
            # the second kernel of a split-K launch, per name (see traffic)
            for c, table in vals.items():
                kept = [vs[len(vs) - len(vs) * last // chunks:] for kn, vs in table.items()
                        if re.search(SECOND_PATTERNS[kind], kn) and len(vs) % chunks == 0]
                n2 = sum(len(k) for k in kept)
                if n2:
                    mean[c] += sum(sum(k) for k in kept) / n2
        busy, mops, active = (mean[c] for c in MFMA_COUNTERS)
        out[kind] = {"launches": launches, "mfma_busy_cycles": busy, "gpu_active_cycles_per_xcd": active / xcds,
                     "mfma_util": busy / (active / xcds * simds) if active > 0 else None,
                     "bf16_mfma_flops": mops * 512.0, "source_file": KERNEL_SOURCE[kind],
                     "source_sha256_16": source_hash(KERNEL_SOURCE[kind])}
    return {"counters": list(MFMA_COUNTERS), "simds": simds, "xcds": xcds, "kernels": out}


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
    q = sub.add_parser("sq")
    q.add_argument("db")
    c = sub.add_parser("mfma")
    c.add_argument("db")
    c.add_argument("--config", default="c3_stack")
    c.add_argument("--chunks", type=int, required=True, help="steps the run made (warm-up included)")
    c.add_argument("--last", type=int, required=True, help="steps summarised: the last ones of the run")
    c.add_argument("--simds", type=int, default=1024, help="SIMDs of the chip (256 CUs x 4)")
    c.add_argument("--xcds", type=int, default=8, help="instances GRBM_GUI_ACTIVE is summed over")
    c.add_argument("--out")
    args = ap.parse_args(argv)

    if args.cmd == "mfma":
        rec = mfma_summary(args.db, args.chunks, args.last, args.simds, args.xcds)
        rec["config"] = args.config
        text = json.dumps(rec, indent=1)
        if args.out:
            with open(args.out, "w") as fh:
                fh.write(text + "\n")
        print(text)
        return

    if args.cmd == "sq":
        print(f"{'kernel':90s} {'launches':>8s} {'waves':>7s} {'wait':>6s} {'dep':>6s} {'valu':>6s} {'lds':>6s}")
        for kn, n, waves, sh, _ in sq_summary(args.db):
            print(f"{kn[:90]:90s} {n:8d} {waves:7.0f} {100 * sh['SQ_WAIT_ANY']:5.0f}% {100 * sh['SQ_WAIT_INST_ANY']:5.0f}%"
                  f" {100 * sh['SQ_ACTIVE_INST_VALU']:5.0f}% {100 * sh['SQ_ACTIVE_INST_LDS']:5.1f}%")
        return

    if args.cmd == "stats":
        # the rocpd top_kernels view reports durations in microseconds
        print(f"{'kernel':90s} {'calls':>6s} {'total_us':>11s} {'avg_us':>9s}")
        rows = kernel_stats_timed(args.db, args.steps, args.warmup) if args.steps > 0 else kernel_stats(args.db)
        for n, c, t, av in rows:
            print(f"{n[:90]:90s} {c:6d} {t:11.1f} {av:9.2f}")
        # a projection launch that runs a split-K reduction too is the pair
        pairs = []
        for kind, pat in KIND_PATTERNS.items():
            if kind not in SECOND_PATTERNS:
                continue
            first = [r for r in rows if re.search(pat, r[0])]
            second = [r for r in rows if re.search(SECOND_PATTERNS[kind], r[0])]
            if first and second:
                calls = sum(r[1] for r in first)
                pairs.append((kind, calls, sum(r[2] for r in first + second)))
        if pairs:
            print()
            print("per launch of a projection whose split-K reduction is a second kernel (both kernels):")
            for kind, calls, tot in pairs:
                print(f"{kind:90s} {calls:6d} {tot:11.1f} {tot / calls:9.2f}")
        return

    pats = [KIND_PATTERNS[args.kernel]] + ([SECOND_PATTERNS[args.kernel]] if args.kernel in SECOND_PATTERNS else [])
    res = {}
    for key, db, cname in (("fetch", args.fetch_db, "FETCH_SIZE"), ("write", args.write_db, "WRITE_SIZE")):
        vals = counters(db, cname)
        f = copy_factor(vals, cname)
        first = [v for kn, vs in vals.items() if re.search(pats[0], kn) for v in vs]
        total = len(first)
        launches = first[args.skip_first * args.per_step:]
        launches = launches[args.occurrence::args.per_step]
        if not launches:
            raise SystemExit(f"no launches of {pats[0]} in {db}")
        kib, n_launch, parts = sum(launches) / len(launches), len(launches), 1
        if len(pats) > 1:
            # the second kernel may be one of several (the reduction with the
            # LayerNorm, or without it after the last layer): each name drops
            # the warm-up share of its own launches, then the launch-weighted mean
            frac = args.skip_first * args.per_step / total
            kept = [vs[round(len(vs) * frac):] for kn, vs in vals.items() if re.search(pats[1], kn)]
            n2 = sum(len(k) for k in kept)
            if n2:
                kib += sum(sum(k) for k in kept) / n2
                parts += 1
        res[key] = {"raw_kib_per_launch": kib, "copy_factor": f, "bytes_per_launch": kib * 1024.0 * f,
                    "launches": n_launch, "kernels_per_launch": parts}
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
