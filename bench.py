"""Benchmark of the sparse KV-refresh prefill on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c3_stack]

A step is one refresh chunk: token scores (attention mass + surprise),
selection with the age bound, gather, then every layer on the refreshed rows
(WAM-Cache, paperpeel 2610.11401, §4).  The default workload is the 30-layer
bf16 stack with d=1536, 12 heads, FFN 8960, N=4680 visual tokens (3 views of
30x52) and k=2808 (60 % refresh), 64 action queries, age bound 3, on a
16-chunk rollout of two moving blobs over a static scene.  Inputs are seeded
synthetic data already resident in HBM.  The steps walk the rollout's refresh
chunks in turn; the state after the dense chunk 0 is restored before each
pass over the rollout.

Printed as one JSON line: ms per refresh chunk (the metric: the mean, with
the median and p10/p90 of the per-chunk times), the library's own dense
prefill of the same chunks' latents, the speedup (mean ratio, paired median
and its bootstrap 95 % interval) and its k_eff/N bound, refreshed tokens/s,
the roofline of the dominant kernel (a further pass of the same K steps in
which every launch carries HIP events stamped with that kernel's own start
and end), and the CPU oracle timed on a bounded sample of the same workload.
Every timed loop starts behind a clock warm-up (clock_warm, reported as
clock_warm_chunks) and then W untimed warm-up steps.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps before each timed loop (default 5), after a clock warm-up of "
                         "at least %.2f s of the same work (the GPU clocks ramp up after idle)" % WARM_SECONDS)
    ap.add_argument("--config", default="c3_stack")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU time of the oracle sample")
    ap.add_argument("--profile-steps", action="store_true",
                    help="only run warmup + timed refresh steps (for rocprofv3 runs)")
    ap.add_argument("--profile-events", action="store_true",
                    help="with --profile-steps: HIP events around every launch, as in the per-kernel pass")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (HBM counter calibration)")
    ap.add_argument("--sweep", action="store_true",
                    help="refresh-fraction x age-bound sweep on the 30-layer stack shapes (one JSON line per point)")
    ap.add_argument("--plateau", action="store_true",
                    help="one-layer refresh latency vs refreshed rows, stepped every 32 rows (one JSON line)")
    ap.add_argument("--sweep-layers", type=int, default=30, help="layers of the stack used by --sweep")
    ap.add_argument("--small-n", action="store_true",
                    help="30-layer d=1536 stack at 120 / 480 / 1080 tokens with k = 0.584 N, eager and HIP-graph "
                         "replay (one JSON line each)")
    ap.add_argument("--capacity", action="store_true",
                    help="capacity filling on the 30-layer stack: chunk latency measured from k upward, then chunks at k and "
                         "at the plateau's upper end (one JSON line per k)")
    ap.add_argument("--union", action="store_true",
                    help="the pages' union rule on the 30-layer stack at budgets (b_a, b_s) = (0.4, 0.1) and "
                         "(0.6, 0.1), G = 2 (one JSON line each)")
    return ap.parse_args()


WARM_SECONDS = 0.15


def clock_warm(fn, min_calls: int = 1, seconds: float = WARM_SECONDS) -> int:
    """Call fn at least `min_calls` times and until `seconds` of wall time have
    passed; returns the number of calls.  After an idle gap (0.2 s is enough)
    the GPU needs about 40 ms of back-to-back work to bring its clocks back up:
    on the one-layer d=1536 chunk, steps timed straight after idle read
    0.45 ms and fall to a flat 0.382 ms after ~100 steps.  Every timed loop
    here starts behind such a warm-up so that it times the steady state."""
    import torch
    n = 0
    t0 = time.perf_counter()
    while True:
        for _ in range(4):
            fn()
        n += 4
        torch.cuda.synchronize()
        if n >= min_calls and time.perf_counter() - t0 >= seconds:
            return n


def kernel_work(wl, k_eff_total: int):
    """Algorithmic work per launch of each kernel kind: FLOPs for the MFMA
    kernels, HBM bytes for the memory-bound ones (act = 2 bytes in bf16).
    With a text cross-attention the attention kind holds two launches per
    layer (over N keys and over T text keys); its figure is their mean."""
    L, B, N, d, F, H, A = wl.n_layers, wl.batch, wl.n_tokens, wl.d_model, wl.d_ffn, wl.n_heads, wl.n_action
    T = getattr(wl, "n_text", 0)
    M = k_eff_total
    es = 2 if wl.dtype == "bf16" else 4
    attn = 4.0 * M * N * d if T == 0 else 0.5 * (4.0 * M * N * d + 4.0 * M * T * d)
    return {
        "gemm_ca_q": ("flop", 2.0 * M * d * d),
        "gemm_ca_out": ("flop", 2.0 * M * d * d),
        "gemm_qkv": ("flop", 2.0 * M * 3 * d * d),
        "gemm_out_resid": ("flop", 2.0 * M * d * d),
        "gemm_up_gelu": ("flop", 2.0 * M * F * d),
        "gemm_down_resid": ("flop", 2.0 * M * d * F),
        "attention": ("flop", attn),
        # K cache once (+ queries) per pass
        "score_pass1": ("byte", float(L * B * N * d * es + L * B * A * d * es)),
        "score_pass2": ("byte", float(L * B * N * d * es + L * B * A * d * es + L * H * B * N * 4)),
        "gather": ("byte", float(M * d * (es + 4 + es))),
        "gather_ln": ("byte", float(M * d * (es + 4 + es + es))),
        "ln_mod": ("byte", float(M * d * (4 + es))),
        "select": ("byte", float(B * N * (4 + 4 + 4 + 4))),
    }


KERNEL_SOURCE = {"gemm_qkv": "gemm.hip", "gemm_out_resid": "gemm.hip", "gemm_up_gelu": "gemm.hip",
                 "gemm_down_resid": "gemm.hip", "attention": "attention.hip", "score_pass1": "score.hip",
                 "score_pass2": "score.hip", "select": "select.hip", "gather": "rows.hip", "gather_ln": "rows.hip", "ln_mod": "rows.hip"}


def measured_traffic(kind: str, config: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or
    None when there is none or the kernel source changed since."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kind}_{config}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    from sparse_kv_refresh_amd.rocprof_summary import source_hash
    if rec.get("source_sha256_16") != source_hash(KERNEL_SOURCE[kind]):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(wl, seconds: float):
    """The oracle as it stands, on the host cores: one dense chunk to build the
    state, then refresh chunks of the same workload until ~`seconds`.  Stacks
    deeper than two layers or batches of episodes are sampled on the first two
    layers of episode 0 and scaled by layers x episodes (stated in `sample`)."""
    from oracle import wamc_oracle as O
    from sparse_kv_refresh_amd import inputs as W
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    L_used = min(2, wl.n_layers)
    swl = wl.with_(n_layers=L_used, batch=1)
    scale = (wl.n_layers / L_used) * wl.batch
    r = W.make_rollout(swl, chunks=2)
    prec = O.Precision(wl.dtype)
    t0 = time.perf_counter()
    st, _ = O.dense_prefill(r.z[0][0], r.weights, wl.n_heads, wl.ln_eps, prec,
                            text_emb=None if r.text is None else r.text[0])
    dense_s = time.perf_counter() - t0
    st.age = r.ages0[0].astype(np.int64)
    times = []
    while True:
        s = st.copy()
        t0 = time.perf_counter()
        O.refresh_chunk(s, r.z[0][1], r.qa[0][1], r.weights, wl.k, wl.age_bound, wl.n_heads, wl.ln_eps,
                        wl.w_attn, wl.w_surprise, prec)
        times.append(time.perf_counter() - t0)
        if sum(times) + dense_s >= seconds or len(times) >= 5:
            break
    what = (f"{len(times)} refresh chunk(s) of the {wl.name} workload (score + select + {wl.n_layers} layer(s), "
            f"k={wl.k} of N={wl.n_tokens})")
    if scale != 1:
        what = (f"{len(times)} refresh chunk(s) of the first {L_used} layers of one episode of the {wl.name} "
                f"workload (k={wl.k} of N={wl.n_tokens}), scaled x{scale:g} to {wl.n_layers} layers x "
                f"{wl.batch} episode(s)")
    return {"value": 1e3 * float(np.median(times)) * scale, "unit": "ms/chunk", "cores": int(threads),
            "kind": "oracle",
            "sample": what + f"; numpy {'float32+bf16 rounding' if wl.dtype == 'bf16' else 'float64'}; "
                             f"the oracle's dense chunk of the sample took {1e3 * dense_s:.0f} ms"}


def run_sweep(args):
    """Refresh fraction k/N x age bound G on the 30-layer stack shapes.  Per
    point: a dense chunk, then 15 refresh chunks of the moving-blob rollout
    with rows_cap = N (k_eff is only known on the device).  Reports the mean ms
    per refresh chunk over chunks 2..15, the realised k_eff per chunk, the dense
    ms, and two checks on the GPU's own state: k = N reproduces the dense
    prefill bitwise, and k = 0 from ages below the bound leaves the cache
    bitwise unchanged."""
    import torch
    from sparse_kv_refresh_amd import inputs as W
    from sparse_kv_refresh_amd import wamc
    base = W.preset("c3_stack", n_layers=args.sweep_layers)
    T = base.chunks
    r = W.make_rollout(base, chunks=T)
    dev = "cuda:0"
    weights = wamc.Engine.upload_weights(r.weights, torch.bfloat16, dev)
    N = base.n_tokens
    zs = [torch.from_numpy(r.z[0][t]).to(dev, torch.bfloat16)[None].contiguous() for t in range(T)]
    qs = [None] + [torch.from_numpy(r.qa[0][t]).to(dev, torch.bfloat16)[:, None].contiguous() for t in range(1, T)]
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * T)]
    for G in (2, 4, 8):
        wl = base.with_(age_bound=G)
        eng = wamc.Engine(wamc.dims_for(wl), weights, N, dev)
        for frac in (0.0, 0.1, 0.25, 0.5, 0.75, 1.0):
            k = int(round(frac * N))
            clock_warm(lambda: eng.dense(zs[0]))
            before = eng.snapshot() if k == 0 else None
            check = {}
            for t in range(1, T):
                ev[2 * t].record(stream)
                eng.chunk(zs[t], qs[t], k, stream=stream)
                ev[2 * t + 1].record(stream)
                if t == 1 and k == 0:
                    check["k0_cache_unchanged"] = bool(torch.equal(eng.k_cache, before["k_cache"]) and
                                                       torch.equal(eng.v_cache, before["v_cache"]) and
                                                       torch.equal(eng.zref, before["zref"]))
                    before = None
                if t == 1 and k == N:
                    after = eng.snapshot()
                    eng.dense(zs[1])
                    check["kN_equals_dense"] = bool(torch.equal(eng.k_cache, after["k_cache"]) and
                                                    torch.equal(eng.v_cache, after["v_cache"]))
                    eng.restore(after)
                    del after
            torch.cuda.synchronize()
            ms = [ev[2 * t].elapsed_time(ev[2 * t + 1]) for t in range(2, T)]
            dms = []
            for _ in range(3):
                ev[0].record(stream)
                eng.dense(zs[T - 1], stream=stream)
                ev[1].record(stream)
                torch.cuda.synchronize()
                dms.append(ev[0].elapsed_time(ev[1]))
            # k_eff per chunk is re-derived from a replay that records it
            eng.dense(zs[0])
            keffs = []
            for t in range(1, T):
                eng.chunk(zs[t], qs[t], k, stream=stream)
                keffs.append(int(eng.k_eff[0]))
            mean_ms = float(np.mean(ms))
            print(json.dumps({"sweep": "refresh_fraction_x_age_bound", "layers": wl.n_layers, "n_tokens": N,
                              "age_bound": G, "k": k, "k_over_n": frac, "k_eff_per_chunk": keffs,
                              "k_eff_mean": float(np.mean(keffs)), "ms_per_chunk": mean_ms,
                              "ms_per_chunk_p10_p90": [float(np.percentile(ms, 10)), float(np.percentile(ms, 90))],
                              "dense_ms": float(np.median(dms)), "speedup_vs_dense": float(np.median(dms)) / mean_ms,
                              "speedup_bound": N / max(float(np.mean(keffs)), 1.0), **check}), flush=True)
        del eng


def budget_rows(fraction: float, n_tokens: int) -> int:
    """Token count of a refresh budget given as a fraction of the tokens:
    ceil(fraction * n_tokens), taken on the decimal value (0.4 of 4680 is
    1872, where binary floating point would give 1873).  The library takes
    the counts; turning the pages' budget fractions into counts is the
    caller's part."""
    from fractions import Fraction
    return min(n_tokens, -(-Fraction(repr(float(fraction))) * n_tokens // 1))


def run_union(args):
    """The union refresh rule (top ceil(b_a N) by attention mass, top
    ceil(b_s N) by surprise, forced tokens; WAM-Cache §1, §4.3, §4.4) on the
    30-layer stack shapes with G = 2: a dense chunk, then 15 refresh chunks;
    ms per chunk over chunks 2..15, the recompute ratio rho = mean k_eff / N
    (WAM-Cache §5.3) and the speedup against its bound 1/rho (§5.2)."""
    import torch
    from sparse_kv_refresh_amd import inputs as W
    from sparse_kv_refresh_amd import wamc
    base = W.preset("c3_stack", n_layers=args.sweep_layers, age_bound=2)
    T = base.chunks
    r = W.make_rollout(base, chunks=T)
    dev = "cuda:0"
    weights = wamc.Engine.upload_weights(r.weights, torch.bfloat16, dev)
    N = base.n_tokens
    zs = [torch.from_numpy(r.z[0][t]).to(dev, torch.bfloat16)[None].contiguous() for t in range(T)]
    qs = [None] + [torch.from_numpy(r.qa[0][t]).to(dev, torch.bfloat16)[:, None].contiguous() for t in range(1, T)]
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * T)]
    eng = wamc.Engine(wamc.dims_for(base), weights, N, dev)
    for b_a, b_s in ((0.4, 0.1), (0.6, 0.1)):
        na, ns = budget_rows(b_a, N), budget_rows(b_s, N)
        clock_warm(lambda: eng.dense(zs[0]))
        keffs = []
        for t in range(1, T):
            ev[2 * t].record(stream)
            eng.chunk_union(zs[t], qs[t], na, ns, stream=stream)
            ev[2 * t + 1].record(stream)
            keffs.append(eng.k_eff[0].clone())
        torch.cuda.synchronize()
        keffs = [int(k) for k in keffs]
        ms = [ev[2 * t].elapsed_time(ev[2 * t + 1]) for t in range(2, T)]
        dms = []
        for _ in range(3):
            ev[0].record(stream)
            eng.dense(zs[T - 1], stream=stream)
            ev[1].record(stream)
            torch.cuda.synchronize()
            dms.append(ev[0].elapsed_time(ev[1]))
        rho = float(np.mean(keffs[1:])) / N
        mean_ms = float(np.mean(ms))
        print(json.dumps({"union": {"b_a": b_a, "b_s": b_s, "n_attn": na, "n_surprise": ns}, "age_bound": 2,
                          "layers": base.n_layers, "n_tokens": N, "k_eff_per_chunk": keffs, "rho": rho,
                          "ms_per_chunk": mean_ms, "dense_ms": float(np.median(dms)),
                          "speedup_vs_dense": float(np.median(dms)) / mean_ms, "speedup_bound": 1.0 / rho}),
              flush=True)


def run_small_n(args):
    """The pages' latency experiment (WAM-Cache §5.2, Figure 3): the refresh
    ratio measured at the native 120 tokens (0.584) replayed at 120, 480 and
    1080 tokens (a 12x10 grid and 4x / 9x larger ones) on the 30-layer d=1536
    stack; refresh and dense chunks timed eagerly and as HIP-graph replays
    (the pages use CUDA-graph replay)."""
    import torch
    from sparse_kv_refresh_amd import inputs as W
    from sparse_kv_refresh_amd import wamc
    dev = "cuda:0"
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    weights = None
    for rows, cols in ((12, 10), (24, 20), (36, 30)):
        N = rows * cols
        k = int(round(0.584 * N))
        wl = W.preset("c3_stack", n_layers=args.sweep_layers, views=1, rows=rows, cols=cols, k=k, age_bound=2)
        r = W.make_rollout(wl, chunks=2)
        if weights is None:
            weights = wamc.Engine.upload_weights(r.weights, torch.bfloat16, dev)
        eng = wamc.Engine(wamc.dims_for(wl), weights, k, dev)
        z0 = torch.from_numpy(r.z[0][0]).to(dev, torch.bfloat16)[None].contiguous()
        z1 = torch.from_numpy(r.z[0][1]).to(dev, torch.bfloat16)[None].contiguous()
        q1 = torch.from_numpy(r.qa[0][1]).to(dev, torch.bfloat16)[:, None].contiguous()
        eng.dense(z0)
        torch.cuda.synchronize()
        snap = eng.snapshot()

        def refresh():
            eng.chunk(z1, q1, k)

        def dense():
            eng.dense(z1)

        def eager(fn, reps=20):
            clock_warm(fn, 3)
            a.record(stream)
            for _ in range(reps):
                fn()
            b.record(stream)
            torch.cuda.synchronize()
            return a.elapsed_time(b) / reps

        def graphed(fn, reps=20):
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                fn()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn()
            clock_warm(g.replay, 3)
            a.record(stream)
            for _ in range(reps):
                g.replay()
            b.record(stream)
            torch.cuda.synchronize()
            return a.elapsed_time(b) / reps

        # k >= N/2, so k_eff = k in every chunk and repeated chunks do equal work
        out = {"small_n": N, "grid": [rows, cols], "layers": wl.n_layers, "k": k, "rho": k / N}
        out["refresh_ms_eager"] = eager(refresh)
        eng.restore(snap)
        out["refresh_ms_graph"] = graphed(refresh)
        out["dense_ms_eager"] = eager(dense)
        out["dense_ms_graph"] = graphed(dense)
        out["speedup_eager"] = out["dense_ms_eager"] / out["refresh_ms_eager"]
        out["speedup_graph"] = out["dense_ms_graph"] / out["refresh_ms_graph"]
        out["speedup_bound"] = N / k
        # per-kernel split of one layer's time, refresh and dense (eager calls, kernel timer)
        for name, fn in (("refresh", refresh), ("dense", dense)):
            eng.restore(snap)
            wamc.timing_enable(True)
            for _ in range(5):
                fn()
            torch.cuda.synchronize()
            kt = wamc.timing_read()
            wamc.timing_enable(False)
            out[f"{name}_kernel_us_per_chunk"] = {kk: 1e3 * tot / 5 for kk, (n, tot) in kt.items()}
        print(json.dumps(out), flush=True)
        del eng


def run_capacity(args):
    """Capacity filling (RealtimeWAM §3: the upper end of the latency plateau
    holding the required token count is the execution capacity; the spare
    slots are filled with the next-ranked tokens).  The curve is measured on
    whole 30-layer chunks: for each requested k the chunk is timed at
    k, k + 32, ..., k + 512 rows (one engine sized for every token, ages reset
    before each chunk so exactly that many rows refresh), and k_fill is the
    largest count whose latency stays within 1 % of the latency at k.  Each
    line reports the curve, k_fill and the chunk latency at k and at k_fill."""
    import torch
    from sparse_kv_refresh_amd import inputs as W
    from sparse_kv_refresh_amd import wamc
    from sparse_kv_refresh_amd.capacity import plateau_capacity
    dev = "cuda:0"
    stream = torch.cuda.current_stream()
    wl = W.preset("c3_stack", n_layers=args.sweep_layers)
    N = wl.n_tokens
    r = W.make_rollout(wl, chunks=2)
    weights = wamc.Engine.upload_weights(r.weights, torch.bfloat16, dev)
    z0 = torch.from_numpy(r.z[0][0]).to(dev, torch.bfloat16)[None].contiguous()
    z1 = torch.from_numpy(r.z[0][1]).to(dev, torch.bfloat16)[None].contiguous()
    q1 = torch.from_numpy(r.qa[0][1]).to(dev, torch.bfloat16)[:, None].contiguous()
    eng = wamc.Engine(wamc.dims_for(wl), weights, N, dev)
    eng.dense(z0)
    start = eng.snapshot()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(8)]

    def chunk_ms(kk, reps=7):
        eng.restore(start)
        for i in range(reps):
            eng.age.zero_()
            ev[i][0].record(stream)
            eng.chunk(z1, q1, kk, stream=stream)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        return float(np.median([x.elapsed_time(y) for x, y in ev[1:reps]]))

    def one_chunk():
        eng.age.zero_()
        eng.chunk(z1, q1, 2808, stream=stream)
    clock_warm(one_chunk)
    for k in (468, 1170, 2340, 2458, 2808):
        rows = [k + 32 * j for j in range(17) if k + 32 * j <= N]
        curve = [chunk_ms(kk) for kk in rows]
        k_fill = plateau_capacity(rows, curve, k, tol=0.01)
        at_k, at_fill = chunk_ms(k), chunk_ms(k_fill)
        print(json.dumps({"capacity": {"k": k, "k_fill": k_fill, "extra_tokens": k_fill - k, "tolerance": 0.01},
                          "layers": wl.n_layers, "n_tokens": N, "curve_rows": rows, "curve_ms": curve,
                          "ms_at_k": at_k, "ms_at_fill": at_fill, "latency_change": at_fill / at_k - 1.0}),
              flush=True)


def run_plateau(args):
    """One d=1536 layer over N=4680 cached tokens: wamc_refresh_layer latency
    as the number of refreshed rows m grows by 32, once with the launch sized
    for the rows (rows_cap = m) and once sized for all N tokens with k_eff = m
    read on the device (rows_cap = N)."""
    import torch
    from sparse_kv_refresh_amd import inputs as W
    from sparse_kv_refresh_amd import wamc
    wl = W.preset("c3_stack", n_layers=1)
    r = W.make_rollout(wl, chunks=1)
    dev = "cuda:0"
    dims = wamc.dims_for(wl)
    w = wamc.Engine.upload_weights(r.weights, torch.bfloat16, dev)[0]
    N, d = wl.n_tokens, wl.d_model
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    kc = torch.randn((1, N, d), device=dev, generator=g).to(torch.bfloat16)
    vc = torch.randn((1, N, d), device=dev, generator=g).to(torch.bfloat16)
    x0 = torch.randn((1, N, d), device=dev, generator=g)
    idx = torch.arange(N, dtype=torch.int32, device=dev)[None].contiguous()
    ws = torch.empty(wamc.workspace_bytes(dims, N), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    rows = list(range(32, N + 1, 32)) + ([N] if N % 32 else [])
    curves = {}
    keff_n = torch.tensor([N], dtype=torch.int32, device=dev)
    xw = x0.clone()  # the call updates its rows in place
    for mode in ("rows_cap_m", "rows_cap_N"):
        clock_warm(lambda: wamc.refresh_layer(dims, 0, w, xw, idx, keff_n, N, kc, vc, ws, stream=stream))
        times = []
        for m in rows:
            cap = m if mode == "rows_cap_m" else N
            keff = torch.tensor([m], dtype=torch.int32, device=dev)
            x = x0[:, :cap].contiguous()
            for _ in range(2):
                wamc.refresh_layer(dims, 0, w, x, idx, keff, cap, kc, vc, ws, stream=stream)
            a.record(stream)
            for _ in range(5):
                wamc.refresh_layer(dims, 0, w, x, idx, keff, cap, kc, vc, ws, stream=stream)
            b.record(stream)
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b) / 5)
        curves[mode] = times
    # per-kernel split of the same calls (HIP events around every launch), every 128 rows
    kernel_rows = [m for m in rows if m % 128 == 0 or m == 32 or m == N]
    per_kernel = {}
    for mode in ("rows_cap_m", "rows_cap_N"):
        per_kernel[mode] = []
        for m in kernel_rows:
            cap = m if mode == "rows_cap_m" else N
            keff = torch.tensor([m], dtype=torch.int32, device=dev)
            x = x0[:, :cap].contiguous()
            wamc.refresh_layer(dims, 0, w, x, idx, keff, cap, kc, vc, ws, stream=stream)
            torch.cuda.synchronize()
            wamc.timing_enable(True)
            for _ in range(3):
                wamc.refresh_layer(dims, 0, w, x, idx, keff, cap, kc, vc, ws, stream=stream)
            torch.cuda.synchronize()
            kt = wamc.timing_read()
            wamc.timing_enable(False)
            per_kernel[mode].append({k: 1e3 * tot / max(n, 1) for k, (n, tot) in kt.items()})
    print(json.dumps({"plateau": "refresh_layer", "d_model": d, "n_tokens": N, "rows": rows,
                      "ms_per_layer": curves, "kernel_rows": kernel_rows, "kernel_us": per_kernel}), flush=True)


def bootstrap_ci(values, stat=np.median, reps: int = 2000, seed: int = 0):
    """95 % percentile-bootstrap interval of `stat` over the values."""
    v = np.asarray(values, dtype=np.float64)
    rng = np.random.default_rng(seed)
    boots = [stat(v[rng.integers(0, len(v), len(v))]) for _ in range(reps)]
    return [float(np.percentile(boots, 2.5)), float(np.percentile(boots, 97.5))]


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); episodes shard across GPUs "
              "with no exchange, so the per-GPU figure at --gpus 1 is the whole story", file=sys.stderr)
        sys.exit(2)

    if args.sweep:
        return run_sweep(args)
    if args.plateau:
        return run_plateau(args)
    if args.union:
        return run_union(args)
    if args.capacity:
        return run_capacity(args)
    if args.small_n:
        return run_small_n(args)

    import torch
    from sparse_kv_refresh_amd import inputs as W
    from sparse_kv_refresh_amd import wamc

    wl = W.preset(args.config)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    adt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    # the rollout: a dense chunk 0, then refresh chunks 1..T-1, every chunk's
    # latents and action queries resident in HBM before anything is timed
    T = max(2, wl.chunks)
    r = W.make_rollout(wl, chunks=T)
    dims = wamc.dims_for(wl)
    weights = wamc.Engine.upload_weights(r.weights, adt, dev)
    rows_cap = wl.k if wl.k >= (wl.n_tokens + 1) // 2 else wl.n_tokens
    eng = wamc.Engine(dims, weights, rows_cap, dev)
    if r.text is not None:
        # the instruction's keys/values, once per episode (outside the timed steps)
        eng.text_kv(torch.from_numpy(np.stack(r.text)).to(dev, adt).contiguous())

    zs = [torch.from_numpy(np.stack([r.z[e][t] for e in range(wl.batch)])).to(dev, adt).contiguous()
          for t in range(T)]
    qs = [None] + [torch.from_numpy(np.stack([r.qa[e][t] for e in range(wl.batch)], axis=1)).to(dev, adt)
                   .contiguous() for t in range(1, T)]
    ages0 = torch.from_numpy(np.stack(r.ages0)).to(dev)
    stream = torch.cuda.current_stream()

    if not args.profile_steps:
        # profiled runs skip the dense chunk so every traced launch is a refresh launch
        eng.dense(zs[0])
    eng.age.copy_(ages0)
    torch.cuda.synchronize()
    start = eng.snapshot()       # the state after chunk 0; every pass over the rollout starts here

    def chunk_of(i):
        return 1 + i % (T - 1)

    def before_step(i):
        # a new pass over the rollout restores the state after chunk 0
        # (outside the chunk's own events)
        if i > 0 and chunk_of(i) == 1:
            eng.restore(start)

    def refresh_step(i):
        t = chunk_of(i)
        eng.chunk(zs[t], qs[t], wl.k, stream=stream)

    def dense_step(i):
        eng.dense(zs[chunk_of(i)], stream=stream)

    def run(step, n, events=None, on_step=None):
        for i in range(n):
            before_step(i)
            if events is not None:
                events[i][0].record(stream)
            step(i)
            if events is not None:
                events[i][1].record(stream)
            if on_step is not None:
                on_step(i)

    def warm(step, warmup):
        """Clock warm-up (at least 0.15 s of this work: the clocks ramp for
        ~40 ms after idle), then the requested warm-up steps; the state is
        restored after it."""
        calls = [0]

        def one():
            before_step(calls[0])
            step(calls[0])
            calls[0] += 1
        n_clock = clock_warm(one, 1)
        run(step, warmup)
        torch.cuda.synchronize()
        eng.restore(start)
        return n_clock

    def timed(step, steps, warmup, on_step=None):
        n_clock = warm(step, warmup)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run(step, steps, ev, on_step)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        per = np.array([a.elapsed_time(b) for a, b in ev])
        return per, 1e3 * wall / steps, n_clock

    warmup = 5 if args.warmup is None else args.warmup
    if args.profile_steps:
        if args.profile_events:
            wamc.timing_enable(True)
        per, _, n_clock = timed(refresh_step, args.steps, warmup)
        if args.profile_events:
            kt = wamc.timing_read()
            wamc.timing_enable(False)
            print(json.dumps({k: 1e3 * tot / max(n, 1) for k, (n, tot) in kt.items()}))
        if args.copy_calibration:
            src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
            dst = torch.empty_like(src)
            for _ in range(3):
                dst.copy_(src)
            torch.cuda.synchronize()
        print(json.dumps({"profile_steps": args.steps, "warmup": warmup, "clock_warm_chunks": n_clock,
                          "ms_per_step": float(per.mean())}))
        return

    # refresh chunks, each timed by its own event pair; k_eff of every step kept
    keff_log = torch.zeros((args.steps, wl.batch), dtype=torch.int32, device=dev)
    per_refresh, wall_refresh, clock_refresh = timed(refresh_step, args.steps, warmup,
                                                     on_step=lambda i: keff_log[i].copy_(eng.k_eff))
    keff_steps = keff_log.cpu().numpy().astype(np.int64)
    k_total = float(keff_steps.sum(axis=1).mean())        # refreshed rows per chunk, all episodes
    # the library's dense prefill of the same chunks' latents, step for step
    per_dense, _, _ = timed(dense_step, args.steps, warmup)
    eng.restore(start)

    # per-kernel pass: HIP events carried by every launch, same K steps
    warm(refresh_step, warmup)
    wamc.timing_enable(True)
    run(refresh_step, args.steps)
    torch.cuda.synchronize()
    kt = wamc.timing_read()
    wamc.timing_enable(False)

    work = kernel_work(wl, k_total)
    kernels = {}
    for kind, (n, tot) in kt.items():
        entry = {"launches": n, "avg_us": 1e3 * tot / max(n, 1), "ms_per_step": tot / args.steps}
        if kind in work:
            unit, amount = work[kind]
            avg_s = tot / max(n, 1) / 1e3
            if unit == "flop":
                entry["tflops"] = amount / avg_s / 1e12
                entry["frac_bf16_peak"] = entry["tflops"] / PEAK_BF16_TFLOPS
            else:
                entry["gbs"] = amount / avg_s / 1e9
                entry["frac_hbm_peak"] = entry["gbs"] / PEAK_HBM_GBS
        kernels[kind] = entry
    dominant = max((k for k in kernels if k in work), key=lambda k: kernels[k]["ms_per_step"])
    unit, amount = work[dominant]
    avg_s = kernels[dominant]["avg_us"] / 1e6
    if unit == "flop":
        ach = amount / avg_s / 1e12
        peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_FP32_TFLOPS
        roof = {"bound": "mfma", "achieved": ach, "peak": peak, "unit": "TFLOP/s", "frac": ach / peak}
    else:
        ach = amount / avg_s / 1e9
        roof = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": ach / PEAK_HBM_GBS}
    roof["traffic"] = measured_traffic(dominant, args.config)
    roof["kernel"] = dominant
    roof["work_per_launch"] = amount
    roof["avg_launch_us"] = kernels[dominant]["avg_us"]

    cpu = None if args.no_cpu_baseline else cpu_baseline(wl, args.cpu_seconds)

    ms_refresh = float(per_refresh.mean())
    ratio = per_dense / per_refresh                      # paired: the same chunk's latents
    bound = wl.n_tokens * wl.batch / max(k_total, 1.0)
    pct = lambda a, q: float(np.percentile(a, q))
    line = {
        "metric": "refresh-prefill ms/chunk & speedup vs dense at 60% refresh; MFMA/HBM % peak",
        "value": ms_refresh,
        "unit": "ms/chunk",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": warmup,
        "clock_warm_chunks": clock_refresh,
        "ms_per_step": ms_refresh,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "n_layers": wl.n_layers, "d_model": wl.d_model, "n_heads": wl.n_heads,
                   "d_ffn": wl.d_ffn, "n_tokens": wl.n_tokens, "k": wl.k, "k_eff_mean": k_total / wl.batch,
                   "n_action": wl.n_action, "age_bound": wl.age_bound, "batch": wl.batch,
                   "rollout_chunks": T, "rows_cap": rows_cap, "parallelism": "single GPU"},
        "ms_per_chunk_median": float(np.median(per_refresh)),
        "ms_per_chunk_p10_p90": [pct(per_refresh, 10), pct(per_refresh, 90)],
        "dense_ms_per_chunk": float(per_dense.mean()),
        "dense_ms_median": float(np.median(per_dense)),
        "dense_ms_p10_p90": [pct(per_dense, 10), pct(per_dense, 90)],
        "speedup_vs_dense": float(per_dense.mean()) / ms_refresh,
        "speedup_median_paired": float(np.median(ratio)),
        "speedup_ci95_bootstrap": bootstrap_ci(ratio),
        "speedup_bound": bound,
        "speedup_frac_of_bound": (float(per_dense.mean()) / ms_refresh) / bound,
        "refreshed_tokens_per_s": k_total / (ms_refresh / 1e3),
        "wall_ms_per_step": wall_refresh,
        "timing": (f"each step is one refresh chunk of a {T}-chunk rollout (chunks 1..{T - 1} in turn; the state "
                   "after the dense chunk 0 is restored before each pass, outside the chunk's events) timed by "
                   "its own HIP event pair; dense steps run the library's dense prefill on the same chunks' "
                   "latents, step for step, and the speedup CI resamples those pairs; before each timed loop "
                   "the clocks are warmed by clock_warm_chunks chunks (>= 0.15 s), then `warmup` more"),
        "roofline": roof,
        "kernels": kernels,
        "kernel_timing": "third pass of the same steps; every launch carries HIP events stamped with the "
                         "kernel's own start and end on the launch stream (hipExtLaunchKernel)",
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
