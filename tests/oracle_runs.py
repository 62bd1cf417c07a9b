"""Oracle rollouts of one episode, for the full-size GPU parity tests.

CPU only: imports the oracle and the seeded input generators, never torch or
the HIP library, so the tests can run several episodes in spawned worker
processes while the test process holds the GPU.  Results come back as plain
arrays; the bf16 cache values are returned as their raw 16-bit patterns
(every value the oracle stores at a bf16 storage point is exactly
representable), which halves what crosses the process boundary.
"""
from __future__ import annotations

import multiprocessing
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np

from oracle import wamc_oracle as O
from sparse_kv_refresh_amd import inputs as W


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """The upper 16 bits of float32 values that are bf16-representable."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    assert not (u & 0xFFFF).any(), "value is not bf16-representable"
    return (u >> 16).astype(np.uint16)


def from_bf16_bits(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def episode_inputs(wl: W.Workload, episode: int, chunks: int):
    """z[t] and Qa[t] of one episode, drawn exactly as make_rollout does."""
    w_pe = W.make_patch_embed(wl)
    src = W.LatentSource(wl, episode)
    z = [W.tokens_from_latent(wl, src.latent(t), w_pe) for t in range(chunks)]
    qa = [None] + [W.make_queries(wl, t, episode) for t in range(1, chunks)]
    return z, qa


def _pack(wl, a):
    return bf16_bits(a) if wl.dtype == "bf16" else np.asarray(a, dtype=np.float64)


def episode_chunks(preset: str, overrides: dict, episode: int, chunks: int):
    """Dense chunk 0, then refresh chunks 1..chunks-1 with the oracle's own
    selection, yielded one chunk at a time.  Chunk t gives a dict with the
    cache after the chunk (K, V [L, N, d]), the layer outputs X [L, rows, d]
    (rows in idx order), the reference embeddings and the ages, and for
    t >= 1 also the pre-chunk ages and reference embeddings, the score, P, U,
    idx and k_eff."""
    wl = W.preset(preset, **overrides)
    weights = W.make_weights(wl)
    z, qa = episode_inputs(wl, episode, chunks)
    prec = O.Precision(wl.dtype)
    st, outs = O.dense_prefill(z[0], weights, wl.n_heads, wl.ln_eps, prec)
    st.age = np.asarray(W.make_initial_ages(wl, episode), dtype=np.int64)
    yield dict(K=_pack(wl, st.K), V=_pack(wl, st.V), X=np.stack(outs).astype(np.float32),
               zref=_pack(wl, st.zref), age=st.age.copy())
    del outs
    for t in range(1, chunks):
        age_before, zref_before = st.age.copy(), _pack(wl, st.zref)
        res = O.refresh_chunk(st, z[t], qa[t], weights, wl.k, wl.age_bound, wl.n_heads, wl.ln_eps,
                              wl.w_attn, wl.w_surprise, prec)
        yield dict(K=_pack(wl, st.K), V=_pack(wl, st.V), X=np.stack(res.outs).astype(np.float32),
                   zref=_pack(wl, st.zref), age=st.age.copy(), age_before=age_before, zref_before=zref_before,
                   score=res.score, P=np.asarray(res.mass, dtype=np.float64),
                   U=np.asarray(res.surprise, dtype=np.float64), idx=res.idx, k_eff=res.k_eff)


def episode_rollout(preset: str, overrides: dict, episode: int, chunks: int, threads: int = 0):
    """All chunks of episode_chunks as a list, with the BLAS threads of this
    process limited to `threads` (0: no limit)."""
    if threads:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(threads):
            return list(episode_chunks(preset, overrides, episode, chunks))
    return list(episode_chunks(preset, overrides, episode, chunks))


def host_threads() -> int:
    """CPU threads this process may use (at most 16, the GPU machine's share)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def episodes_in_parallel(preset: str, overrides: dict, episodes, chunks: int):
    """episode_rollout for each episode, in spawned worker processes that
    split the host threads between them."""
    episodes = list(episodes)
    workers = max(1, min(len(episodes), host_threads()))
    threads = max(1, host_threads() // workers)
    ctx = multiprocessing.get_context("spawn")
    with ProcessPoolExecutor(max_workers=workers, mp_context=ctx) as pool:
        futs = [pool.submit(episode_rollout, preset, overrides, e, chunks, threads) for e in episodes]
        return [f.result() for f in futs]
