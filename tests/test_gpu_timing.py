"""The optional per-kernel timer (wamc_timing_*).  Timed launches carry HIP
events stamped with the kernel's own start and end, so: the chunk's state is
bitwise the same with timing on and off; every kernel of a refresh chunk is
recorded once per launch; the kernels of one stream never sum to more than
the span around them; and a chunk on a caller-given refresh set records its
multi-kernel age update as one entry."""
import numpy as np
import pytest
import torch

from sparse_kv_refresh_amd import inputs as W
from sparse_kv_refresh_amd import wamc

from gpu_util import DEV, batch_q, batch_z, engine, to_dev

pytestmark = pytest.mark.gpu


def _state(eng):
    return {n: t.clone() for n, t in (("k", eng.k_cache), ("v", eng.v_cache), ("zref", eng.zref),
                                      ("age", eng.age), ("idx", eng.idx), ("k_eff", eng.k_eff))}


def test_timed_chunk_bitwise_and_counts():
    wl = W.preset("t_bf16_small")
    r = W.make_rollout(wl, chunks=2)
    eng = engine(wl, r)
    L = wl.n_layers
    eng.dense(batch_z(wl, r, 0))
    eng.age.copy_(to_dev(np.stack(r.ages0)))
    z1, q1 = batch_z(wl, r, 1), batch_q(wl, r, 1)
    torch.cuda.synchronize()
    snap = eng.snapshot()

    eng.chunk(z1, q1, wl.k)
    torch.cuda.synchronize()
    want = _state(eng)

    eng.restore(snap)
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wamc.timing_enable(True)
    try:
        a.record(s)
        eng.chunk(z1, q1, wl.k, stream=s)
        b.record(s)
        torch.cuda.synchronize()
        kt = wamc.timing_read()
    finally:
        wamc.timing_enable(False)
    got = _state(eng)
    for n in want:
        assert torch.equal(got[n], want[n]), n

    expect = {"score_pass1": 1, "score_pass2": 1, "score_combine": 1, "select": 1, "gather_ln": 1,
              "gemm_qkv": L, "attention": L, "gemm_out_resid": L, "ln_mod": 2 * L - 1,
              "gemm_up_gelu": L, "gemm_down_resid": L}
    assert set(kt) == set(expect), sorted(kt)
    for kind, n in expect.items():
        launches, ms = kt[kind]
        assert launches == n, (kind, launches, n)
        assert ms > 0.0, kind
    span = a.elapsed_time(b)
    total = sum(ms for _, ms in kt.values())
    assert total <= span * 1.02 + 0.005, (total, span)


def test_timed_override_ages_entry():
    wl = W.preset("t_bf16_small")
    r = W.make_rollout(wl, chunks=2)
    eng = engine(wl, r)
    N = wl.n_tokens
    eng.dense(batch_z(wl, r, 0))
    torch.cuda.synchronize()
    rows = np.arange(0, N, 3, dtype=np.int32)
    idx = np.full((1, N), -1, dtype=np.int32)
    idx[0, :rows.size] = rows
    wamc.timing_enable(True)
    try:
        eng.chunk(batch_z(wl, r, 1), batch_q(wl, r, 1), 0, idx_override=to_dev(idx),
                  k_eff_override=to_dev(np.array([rows.size], dtype=np.int32)))
        torch.cuda.synchronize()
        kt = wamc.timing_read()
    finally:
        wamc.timing_enable(False)
    assert kt["ages_from_set"][0] == 1 and kt["ages_from_set"][1] > 0.0
    assert "select" not in kt and "score_pass1" not in kt
    assert kt["attention"][0] == wl.n_layers
    age = eng.age.cpu().numpy()[0]
    assert (age[rows] == 0).all() and (np.delete(age, rows) == 1).all()
