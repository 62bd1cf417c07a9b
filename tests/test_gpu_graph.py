"""A whole refresh chunk and a dense prefill captured in a HIP graph and
replayed: every replay (with eager work and state restores between replays)
is bitwise equal to the eager call on the same state.  Graph replay removes
the per-launch host cost that dominates at small token counts (WAM-Cache
§5.2 "CUDA latency": at the native 120 tokens weight loading and graph replay
take a fixed share of each layer)."""
import numpy as np
import pytest
import torch

from sparse_kv_refresh_amd import inputs as W

from gpu_util import DEV, batch_q, batch_z, engine, to_dev

pytestmark = pytest.mark.gpu


# the d=1536 stack at 120 tokens: its projections take the split-K path with
# a separate reduction and the fused LayerNorms
SMALL_STACK = dict(n_layers=2, views=1, rows=12, cols=10, k=70, age_bound=2, chunks=3)


@pytest.mark.parametrize("name,rule,over", [("t_bf16_small", "fixed", {}), ("t_bf16_batch", "fixed", {}),
                                            ("t_bf16_small", "union", {}), ("c3_stack", "fixed", SMALL_STACK)])
def test_chunk_graph_replay_bitwise(name, rule, over):
    wl = W.preset(name, **over)
    r = W.make_rollout(wl, chunks=3)
    eng = engine(wl, r)
    L, B, N, d = wl.n_layers, wl.batch, wl.n_tokens, wl.d_model
    eng.dense(batch_z(wl, r, 0))
    eng.age.copy_(to_dev(np.stack(r.ages0)))
    z1, q1 = batch_z(wl, r, 1), batch_q(wl, r, 1)
    lo = torch.zeros((L, B, N, d), dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    snap = eng.snapshot()

    def step():
        if rule == "fixed":
            eng.chunk(z1, q1, wl.k, layer_out=lo)
        else:
            eng.chunk_union(z1, q1, 2 * wl.k // 3, wl.k // 3, layer_out=lo)

    # eager reference
    step()
    torch.cuda.synchronize()
    want = {n: t.clone() for n, t in (("k", eng.k_cache), ("v", eng.v_cache), ("zref", eng.zref), ("age", eng.age),
                                      ("idx", eng.idx), ("k_eff", eng.k_eff), ("lo", lo))}
    # capture on a side stream (warm-up call first, as graph capture requires)
    eng.restore(snap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eng.restore(snap)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        eng.restore(snap)
        lo.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = {"k": eng.k_cache, "v": eng.v_cache, "zref": eng.zref, "age": eng.age, "idx": eng.idx,
               "k_eff": eng.k_eff, "lo": lo}
        for n in want:
            assert torch.equal(got[n], want[n]), f"replay {rep}: {n} differs"
        # eager work between replays
        eng.dense(batch_z(wl, r, 2))
        torch.cuda.synchronize()


def test_dense_graph_replay_bitwise():
    wl = W.preset("t_bf16_small")
    r = W.make_rollout(wl, chunks=2)
    eng = engine(wl, r)
    z = batch_z(wl, r, 1)
    eng.dense(z)
    torch.cuda.synchronize()
    want = (eng.k_cache.clone(), eng.v_cache.clone())
    eng.k_cache.zero_()
    eng.v_cache.zero_()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        eng.dense(z)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        eng.dense(z)
    for _ in range(3):
        eng.k_cache.zero_()
        eng.v_cache.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(eng.k_cache, want[0]) and torch.equal(eng.v_cache, want[1])
