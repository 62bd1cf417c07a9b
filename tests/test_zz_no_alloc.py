"""wamc_prefill_chunk_noalloc (the chunk with its workspace in the library's
static scratch) against wamc_prefill_chunk with a caller workspace, through
the C ABI: two calls in a row on one GPU, the second with a smaller chunk, so
the second starts from the first call's leftovers in the scratch.  Both
entry points run the same kernels with fixed-order reductions, so every
output must agree bitwise."""
import numpy as np
import pytest
import torch

from sparse_kv_refresh_amd import inputs as W
from sparse_kv_refresh_amd import wamc

from gpu_util import DEV, act, to_dev

pytestmark = pytest.mark.gpu


def _state(wl, r, dims, weights, larr):
    """A state after the dense chunk: caches, references and ages."""
    B, L, N, d = wl.batch, wl.n_layers, wl.n_tokens, wl.d_model
    adt = act(wl)
    k_cache = torch.zeros((L, B, N, d), dtype=adt, device=DEV)
    v_cache = torch.zeros_like(k_cache)
    zref = torch.zeros((B, N, d), dtype=adt, device=DEV)
    age = torch.zeros((B, N), dtype=torch.int32, device=DEV)
    ws = torch.empty(wamc.workspace_bytes(dims, N), dtype=torch.uint8, device=DEV)
    z0 = to_dev(np.stack([r.z[e][0] for e in range(B)]), adt)
    wamc.dense_prefill(dims, weights, z0, zref, k_cache, v_cache, age, ws, _layer_array=larr)
    age.copy_(to_dev(np.stack(r.ages0)))
    return dict(k_cache=k_cache, v_cache=v_cache, zref=zref, age=age)


def _chunk(wl, r, dims, weights, larr, state, rows_cap, noalloc):
    B, L, N, d = wl.batch, wl.n_layers, wl.n_tokens, wl.d_model
    adt = act(wl)
    st = {k: v.clone() for k, v in state.items()}
    z1 = to_dev(np.stack([r.z[e][1] for e in range(B)]), adt)
    qa = to_dev(np.stack([r.qa[e][1] for e in range(B)], axis=1), adt)
    idx = torch.full((B, N), -7, dtype=torch.int32, device=DEV)
    k_eff = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    score = torch.full((B, N), float("nan"), dtype=torch.float32, device=DEV)
    lo = torch.full((L, B, rows_cap, d), float("nan"), dtype=torch.float32, device=DEV)
    if noalloc:
        wamc.prefill_chunk_noalloc(dims, weights, z1, st["zref"], qa, st["k_cache"], st["v_cache"], st["age"], wl.k,
                                   idx, k_eff, rows_cap, score_out=score, layer_out=lo, _layer_array=larr)
    else:
        ws = torch.empty(wamc.workspace_bytes(dims, rows_cap), dtype=torch.uint8, device=DEV)
        wamc.prefill_chunk(dims, weights, z1, st["zref"], qa, st["k_cache"], st["v_cache"], st["age"], wl.k, idx,
                           k_eff, rows_cap, ws, score_out=score, layer_out=lo, _layer_array=larr)
    torch.cuda.synchronize()
    st.update(idx=idx, k_eff=k_eff, score=score)
    keff = k_eff.cpu().numpy()
    # layer outputs: only the k_eff rows of each episode are defined
    st["layer_out"] = [lo[:, b, :int(keff[b])].clone() for b in range(B)]
    return st


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_matches_workspace_entry_point(order):
    cases = [W.preset("t_bf16_batch"), W.preset("t_bf16_small", rows=10, cols=31, k=160)]
    assert cases[1].n_tokens < cases[0].n_tokens
    for wl in cases:
        print(f"noalloc case {wl.name} B={wl.batch} N={wl.n_tokens} k={wl.k}", flush=True)
        r = W.make_rollout(wl, chunks=2)
        dims = wamc.dims_for(wl)
        assert wamc.workspace_bytes(dims, wl.n_tokens) <= wamc.noalloc_scratch_bytes()
        weights = wamc.Engine.upload_weights(r.weights, act(wl), DEV)
        larr = wamc._layers(weights)
        state = _state(wl, r, dims, weights, larr)
        torch.cuda.synchronize()
        rows_cap = wl.n_tokens
        want = _chunk(wl, r, dims, weights, larr, state, rows_cap, noalloc=False)
        got = _chunk(wl, r, dims, weights, larr, state, rows_cap, noalloc=True)
        for name in ("k_eff", "idx", "age", "zref", "k_cache", "v_cache", "score"):
            assert torch.equal(got[name], want[name]), f"{wl.name}: {name} differs"
        for b in range(wl.batch):
            assert torch.equal(got["layer_out"][b], want["layer_out"][b]), f"{wl.name}: layer outputs, episode {b}"
        assert (want["k_eff"] > 0).all()
