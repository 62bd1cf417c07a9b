"""GPU token scores against the oracle (WAM-Cache §1, §4.2, §4.3): attention
mass P over the current cache, latent surprise U, and the combined score,
on caches produced by the oracle's dense prefill."""
import numpy as np
import pytest
import torch

from oracle import wamc_oracle as O
from sparse_kv_refresh_amd import inputs as W
from sparse_kv_refresh_amd import wamc

from gpu_util import DEV, act, batch_q, batch_z, max_rel, to_dev, to_np

pytestmark = pytest.mark.gpu


def _setup(name, **over):
    wl = W.preset(name, **over)
    r = W.make_rollout(wl, chunks=2)
    prec = O.Precision(wl.dtype)
    states = [O.dense_prefill(r.z[e][0], r.weights, wl.n_heads, wl.ln_eps, prec)[0] for e in range(wl.batch)]
    K = to_dev(np.stack([s.K.astype(np.float32) for s in states], axis=1), act(wl))      # [L, B, N, d]
    zref = to_dev(np.stack([s.zref.astype(np.float32) for s in states]), act(wl))
    return wl, r, prec, states, K, zref


@pytest.mark.parametrize("name,over", [("c1_tiny", {}), ("t_fp32_ragged", {}), ("t_bf16_small", {}),
                                       ("t_bf16_batch", {}),
                                       # action-query counts: one, ragged, the 128 maximum, fp32 past one tile
                                       ("t_bf16_small", {"n_action": 1}), ("t_bf16_small", {"n_action": 7}),
                                       ("t_bf16_batch", {"n_action": 128}), ("t_fp32_ragged", {"n_action": 130})])
def test_score_parity(name, over):
    wl, r, prec, states, K, zref = _setup(name, **over)
    dims = wamc.dims_for(wl)
    B, N = wl.batch, wl.n_tokens
    z1, qa = batch_z(wl, r, 1), batch_q(wl, r, 1)
    ws = torch.empty(wamc.workspace_bytes(dims, 0), dtype=torch.uint8, device=DEV)
    score = torch.empty((B, N), dtype=torch.float32, device=DEV)
    P = torch.empty_like(score)
    U = torch.empty_like(score)
    wamc.score(dims, z1, zref, qa, K, score, ws, mass_out=P, surprise_out=U)
    torch.cuda.synchronize()
    for b in range(B):
        s_o, P_o, U_o = O.score(r.z[b][1], states[b].zref, r.qa[b][1], states[b].K, wl.n_heads,
                                wl.w_attn, wl.w_surprise, prec)
        assert max_rel(to_np(P[b]), P_o) < 1e-4
        assert max_rel(to_np(U[b]), U_o) < 1e-5
        assert max_rel(to_np(score[b]), s_o) < 1e-4
        assert abs(float(P[b].sum()) - wl.n_layers * wl.n_heads * wl.n_action) < 1e-3 * N


def test_score_with_supplied_mass():
    wl, r, prec, states, K, zref = _setup("t_bf16_small")
    dims = wamc.dims_for(wl)
    N = wl.n_tokens
    rng = np.random.default_rng(1)
    mass = rng.random((1, N)).astype(np.float32)
    z1 = batch_z(wl, r, 1)
    ws = torch.empty(wamc.workspace_bytes(dims, 0), dtype=torch.uint8, device=DEV)
    score = torch.empty((1, N), dtype=torch.float32, device=DEV)
    wamc.score(dims, z1, zref, None, None, score, ws, mass_in=to_dev(mass))
    s_o, _, _ = O.score(r.z[0][1], states[0].zref, None, states[0].K, wl.n_heads, wl.w_attn, wl.w_surprise,
                        prec, mass=mass[0], n_action=wl.n_action)
    assert max_rel(to_np(score[0]), s_o) < 1e-5


def test_static_frame_scores_mass_only():
    """Nothing moved: the surprise term vanishes and the score is w_a P/(LHA)."""
    wl, r, prec, states, K, zref = _setup("t_bf16_small")
    dims = wamc.dims_for(wl)
    N = wl.n_tokens
    ws = torch.empty(wamc.workspace_bytes(dims, 0), dtype=torch.uint8, device=DEV)
    score = torch.empty((1, N), dtype=torch.float32, device=DEV)
    P = torch.empty_like(score)
    U = torch.empty_like(score)
    wamc.score(dims, zref, zref, batch_q(wl, r, 1), K, score, ws, mass_out=P, surprise_out=U)
    torch.cuda.synchronize()
    assert (U == 0).all()
    norm = wl.n_layers * wl.n_heads * wl.n_action
    assert max_rel(to_np(score), wl.w_attn * to_np(P) / norm) < 1e-6
