"""The seeded input generators: deterministic, correctly shaped, bf16
workloads exactly bf16-representable, static background with local motion."""
import numpy as np
import pytest

from sparse_kv_refresh_amd import inputs as W


def test_deterministic_bytes():
    wl = W.preset("t_bf16_small")
    a, b = W.make_rollout(wl), W.make_rollout(wl)
    assert all(np.array_equal(x.w_qkv, y.w_qkv) and np.array_equal(x.mod, y.mod) for x, y in zip(a.weights, b.weights))
    assert all(np.array_equal(x, y) for x, y in zip(a.z[0], b.z[0]))
    assert all(np.array_equal(x, y) for x, y in zip(a.qa[0][1:], b.qa[0][1:]))


@pytest.mark.parametrize("name", ["t_bf16_small", "t_bf16_batch", "c1_tiny", "t_fp32_ragged"])
def test_shapes_and_representable(name):
    wl = W.preset(name)
    r = W.make_rollout(wl)
    d, F, L, N = wl.d_model, wl.d_ffn, wl.n_layers, wl.n_tokens
    w = r.weights[0]
    assert w.w_qkv.shape == (3 * d, d) and w.w_2.shape == (d, F) and w.mod.shape == (6, d)
    assert len(r.weights) == L and len(r.z) == wl.batch
    assert r.z[0][0].shape == (N, d) and r.qa[0][1].shape == (L, wl.n_action, d)
    if wl.dtype == "bf16":
        for arr in (w.w_qkv, w.b_1, r.z[0][1], r.qa[0][1]):
            assert np.array_equal(W.to_bf16_values(arr), arr)


def test_motion_is_local():
    for name in ("c1_tiny", "t_bf16_small"):
        wl = W.preset(name)
        src = W.LatentSource(wl)
        a, b = src.latent(1), src.latent(2)
        changed = np.any(a != b, axis=-1).mean()
        assert 0 < changed < 0.25


def test_patch_drift_region():
    wl = W.preset("c2_layer")
    src = W.LatentSource(wl)
    changed = np.any(src.latent(0) != src.latent(1), axis=-1)
    assert changed.sum() == 400        # rows 22-41 x cols 22-41


def test_episodes_differ():
    wl = W.preset("t_bf16_batch")
    r = W.make_rollout(wl)
    assert not np.array_equal(r.z[0][1], r.z[1][1])


def test_initial_ages():
    wl = W.preset("c2_layer")
    a = W.make_initial_ages(wl)
    assert a.min() == 0 and a.max() == wl.age_bound and a.dtype == np.int32
    assert 0.15 < (a >= wl.age_bound).mean() < 0.35
