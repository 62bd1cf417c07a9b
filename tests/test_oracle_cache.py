"""Pins of the oracle's chunk semantics: scoring, cache updates and rollouts.

* Full refresh equals dense computation bitwise (RealtimeWAM App. D.2 states
  this for its engine; here k = N from any stale state must give exactly the
  dense prefill of the new frame).
* k = 0 from ages below the bound leaves K, V and the reference embeddings
  untouched and ages every token by one.
* A static frame is a fixed point: reusing any subset reproduces the cache.
* Permuting tokens permutes every output (the block has no positional term).
* Attention mass sums to L*H*A; identical keys spread it evenly; surprise is
  zero on tokens that did not move (WAM-Cache §4.2, §4.3).
* Over rollouts no age exceeds the bound and forced tokens are always
  refreshed (WAM-Cache §4.4).
* Cost model: refresh/dense FLOPs = k_eff/N, which reproduces the pages'
  arithmetic 1 - 0.584 = 41.6 % and 1/0.584 = 1.71 (WAM-Cache §5.2, §5.3).
"""
import json
import os

import numpy as np
import pytest

from oracle import wamc_oracle as O
from sparse_kv_refresh_amd import inputs as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _setup(name="t_fp32_ragged", **kw):
    wl = W.preset(name, **kw)
    r = W.make_rollout(wl, chunks=min(wl.chunks, 4))
    return wl, r, O.Precision(wl.dtype)


def _chunk(wl, st, r, t, prec, k=None, idx=None, e=0):
    return O.refresh_chunk(st, r.z[e][t], r.qa[e][t], r.weights, wl.k if k is None else k, wl.age_bound,
                           wl.n_heads, wl.ln_eps, wl.w_attn, wl.w_surprise, prec, idx_override=idx)


@pytest.mark.parametrize("name", ["t_fp32_ragged", "t_bf16_small"])
def test_full_refresh_equals_dense_bitwise(name):
    wl, r, prec = _setup(name)
    st, _ = O.dense_prefill(r.z[0][0], r.weights, wl.n_heads, wl.ln_eps, prec)
    _chunk(wl, st, r, 1, prec)                       # make the cache stale
    st.age[:] = 0
    res = _chunk(wl, st, r, 2, prec, k=wl.n_tokens)
    ref, outs = O.dense_prefill(r.z[0][2], r.weights, wl.n_heads, wl.ln_eps, prec)
    assert res.k_eff == wl.n_tokens
    assert np.array_equal(st.K, ref.K) and np.array_equal(st.V, ref.V)
    assert all(np.array_equal(a, b) for a, b in zip(res.outs, outs))
    assert np.array_equal(st.zref, ref.zref) and (st.age == 0).all()


def test_zero_refresh_keeps_cache():
    wl, r, prec = _setup()
    st, _ = O.dense_prefill(r.z[0][0], r.weights, wl.n_heads, wl.ln_eps, prec)
    before = st.copy()
    res = _chunk(wl, st, r, 1, prec, k=0)
    assert res.k_eff == 0 and len(res.idx) == 0
    assert np.array_equal(st.K, before.K) and np.array_equal(st.V, before.V)
    assert np.array_equal(st.zref, before.zref)
    assert (st.age == before.age + 1).all()


def test_static_frame_fixed_point():
    wl, r, prec = _setup()
    z0 = r.z[0][0]
    st, _ = O.dense_prefill(z0, r.weights, wl.n_heads, wl.ln_eps, prec)
    before = st.copy()
    rng = np.random.default_rng(5)
    for m in (1, 37, wl.n_tokens - 1):
        idx = np.sort(rng.choice(wl.n_tokens, size=m, replace=False))
        O.refresh_chunk(st, z0, r.qa[0][1], r.weights, m, wl.age_bound, wl.n_heads, wl.ln_eps,
                        wl.w_attn, wl.w_surprise, prec, idx_override=idx)
        scale = np.abs(before.K).max()
        assert np.abs(st.K - before.K).max() <= 1e-12 * scale
        assert np.abs(st.V - before.V).max() <= 1e-12 * np.abs(before.V).max()


def test_permutation_equivariance():
    wl, r, prec = _setup()
    N = wl.n_tokens
    perm = np.random.default_rng(9).permutation(N)
    inv = np.argsort(perm)
    z0, z1 = r.z[0][0], r.z[0][1]
    st, _ = O.dense_prefill(z0, r.weights, wl.n_heads, wl.ln_eps, prec)
    stp, _ = O.dense_prefill(z0[perm], r.weights, wl.n_heads, wl.ln_eps, prec)
    assert np.allclose(stp.K, st.K[:, perm], rtol=1e-12, atol=1e-13)
    res = _chunk(wl, st, r, 1, prec)
    idx_p = np.sort(inv[res.idx])
    resp = O.refresh_chunk(stp, z1[perm], r.qa[0][1], r.weights, wl.k, wl.age_bound, wl.n_heads, wl.ln_eps,
                           wl.w_attn, wl.w_surprise, prec, idx_override=idx_p)
    assert np.allclose(resp.score, res.score[perm], rtol=1e-6)
    assert np.allclose(stp.K, st.K[:, perm], rtol=1e-11, atol=1e-12)
    assert np.allclose(stp.V, st.V[:, perm], rtol=1e-11, atol=1e-12)
    # rows of the layer outputs are in ascending token order on both sides
    order = np.argsort(perm[idx_p])
    assert np.allclose(resp.outs[-1][order], res.outs[-1], rtol=1e-11, atol=1e-12)


def test_score_invariants():
    wl, r, prec = _setup()
    st, _ = O.dense_prefill(r.z[0][0], r.weights, wl.n_heads, wl.ln_eps, prec)
    s, P, U = O.score(r.z[0][1], st.zref, r.qa[0][1], st.K, wl.n_heads, wl.w_attn, wl.w_surprise, prec)
    L, H, A = wl.n_layers, wl.n_heads, wl.n_action
    assert abs(P.sum() - L * H * A) <= 1e-10 * L * H * A
    moved = np.any(r.z[0][1] != r.z[0][0], axis=1)
    assert moved.any() and (U[~moved] == 0).all() and (U[moved] > 0).all()
    assert abs(float(s.sum()) - (wl.w_attn + wl.w_surprise)) < 1e-5
    # identical keys: uniform mass
    Kflat = np.repeat(st.K[:, :1], wl.n_tokens, axis=1)
    P2 = O.attention_mass(r.qa[0][1], Kflat, wl.n_heads, prec)
    assert np.allclose(P2, L * H * A / wl.n_tokens, rtol=1e-12)
    # nothing moved: the surprise term vanishes
    s3, _, U3 = O.score(r.z[0][0], st.zref, r.qa[0][1], st.K, wl.n_heads, wl.w_attn, wl.w_surprise, prec)
    assert (U3 == 0).all()
    assert np.allclose(s3, wl.w_attn * P / (L * H * A), rtol=1e-6)


def test_mass_against_loop_formulation():
    """P written as an explicit loop over (layer, head, query) with
    scalar-free numpy rows -- a second formulation on small shapes."""
    rng = np.random.default_rng(4)
    L, N, H, dh, A = 2, 9, 3, 4, 5
    K = rng.standard_normal((L, N, H * dh))
    qa = rng.standard_normal((L, A, H * dh))
    want = np.zeros(N)
    for l in range(L):
        for h in range(H):
            for a in range(A):
                s = np.array([qa[l, a, h * dh:(h + 1) * dh] @ K[l, j, h * dh:(h + 1) * dh] for j in range(N)]) / np.sqrt(dh)
                e = np.exp(s - s.max())
                want += e / e.sum()
    got = O.attention_mass(qa, K, H, O.Precision("fp32"))
    assert np.allclose(got, want, rtol=1e-12)


@pytest.mark.parametrize("name", ["c1_tiny", "t_fp32_ragged", "t_bf16_batch"])
def test_rollout_age_invariants(name):
    wl = W.preset(name)
    r = W.make_rollout(wl)
    prec = O.Precision(wl.dtype)
    saw_overflow = False
    for e in range(wl.batch):
        st, _ = O.dense_prefill(r.z[e][0], r.weights, wl.n_heads, wl.ln_eps, prec)
        st.age = r.ages0[e].astype(np.int64)
        for t in range(1, wl.chunks):
            forced = np.nonzero(st.age >= wl.age_bound)[0]
            res = _chunk(wl, st, r, t, prec, e=e)
            assert set(forced.tolist()) <= set(res.idx.tolist())
            assert res.k_eff == max(wl.k, len(forced)) == len(res.idx)
            assert st.age.max() <= wl.age_bound
            saw_overflow |= res.k_eff > wl.k
            assert np.array_equal(st.zref[res.idx], prec.load(r.z[e][t])[res.idx])
    if name == "c1_tiny":
        assert saw_overflow     # k < N - k: the age bound forces extra tokens


def test_cost_model_against_pages():
    with open(os.path.join(GOLDEN, "cost_model.json")) as f:
        g = json.load(f)
    N, L, d, F = 4680, 30, 1536, 8960
    for k in (0, 468, 2808, 4680):
        assert O.prefill_flops(k, N, L, d, F) * N == O.prefill_flops(N, N, L, d, F) * k
    rho = g["rho_bar"]
    assert round(100 * (1 - rho), 1) == g["flop_cut_percent"]
    assert round(1 / rho, 2) == g["speedup_bound"]
    assert round(100 * g["measured_speedup_largest_context"] / g["speedup_bound"]) == g["attainment_percent"]
    assert abs(g["refreshed_tokens_approx"] / g["native_tokens"] - rho) < 0.01
    # per-chunk FLOPs of the 30-layer stack: dense 14.416 TF, 60 % refresh 8.650 TF
    assert abs(O.prefill_flops(N, N, L, d, F) / 1e12 - 14.416) < 1e-3
    assert abs(O.prefill_flops(2808, N, L, d, F) / 1e12 - 8.650) < 1e-3


def test_supplied_mass_matches_computed_mass():
    """An action expert that supplies exactly the attention mass the oracle
    would compute must get exactly the same scores (same L*H*A normaliser)."""
    wl, r, prec = _setup()
    st, _ = O.dense_prefill(r.z[0][0], r.weights, wl.n_heads, wl.ln_eps, prec)
    s, P, U = O.score(r.z[0][1], st.zref, r.qa[0][1], st.K, wl.n_heads, wl.w_attn, wl.w_surprise, prec)
    s2, _, _ = O.score(r.z[0][1], st.zref, None, st.K, wl.n_heads, wl.w_attn, wl.w_surprise, prec,
                       mass=P, n_action=wl.n_action)
    assert np.array_equal(s, s2)
    with pytest.raises(ValueError):
        O.score(r.z[0][1], st.zref, None, st.K, wl.n_heads, wl.w_attn, wl.w_surprise, prec, mass=P)


def test_union_rule_chunk():
    """The union rule inside a chunk: the refresh set is the union of the
    mass and surprise top sets and the forced tokens of the chunk's own P and
    U; a budget covering every token equals the dense prefill bitwise."""
    wl, r, prec = _setup()
    N = wl.n_tokens
    st, _ = O.dense_prefill(r.z[0][0], r.weights, wl.n_heads, wl.ln_eps, prec)
    st.age = r.ages0[0].astype(np.int64) + 1
    age0 = st.age.copy()
    na, ns = O.budget_count(0.4, N), O.budget_count(0.1, N)
    res = O.refresh_chunk(st, r.z[0][1], r.qa[0][1], r.weights, 0, wl.age_bound, wl.n_heads, wl.ln_eps,
                          wl.w_attn, wl.w_surprise, prec, union=(na, ns))
    want = set(O.top_by(res.mass.astype(np.float32), na).tolist()) | \
        set(O.top_by(res.surprise.astype(np.float32), ns).tolist()) | set(np.flatnonzero(age0 >= wl.age_bound).tolist())
    assert res.idx.tolist() == sorted(want) and res.k_eff == len(want)
    assert (st.age <= wl.age_bound).all()
    # budgets covering every token: the dense prefill of the new frame, bitwise
    res = O.refresh_chunk(st, r.z[0][2], r.qa[0][2], r.weights, 0, wl.age_bound, wl.n_heads, wl.ln_eps,
                          wl.w_attn, wl.w_surprise, prec, union=(N, 0))
    ref, outs = O.dense_prefill(r.z[0][2], r.weights, wl.n_heads, wl.ln_eps, prec)
    assert res.k_eff == N
    assert np.array_equal(st.K, ref.K) and np.array_equal(st.V, ref.V)
    assert all(np.array_equal(a, b) for a, b in zip(res.outs, outs))


@pytest.mark.parametrize("name", ["t_fp32_text", "t_bf16_text"])
def test_text_cross_attention_chunks(name):
    """With the text cross-attention: k = N from a stale state equals the
    dense prefill bitwise, and k = 0 leaves the cache untouched (the text
    keys/values are the episode's, computed once at the dense chunk)."""
    wl, r, prec = _setup(name)
    st, _ = O.dense_prefill(r.z[0][0], r.weights, wl.n_heads, wl.ln_eps, prec, text_emb=r.text[0])
    assert st.text is not None and len(st.text) == wl.n_layers
    _chunk(wl, st, r, 1, prec)
    st.age[:] = 0
    before = st.copy()
    res = _chunk(wl, st, r, 2, prec, k=0)
    assert res.k_eff == 0 and np.array_equal(st.K, before.K) and np.array_equal(st.V, before.V)
    st.age[:] = 0
    res = _chunk(wl, st, r, 2, prec, k=wl.n_tokens)
    ref, outs = O.dense_prefill(r.z[0][2], r.weights, wl.n_heads, wl.ln_eps, prec, text_emb=r.text[0])
    assert np.array_equal(st.K, ref.K) and np.array_equal(st.V, ref.V)
    assert all(np.array_equal(a, b) for a, b in zip(res.outs, outs))
