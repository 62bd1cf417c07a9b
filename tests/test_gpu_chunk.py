"""Whole refresh chunks on the GPU against the oracle (WAM-Cache §4.1-§4.4).

* Rollouts driven by the oracle-chosen refresh set (idx_override): K/V cache,
  every layer's output rows, ages and reference embeddings per chunk.
* Rollouts with the library's own selection: the selected set is exactly the
  oracle's selection applied to the GPU's scores, ages never exceed the bound.
* Invariants on the GPU: k = N equals the dense prefill bitwise; k = 0 from
  ages below the bound leaves the cache bitwise unchanged; a chunk replayed
  from a snapshot is bitwise identical (fixed-order reductions).
* The single-layer d=1536 workload at full size (N=4096, k=2458), in the
  launch configuration the benchmark times, and a 4-layer slice of the
  30-layer d=1536 stack (N=4680, k=2808).
"""
import numpy as np
import pytest
import torch

from oracle import wamc_oracle as O
from sparse_kv_refresh_amd import inputs as W
from sparse_kv_refresh_amd import wamc

from gpu_util import DEV, act, batch_q, batch_z, close, engine, max_rel, to_dev, to_np

pytestmark = pytest.mark.gpu


def _oracle_states(wl, r, prec):
    out = []
    for e in range(wl.batch):
        st, _ = O.dense_prefill(r.z[e][0], r.weights, wl.n_heads, wl.ln_eps, prec,
                                text_emb=None if r.text is None else r.text[e])
        st.age = r.ages0[e].astype(np.int64)
        out.append(st)
    return out


def _compare_chunk(wl, eng, states, res, lo, t):
    for b in range(wl.batch):
        st, rs = states[b], res[b]
        ke = int(eng.k_eff[b])
        assert ke == rs.k_eff
        assert np.array_equal(to_np(eng.idx[b])[:ke], rs.idx)
        assert np.array_equal(to_np(eng.age[b]), st.age)
        assert np.array_equal(to_np(eng.zref[b]), st.zref.astype(np.float32))
        for l in range(wl.n_layers):
            for nm, g, o in (("K", to_np(eng.k_cache[l, b]), st.K[l]), ("V", to_np(eng.v_cache[l, b]), st.V[l]),
                             ("X", to_np(lo[l, b, :ke]), rs.outs[l])):
                ok, err = close(wl, g, o)
                assert ok, f"chunk {t} episode {b} layer {l} {nm}: error {err}"


def _run_override_rollout(wl, chunks):
    r = W.make_rollout(wl, chunks=chunks)
    prec = O.Precision(wl.dtype)
    states = _oracle_states(wl, r, prec)
    eng = engine(wl, r)
    L, B, N, d = wl.n_layers, wl.batch, wl.n_tokens, wl.d_model
    eng.dense(batch_z(wl, r, 0))
    eng.age.copy_(to_dev(np.stack(r.ages0)))
    lo = torch.zeros((L, B, eng.rows_cap, d), dtype=torch.float32, device=DEV)
    for t in range(1, chunks):
        res = [O.refresh_chunk(states[e], r.z[e][t], r.qa[e][t], r.weights, wl.k, wl.age_bound, wl.n_heads,
                               wl.ln_eps, wl.w_attn, wl.w_surprise, prec) for e in range(B)]
        ov = np.full((B, N), -1, dtype=np.int32)
        kk = np.zeros(B, dtype=np.int32)
        for e in range(B):
            ov[e, :res[e].k_eff] = res[e].idx
            kk[e] = res[e].k_eff
        eng.chunk(batch_z(wl, r, t), batch_q(wl, r, t), wl.k, idx_override=to_dev(ov), k_eff_override=to_dev(kk),
                  layer_out=lo)
        torch.cuda.synchronize()
        _compare_chunk(wl, eng, states, res, lo, t)


@pytest.mark.parametrize("name", ["c1_tiny", "t_fp32_ragged", "t_bf16_small", "t_bf16_batch", "t_bf16_text",
                                  "t_fp32_text"])
def test_rollout_oracle_refresh_set(name):
    wl = W.preset(name)
    _run_override_rollout(wl, wl.chunks)


def test_large_model_shapes_reduced_tokens():
    """The d=3072, 24-head, FFN 12288 layer with 128 action queries and two
    episodes, on a reduced 2x12x20 token grid (k = N/2, age bound 4)."""
    wl = W.preset("c5_large", n_layers=1, batch=2, rows=12, cols=20, k=240, chunks=3)
    _run_override_rollout(wl, wl.chunks)


def test_bench_workload_full_size():
    """d=1536, 12 heads, FFN 8960, N=4096, k=2458 (60 %), ages U{0..3} after
    the dense chunk: dense parity, then one refresh chunk with the oracle's
    refresh set; rows_cap = k as the benchmark runs it."""
    wl = W.preset("c2_layer")
    r = W.make_rollout(wl, chunks=2)
    prec = O.Precision(wl.dtype)
    states = _oracle_states(wl, r, prec)
    res = O.refresh_chunk(states[0], r.z[0][1], r.qa[0][1], r.weights, wl.k, wl.age_bound, wl.n_heads,
                          wl.ln_eps, wl.w_attn, wl.w_surprise, prec)
    assert res.k_eff == wl.k
    eng = engine(wl, r, rows_cap=wl.k)
    eng.dense(batch_z(wl, r, 0))
    eng.age.copy_(to_dev(np.stack(r.ages0)))
    lo = torch.zeros((1, 1, wl.k, wl.d_model), dtype=torch.float32, device=DEV)
    # the library's own selection, checked against the oracle's on the GPU scores
    age_before = to_np(eng.age[0]).copy()
    eng.chunk(batch_z(wl, r, 1), batch_q(wl, r, 1), wl.k, layer_out=lo)
    torch.cuda.synchronize()
    gscore = to_np(eng.score[0])
    assert max_rel(gscore, res.score) < 1e-4
    sel_idx, sel_k, sel_age, _ = O.select(gscore, age_before, wl.k, wl.age_bound, cap=wl.k)
    assert int(eng.k_eff[0]) == sel_k and np.array_equal(to_np(eng.idx[0])[:sel_k], sel_idx)
    assert np.array_equal(to_np(eng.age[0]), sel_age)
    if np.array_equal(sel_idx, res.idx):
        _compare_chunk(wl, eng, states, [res], lo, 1)
    # and driven by the oracle's refresh set
    eng2 = engine(wl, r, rows_cap=wl.k)
    eng2.dense(batch_z(wl, r, 0))
    eng2.age.copy_(to_dev(np.stack(r.ages0)))
    ov = np.full((1, wl.n_tokens), -1, dtype=np.int32)
    ov[0, :res.k_eff] = res.idx
    eng2.chunk(batch_z(wl, r, 1), batch_q(wl, r, 1), wl.k, idx_override=to_dev(ov),
               k_eff_override=to_dev(np.array([res.k_eff], dtype=np.int32)), layer_out=lo)
    torch.cuda.synchronize()
    _compare_chunk(wl, eng2, states, [res], lo, 1)


def test_large_tile_split_schedule():
    """c2 shapes with k = 3840 of N = 4096, the launch sized for every token
    (rows_cap = N) and the library's own selection: the MLP up projection
    takes 256x256 tiles (525 of them at 3840 rows: two full rounds of 256)
    with the 13-tile last round split along K.  The selection is checked
    against the oracle's rule on the GPU scores, the chunk against the oracle
    chunk on that refresh set."""
    wl = W.preset("c2_layer").with_(k=3840)
    r = W.make_rollout(wl, chunks=2)
    prec = O.Precision(wl.dtype)
    states = _oracle_states(wl, r, prec)
    eng = engine(wl, r)
    eng.dense(batch_z(wl, r, 0))
    eng.age.copy_(to_dev(np.stack(r.ages0)))
    lo = torch.zeros((1, 1, wl.n_tokens, wl.d_model), dtype=torch.float32, device=DEV)
    age_before = to_np(eng.age[0]).copy()
    eng.chunk(batch_z(wl, r, 1), batch_q(wl, r, 1), wl.k, layer_out=lo)
    torch.cuda.synchronize()
    sel_idx, sel_k, _, _ = O.select(to_np(eng.score[0]), age_before, wl.k, wl.age_bound, cap=wl.n_tokens)
    assert sel_k == wl.k, "fewer forced tokens than k: the 525-tile case"
    assert int(eng.k_eff[0]) == sel_k and np.array_equal(to_np(eng.idx[0])[:sel_k], sel_idx)
    res = O.refresh_chunk(states[0], r.z[0][1], r.qa[0][1], r.weights, wl.k, wl.age_bound, wl.n_heads,
                          wl.ln_eps, wl.w_attn, wl.w_surprise, prec, idx_override=sel_idx)
    _compare_chunk(wl, eng, states, [res], lo, 1)


def test_ffn_not_multiple_of_64():
    """FFN 520 (a multiple of 8, not of 64): the down projection's K takes the
    plain bf16 GEMM kernel instead of the direct-to-LDS ones; dense prefill
    and two refresh chunks on the oracle's sets."""
    _run_override_rollout(W.preset("t_bf16_small").with_(d_ffn=520), 3)


def test_stack_slice_d1536():
    _run_override_rollout(W.preset("t_bf16_stack"), 3)


@pytest.mark.parametrize("name", ["c1_tiny", "t_bf16_batch"])
def test_own_selection_rollout(name):
    wl = W.preset(name)
    r = W.make_rollout(wl)
    eng = engine(wl, r)
    eng.dense(batch_z(wl, r, 0))
    for t in range(1, wl.chunks):
        age_before = to_np(eng.age).copy()
        eng.chunk(batch_z(wl, r, t), batch_q(wl, r, t), wl.k)
        torch.cuda.synchronize()
        for b in range(wl.batch):
            idx, k_eff, age, _ = O.select(to_np(eng.score[b]), age_before[b], wl.k, wl.age_bound)
            assert int(eng.k_eff[b]) == k_eff
            assert np.array_equal(to_np(eng.idx[b])[:k_eff], idx)
            assert (to_np(eng.idx[b])[k_eff:] == -1).all()
            assert np.array_equal(to_np(eng.age[b]), age)
        assert int(eng.age.max()) <= wl.age_bound


@pytest.mark.parametrize("name", ["c1_tiny", "t_bf16_small", "t_bf16_text"])
def test_full_refresh_equals_dense_on_gpu(name):
    wl = W.preset(name)
    r = W.make_rollout(wl, chunks=3)
    eng = engine(wl, r)
    L, B, N, d = wl.n_layers, wl.batch, wl.n_tokens, wl.d_model
    eng.dense(batch_z(wl, r, 0))
    eng.chunk(batch_z(wl, r, 1), batch_q(wl, r, 1), wl.k)        # stale mixture
    eng.age.zero_()
    lo = torch.zeros((L, B, N, d), dtype=torch.float32, device=DEV)
    eng.chunk(batch_z(wl, r, 2), batch_q(wl, r, 2), N, layer_out=lo)
    ref = engine(wl, r)
    lo_ref = torch.zeros_like(lo)
    ref.dense(batch_z(wl, r, 2), layer_out=lo_ref)
    torch.cuda.synchronize()
    assert int(eng.k_eff[0]) == N
    assert torch.equal(eng.k_cache, ref.k_cache) and torch.equal(eng.v_cache, ref.v_cache)
    assert torch.equal(lo, lo_ref)
    assert torch.equal(eng.zref, ref.zref) and (eng.age == 0).all()


def test_zero_refresh_keeps_cache_on_gpu():
    wl = W.preset("t_bf16_small")
    r = W.make_rollout(wl, chunks=2)
    eng = engine(wl, r)
    eng.dense(batch_z(wl, r, 0))
    snap = eng.snapshot()
    eng.chunk(batch_z(wl, r, 1), batch_q(wl, r, 1), 0)
    torch.cuda.synchronize()
    assert int(eng.k_eff[0]) == 0
    assert torch.equal(eng.k_cache, snap["k_cache"]) and torch.equal(eng.v_cache, snap["v_cache"])
    assert torch.equal(eng.zref, snap["zref"])
    assert torch.equal(eng.age, snap["age"] + 1)


@pytest.mark.parametrize("name", ["c1_tiny", "t_bf16_batch"])
def test_replay_is_bitwise(name):
    wl = W.preset(name)
    r = W.make_rollout(wl, chunks=2)
    eng = engine(wl, r)
    eng.dense(batch_z(wl, r, 0))
    snap = eng.snapshot()
    outs = []
    for _ in range(2):
        eng.restore(snap)
        lo = torch.zeros((wl.n_layers, wl.batch, eng.rows_cap, wl.d_model), dtype=torch.float32, device=DEV)
        eng.chunk(batch_z(wl, r, 1), batch_q(wl, r, 1), wl.k, layer_out=lo)
        torch.cuda.synchronize()
        outs.append([lo.clone(), eng.k_cache.clone(), eng.v_cache.clone(), eng.score.clone(), eng.idx.clone()])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


@pytest.mark.parametrize("name", ["c1_tiny", "t_bf16_small", "t_bf16_batch"])
def test_union_rule_rollout(name):
    """Chunks with the union rule (WAM-Cache §1, §4.3, §4.4) at the pages'
    default budgets (b_a, b_s) = (0.4, 0.1): the library's set is exactly the
    oracle's union on the library's own mass and surprise, k_eff varies from
    chunk to chunk, and the rows, K/V cache and ages match the oracle run on
    the same sets."""
    wl = W.preset(name)
    r = W.make_rollout(wl)
    prec = O.Precision(wl.dtype)
    N, B = wl.n_tokens, wl.batch
    na, ns = O.budget_count(0.4, N), O.budget_count(0.1, N)
    eng = engine(wl, r)
    eng.dense(batch_z(wl, r, 0))
    states = [O.dense_prefill(r.z[e][0], r.weights, wl.n_heads, wl.ln_eps, prec)[0] for e in range(B)]
    lo = torch.zeros((wl.n_layers, B, N, wl.d_model), dtype=torch.float32, device=DEV)
    P = torch.empty((B, N), dtype=torch.float32, device=DEV)
    U = torch.empty_like(P)
    sc = torch.empty_like(P)
    keffs = []
    for t in range(1, wl.chunks):
        z, qa = batch_z(wl, r, t), batch_q(wl, r, t)
        age_before = to_np(eng.age).copy()
        wamc.score(eng.dims, z, eng.zref, qa, eng.k_cache, sc, eng.ws, mass_out=P, surprise_out=U)
        eng.chunk_union(z, qa, na, ns, layer_out=lo)
        torch.cuda.synchronize()
        res = []
        for b in range(B):
            idx, k_eff, age, _ = O.select_union(to_np(P[b]), to_np(U[b]), age_before[b], na, ns, wl.age_bound)
            assert int(eng.k_eff[b]) == k_eff
            assert np.array_equal(to_np(eng.idx[b])[:k_eff], idx)
            assert (to_np(eng.idx[b])[k_eff:] == -1).all()
            assert np.array_equal(to_np(eng.age[b]), age)
            keffs.append(k_eff)
            res.append(O.refresh_chunk(states[b], r.z[b][t], r.qa[b][t], r.weights, 0, wl.age_bound, wl.n_heads,
                                       wl.ln_eps, wl.w_attn, wl.w_surprise, prec, idx_override=idx))
        _compare_chunk(wl, eng, states, res, lo, t)
        assert int(eng.age.max()) <= wl.age_bound
    assert min(keffs) >= max(na, ns)


def test_capacity_filled_chunk():
    """A capacity-filled refresh (RealtimeWAM §3: the plateau's upper end is
    the execution capacity, filled with the next-ranked tokens): the chunk's
    latency is measured on the GPU from k upward, the fill count taken by the
    capacity policy, and the chunk at that count compared with the oracle on
    the same refresh set; then the same at a fixed ragged fill (k + 56)."""
    from sparse_kv_refresh_amd.capacity import plateau_capacity
    wl = W.preset("t_bf16_small")
    r = W.make_rollout(wl, chunks=2)
    prec = O.Precision(wl.dtype)
    N, k = wl.n_tokens, wl.k
    eng = engine(wl, r)                       # rows_cap = N
    eng.dense(batch_z(wl, r, 0))
    snap = eng.snapshot()
    z1, q1 = batch_z(wl, r, 1), batch_q(wl, r, 1)
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
    rows = [k + 32 * j for j in range(9) if k + 32 * j <= N]
    curve = []
    for kk in rows:
        for i in range(5):
            eng.restore(snap)
            ev[i][0].record(stream)
            eng.chunk(z1, q1, kk, stream=stream)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        curve.append(float(np.median([a.elapsed_time(b) for a, b in ev[1:]])))
    k_fill = plateau_capacity(rows, curve, k, tol=0.01)
    assert k <= k_fill <= N
    for kf in sorted({k_fill, k + 56}):
        eng.restore(snap)
        st = _oracle_states(wl, r, prec)[0]
        res = O.refresh_chunk(st, r.z[0][1], r.qa[0][1], r.weights, kf, wl.age_bound, wl.n_heads, wl.ln_eps,
                              wl.w_attn, wl.w_surprise, prec)
        assert res.k_eff == kf
        ov = np.full((1, N), -1, dtype=np.int32)
        ov[0, :kf] = res.idx
        lo = torch.zeros((wl.n_layers, 1, N, wl.d_model), dtype=torch.float32, device=DEV)
        eng.chunk(z1, q1, kf, idx_override=to_dev(ov), k_eff_override=to_dev(np.array([kf], dtype=np.int32)),
                  layer_out=lo)
        torch.cuda.synchronize()
        _compare_chunk(wl, eng, [st], [res], lo, 1)
        # with its own selection the library fills by rank: the oracle's rule on the GPU's scores
        eng.restore(snap)
        eng.chunk(z1, q1, kf, layer_out=lo)
        torch.cuda.synchronize()
        sel, ke, _, _ = O.select(to_np(eng.score[0]), np.zeros(N, dtype=np.int64), kf, wl.age_bound)
        assert int(eng.k_eff[0]) == ke == kf
        assert np.array_equal(to_np(eng.idx[0])[:ke], sel)


@pytest.mark.parametrize("name,rows,cols", [("c3_stack", 12, 10), ("c3_stack", 36, 30), ("c3_text", 12, 10)])
def test_small_token_stack(name, rows, cols):
    """The small-context regime of the pages' latency experiment (WAM-Cache
    §5.2: the refresh ratio 0.584 of the native 120 visual tokens, here at 120
    and 1080 tokens) on three layers of the d=1536 stack, G = 2, in the
    launch configuration the small-N benchmark uses (rows_cap = k): the dense
    chunk's K/V caches, then three refresh chunks driven by the oracle's
    refresh sets.  With a few hundred rows the projections take the split-K
    path with a separate reduction (4 to 16 pieces per 64x128 tile at 70
    rows, 2 at 1080); with the module's text cross-attention (128 text
    tokens) its K/V, query and output projections take it too (WAM-Cache §3)."""
    N = rows * cols
    k = int(round(0.584 * N))
    wl = W.preset(name, n_layers=3, views=1, rows=rows, cols=cols, k=k, age_bound=2, chunks=4)
    r = W.make_rollout(wl, chunks=wl.chunks)
    prec = O.Precision(wl.dtype)
    states = _oracle_states(wl, r, prec)
    eng = engine(wl, r, rows_cap=k)
    eng.dense(batch_z(wl, r, 0))
    torch.cuda.synchronize()
    for l in range(wl.n_layers):
        for nm, g, o in (("K", eng.k_cache[l, 0], states[0].K[l]), ("V", eng.v_cache[l, 0], states[0].V[l])):
            ok, err = close(wl, to_np(g), o)
            assert ok, f"dense chunk {nm} layer {l}: error {err}"
    lo = torch.zeros((wl.n_layers, 1, k, wl.d_model), dtype=torch.float32, device=DEV)
    for t in range(1, wl.chunks):
        res = [O.refresh_chunk(states[0], r.z[0][t], r.qa[0][t], r.weights, k, wl.age_bound, wl.n_heads,
                               wl.ln_eps, wl.w_attn, wl.w_surprise, prec)]
        assert res[0].k_eff == k          # k >= N/2: the forced tokens always fit in k
        ov = np.full((1, N), -1, dtype=np.int32)
        ov[0, :k] = res[0].idx
        eng.chunk(batch_z(wl, r, t), batch_q(wl, r, t), k, idx_override=to_dev(ov),
                  k_eff_override=to_dev(np.array([k], dtype=np.int32)), layer_out=lo)
        torch.cuda.synchronize()
        _compare_chunk(wl, eng, states, res, lo, t)
