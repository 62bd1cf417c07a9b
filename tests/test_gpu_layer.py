"""GPU DiT layers against the oracle: the dense prefill (every token through
every layer, WAM-Cache §4.1) and a single refresh layer on a given row set
(§3, §4.4: fresh K/V written before attention over all N keys)."""
import numpy as np
import pytest
import torch

from oracle import wamc_oracle as O
from sparse_kv_refresh_amd import inputs as W
from sparse_kv_refresh_amd import wamc

from gpu_util import DEV, act, batch_z, close, engine, to_dev, to_np

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["c1_tiny", "t_fp32_ragged", "t_bf16_small", "t_bf16_batch", "t_bf16_text",
                                  "t_fp32_text", "c2_layer"])
def test_dense_parity(name):
    """c2_layer is the benchmark's layer at full size (N=4096): its MLP up
    projection runs on 128x192 tiles with a ragged last column tile (8960
    columns)."""
    wl = W.preset(name)
    r = W.make_rollout(wl, chunks=1)
    prec = O.Precision(wl.dtype)
    eng = engine(wl, r)
    L, B, N, d = wl.n_layers, wl.batch, wl.n_tokens, wl.d_model
    lo = torch.zeros((L, B, N, d), dtype=torch.float32, device=DEV)
    z0 = batch_z(wl, r, 0)
    eng.age.fill_(5)
    eng.dense(z0, layer_out=lo)
    torch.cuda.synchronize()
    assert (eng.age == 0).all()
    assert torch.equal(eng.zref, z0)
    for b in range(B):
        st, outs = O.dense_prefill(r.z[b][0], r.weights, wl.n_heads, wl.ln_eps, prec,
                                   text_emb=None if r.text is None else r.text[b])
        for l in range(L):
            for name_, g, o in (("K", eng.k_cache[l, b], st.K[l]), ("V", eng.v_cache[l, b], st.V[l]),
                                ("X", lo[l, b], outs[l])):
                ok, err = close(wl, to_np(g), o)
                assert ok, f"{name_} layer {l} episode {b}: error {err}"


@pytest.mark.parametrize("name", ["c1_tiny", "t_bf16_small"])
def test_refresh_layer_parity(name):
    """One layer on 3/8 of the tokens, ascending ids, over a cache that holds
    other values everywhere else."""
    wl = W.preset(name)
    r = W.make_rollout(wl, chunks=1)
    prec = O.Precision(wl.dtype)
    N, d = wl.n_tokens, wl.d_model
    rng = np.random.default_rng(3)
    m = (3 * N) // 8
    idx = np.sort(rng.choice(N, size=m, replace=False)).astype(np.int32)
    Kc = prec.store(rng.standard_normal((N, d)).astype(np.float32) * 0.5)
    Vc = prec.store(rng.standard_normal((N, d)).astype(np.float32) * 0.5)
    X = rng.standard_normal((m, d)).astype(np.float32)
    Ko, Vo = Kc.astype(prec.acc).copy(), Vc.astype(prec.acc).copy()
    want = O.block(X.astype(prec.acc), idx, r.weights[0], Ko, Vo, wl.n_heads, wl.ln_eps, prec)

    dims = wamc.dims_for(wl)
    w = wamc.Engine.upload_weights(r.weights, act(wl), DEV)[0]
    rows_cap = m + 5                      # spare rows beyond k_eff stay untouched
    x = torch.zeros((1, rows_cap, d), dtype=torch.float32, device=DEV)
    x[0, :m] = torch.from_numpy(X).to(DEV)
    x[0, m:] = 123.0
    idx_full = np.full((1, N), -1, dtype=np.int32)
    idx_full[0, :m] = idx
    kc, vc = to_dev(Kc, act(wl))[None].contiguous(), to_dev(Vc, act(wl))[None].contiguous()
    keff = torch.tensor([m], dtype=torch.int32, device=DEV)
    ws = torch.empty(wamc.workspace_bytes(dims, rows_cap), dtype=torch.uint8, device=DEV)
    wamc.refresh_layer(dims, 0, w, x, to_dev(idx_full), keff, rows_cap, kc, vc, ws)
    torch.cuda.synchronize()
    for nm, g, o in (("X", to_np(x[0, :m]), want), ("K", to_np(kc[0]), Ko), ("V", to_np(vc[0]), Vo)):
        ok, err = close(wl, g, o)
        assert ok, f"{nm}: {err}"
    assert (x[0, m:] == 123.0).all()
    untouched = np.setdiff1d(np.arange(N), idx)
    assert np.array_equal(to_np(kc[0])[untouched], Kc[untouched])


@pytest.mark.parametrize("m,spare", [(37, False), (37, True), (300, True), (1100, False), (1100, True),
                                     (2458, False), (2808, False), (4096, False)])
def test_refresh_layer_wide(m, spare):
    """The d=1536, FFN 8960 layer over N=4096 cached tokens with m refreshed
    rows, the launch sized for the rows (rows_cap = m) or for every token
    (rows_cap = N, k_eff = m read on the device): covers the GEMM schedules
    that split K over several workgroups and the one-tile-per-workgroup
    rounds of 128x128 tiles (a single-layer call knows no lower bound on
    k_eff on the host, so it never takes the 256x256 tiles; the chunk test
    with k = 3840 covers those).  At 2808 rows the down projection's 264
    tiles of 140 k-tiles run as 792 pieces, more than one round of
    workgroups, from a grid sized for them."""
    _check_refresh_layer(W.preset("c2_layer"), m, spare, seed=m)


def test_refresh_layer_ragged_columns():
    """A d=1152 layer (9 heads of 128) with an FFN of 3000 and 40 refreshed
    rows: the QKV, out- and MLP up projections take the split-K path with
    three pieces per tile, the up projection's last column tile holding 56 of
    its 128 columns (3000 = 23 x 128 + 56); the down projection (K = 3000,
    not a multiple of 64) takes the generic kernel."""
    wl = W.preset("c2_layer", d_model=1152, n_heads=9, d_ffn=3000, k=40)
    _check_refresh_layer(wl, wl.k, False, seed=40)


def test_refresh_layer_batch_split():
    """Three episodes of the d=1536, FFN 8960 layer over N=4096 cached tokens
    with 37, 100 and 0 refreshed rows (rows_cap = 100, k_eff read on the
    device): with this few rows the out-projection and the MLP down
    projection take the split-K path with a separate reduction (4 and 7
    pieces per 64x128 tile), its tiles derived from each episode's k_eff, and
    the out-projection's reduction also does adaLN-2.  Every episode against
    the oracle's block; the empty episode's caches and the rows past k_eff
    stay untouched (WAM-Cache §4.4)."""
    wl = W.preset("c2_layer", batch=3)
    weights = W.make_weights(wl)
    prec = O.Precision(wl.dtype)
    N, d, B = wl.n_tokens, wl.d_model, wl.batch
    rows_cap, ms = 100, [37, 100, 0]
    rng = np.random.default_rng(11)
    x = torch.full((B, rows_cap, d), 77.0, dtype=torch.float32, device=DEV)
    idx_full = np.full((B, N), -1, dtype=np.int32)
    Kcs, Vcs, wants, Kos, Vos = [], [], [], [], []
    for e, m in enumerate(ms):
        idx = np.sort(rng.choice(N, size=m, replace=False)).astype(np.int32)
        Kc = prec.store(rng.standard_normal((N, d)).astype(np.float32) * 0.5)
        Vc = prec.store(rng.standard_normal((N, d)).astype(np.float32) * 0.5)
        X = rng.standard_normal((m, d)).astype(np.float32)
        Ko, Vo = Kc.astype(prec.acc).copy(), Vc.astype(prec.acc).copy()
        wants.append(O.block(X.astype(prec.acc), idx, weights[0], Ko, Vo, wl.n_heads, wl.ln_eps, prec) if m else None)
        Kcs.append(Kc); Vcs.append(Vc); Kos.append(Ko); Vos.append(Vo)
        x[e, :m] = torch.from_numpy(X).to(DEV)
        idx_full[e, :m] = idx
    dims = wamc.dims_for(wl)
    w = wamc.Engine.upload_weights(weights, act(wl), DEV)[0]
    kc = to_dev(np.stack(Kcs), act(wl)).contiguous()
    vc = to_dev(np.stack(Vcs), act(wl)).contiguous()
    keff = torch.tensor(ms, dtype=torch.int32, device=DEV)
    ws = torch.empty(wamc.workspace_bytes(dims, rows_cap), dtype=torch.uint8, device=DEV)
    wamc.refresh_layer(dims, 0, w, x, to_dev(idx_full), keff, rows_cap, kc, vc, ws)
    torch.cuda.synchronize()
    for e, m in enumerate(ms):
        if m:
            for nm, g, o in (("X", to_np(x[e, :m]), wants[e]), ("K", to_np(kc[e]), Kos[e]), ("V", to_np(vc[e]), Vos[e])):
                ok, err = close(wl, g, o)
                assert ok, f"episode {e} {nm}: {err}"
        else:
            assert np.array_equal(to_np(kc[e]), Kcs[e]) and np.array_equal(to_np(vc[e]), Vcs[e])
        assert (x[e, m:] == 77.0).all(), f"episode {e}: rows past k_eff"


@pytest.mark.parametrize("n", [33, 65, 130, 257, 1000, 4000, 4095])
def test_refresh_layer_key_tiles(n):
    """The attention's key-tile paths, on a d=256 layer (two heads of 128)
    with up to 40 refreshed rows, so that its two (query tile, head) units
    are cut into key ranges wherever N has enough tiles: a single ragged
    tile (N < 64); a ragged last tile falling to either key group of the
    last iteration (odd and even tile counts); pieces of several tiles whose
    last piece ends in the ragged tile (N = 4000, 4095); and the fresh K/V
    of the refreshed rows written before the attention reads them."""
    wl = W.preset("t_bf16_small", views=1, rows=1, cols=n, k=min(40, n))
    _check_refresh_layer(wl, wl.k, False, seed=n)


def _check_refresh_layer(wl, m, spare, seed):
    """One wamc_refresh_layer call (twice, reusing the workspace) on m random
    rows of an N-token cache against the oracle's block."""
    r = W.make_rollout(wl, chunks=1)
    prec = O.Precision(wl.dtype)
    N, d = wl.n_tokens, wl.d_model
    rng = np.random.default_rng(seed)
    idx = np.sort(rng.choice(N, size=m, replace=False)).astype(np.int32)
    Kc = prec.store(rng.standard_normal((N, d)).astype(np.float32) * 0.5)
    Vc = prec.store(rng.standard_normal((N, d)).astype(np.float32) * 0.5)
    X = rng.standard_normal((m, d)).astype(np.float32)
    Ko, Vo = Kc.astype(prec.acc).copy(), Vc.astype(prec.acc).copy()
    want = O.block(X.astype(prec.acc), idx, r.weights[0], Ko, Vo, wl.n_heads, wl.ln_eps, prec)

    dims = wamc.dims_for(wl)
    w = wamc.Engine.upload_weights(r.weights, act(wl), DEV)[0]
    rows_cap = N if spare else m
    x = torch.full((1, rows_cap, d), 77.0, dtype=torch.float32, device=DEV)
    x[0, :m] = torch.from_numpy(X).to(DEV)
    idx_full = np.full((1, N), -1, dtype=np.int32)
    idx_full[0, :m] = idx
    kc, vc = to_dev(Kc, act(wl))[None].contiguous(), to_dev(Vc, act(wl))[None].contiguous()
    keff = torch.tensor([m], dtype=torch.int32, device=DEV)
    ws = torch.empty(wamc.workspace_bytes(dims, rows_cap), dtype=torch.uint8, device=DEV)
    for rep in range(2):   # a second call reuses the workspace (arrival counters must be back at zero)
        if rep:
            x[0, :m] = torch.from_numpy(X).to(DEV)
            kc.copy_(to_dev(Kc, act(wl))[None])
            vc.copy_(to_dev(Vc, act(wl))[None])
        wamc.refresh_layer(dims, 0, w, x, to_dev(idx_full), keff, rows_cap, kc, vc, ws)
        torch.cuda.synchronize()
        for nm, g, o in (("X", to_np(x[0, :m]), want), ("K", to_np(kc[0]), Ko), ("V", to_np(vc[0]), Vo)):
            ok, err = close(wl, g, o)
            assert ok, f"call {rep} {nm}: {err}"
        if spare:
            assert (x[0, m:] == 77.0).all()
