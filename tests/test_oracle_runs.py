"""The oracle rollouts that the full-size GPU tests run in worker processes
give exactly what a direct call in this process gives, chunk by chunk and
episode by episode, and their bf16 packing is lossless."""
import numpy as np

from oracle import wamc_oracle as O
from sparse_kv_refresh_amd import inputs as W

from oracle_runs import bf16_bits, episode_rollout, episodes_in_parallel, from_bf16_bits


def test_parallel_rollouts_equal_direct_calls():
    wl = W.preset("t_bf16_batch")
    par = episodes_in_parallel("t_bf16_batch", {}, [0, 2], 2)
    r = W.make_rollout(wl, chunks=2)
    prec = O.Precision(wl.dtype)
    for e, run in zip([0, 2], par):
        again = episode_rollout("t_bf16_batch", {}, e, 2)
        for a, b in zip(run, again):
            assert a.keys() == b.keys()
            for k in a:
                assert np.array_equal(np.asarray(a[k]), np.asarray(b[k])), (e, k)
        # the same inputs as make_rollout draws, and the same oracle chunk
        st, _ = O.dense_prefill(r.z[e][0], r.weights, wl.n_heads, wl.ln_eps, prec)
        st.age = np.asarray(r.ages0[e], dtype=np.int64)
        res = O.refresh_chunk(st, r.z[e][1], r.qa[e][1], r.weights, wl.k, wl.age_bound, wl.n_heads, wl.ln_eps,
                              wl.w_attn, wl.w_surprise, prec)
        assert np.array_equal(run[1]["idx"], res.idx) and run[1]["k_eff"] == res.k_eff
        assert np.array_equal(from_bf16_bits(run[1]["K"]), st.K)
        assert np.array_equal(run[1]["X"], np.stack(res.outs).astype(np.float32))


def test_bf16_packing_is_lossless():
    x = O.round_bf16(np.random.default_rng(0).standard_normal(1000).astype(np.float32))
    assert np.array_equal(from_bf16_bits(bf16_bits(x)), x)
