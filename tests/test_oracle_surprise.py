"""Value pins of the oracle's latent surprise, combined score and reference
embedding (hand-worked values in tests/golden/surprise_worked.json).

* Surprise is the squared Euclidean distance over the channels between a
  token's input embedding and its reference embedding (WAM-Cache §4.2
  "Latent Surprise").
* The reference is the embedding the token had at its most recent refresh
  (WAM-Cache §4.1 "Overview"): a token that moves while it is being reused is
  measured against that older embedding, not against the previous chunk's.
* The combined score normalises the attention mass by L*H*A and the surprise
  by its sum over tokens (the reading of the lost display formula).

Each plausible mistake below (an L1 distance, an unsquared norm, a mean over
channels, the previous frame as the reference, a swapped weight, a missing
normaliser) is planted in the oracle and must fail these pins.
"""
import json
import os

import numpy as np
import pytest

from oracle import wamc_oracle as O
from sparse_kv_refresh_amd import inputs as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "surprise_worked.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_surprise_worked_values():
    for case in _golden()["surprise"]:
        for dtype in ("fp32", "bf16"):
            U = O.surprise(np.array(case["z"], dtype=np.float32), np.array(case["zref"], dtype=np.float32),
                           O.Precision(dtype))
            assert U.tolist() == [float(u) for u in case["U"]], (dtype, U)


def test_combine_worked_values():
    for case in _golden()["combine"]:
        s = O.combine(np.array(case["P"], dtype=np.float64), np.array(case["U"], dtype=np.float64),
                      case["L"], case["H"], case["A"], case["w_attn"], case["w_surprise"])
        assert s.dtype == np.float32
        want = np.array(case["score"], dtype=np.float64)
        assert np.allclose(s.astype(np.float64), want, rtol=1e-6, atol=1e-8), (case["work"], s)


def _tiny_workload():
    # N = 3 tokens of d = 4; only z and the refresh sets matter for U
    return W.Workload("surprise_rollout", 1, 4, 1, 8, 1, 1, 3, 2, 1, 5, "fp32", chunks=4)


def test_reference_is_the_embedding_at_the_last_refresh():
    g = _golden()["rollout"]
    wl = _tiny_workload()
    weights = W.make_weights(wl)
    prec = O.Precision("fp32")
    z = [np.array(zt, dtype=np.float32) for zt in g["z"]]
    st, _ = O.dense_prefill(z[0], weights, wl.n_heads, wl.ln_eps, prec)
    assert st.zref.tolist() == g["zref_after"][0]
    for t in range(1, len(z)):
        res = O.refresh_chunk(st, z[t], W.make_queries(wl, t), weights, wl.k, wl.age_bound, wl.n_heads,
                              wl.ln_eps, wl.w_attn, wl.w_surprise, prec,
                              idx_override=np.array(g["refresh"][t], dtype=np.int32))
        assert res.surprise.tolist() == [float(u) for u in g["U"][t]], (t, res.surprise)
        assert st.zref.tolist() == g["zref_after"][t], t


def _all_pins():
    test_surprise_worked_values()
    test_combine_worked_values()
    test_reference_is_the_embedding_at_the_last_refresh()


def test_pins_pass_as_committed():
    _all_pins()


# ---------------------------------------------------------------- planted mistakes

@pytest.mark.parametrize("mistake", ["l1", "unsquared", "channel_mean"])
def test_planted_distance_mistakes_are_caught(monkeypatch, mistake):
    def wrong(z, zref, prec):
        diff = prec.load(z) - prec.load(zref)
        if mistake == "l1":
            return np.abs(diff).sum(axis=1)
        if mistake == "unsquared":
            return np.sqrt((diff * diff).sum(axis=1))
        return (diff * diff).mean(axis=1)
    monkeypatch.setattr(O, "surprise", wrong)
    with pytest.raises(AssertionError):
        _all_pins()


def test_planted_previous_frame_reference_is_caught(monkeypatch):
    """Every token's reference moved to this chunk's embedding, refreshed or
    not: surprise then measures the change from the previous chunk."""
    def wrong(zref, z, idx):
        zref[:] = z
    monkeypatch.setattr(O, "update_reference", wrong)
    with pytest.raises(AssertionError):
        _all_pins()


@pytest.mark.parametrize("mistake", ["swapped_weights", "unnormalised_surprise", "mass_over_sum"])
def test_planted_combine_mistakes_are_caught(monkeypatch, mistake):
    def wrong(P, U, n_layers, n_heads, n_action, w_attn, w_surprise):
        total = U.sum()
        if mistake == "swapped_weights":
            w_attn, w_surprise = w_surprise, w_attn
        pn = P / P.sum() if mistake == "mass_over_sum" else P / (n_layers * n_heads * n_action)
        s = w_attn * pn
        if total > 0:
            s = s + w_surprise * (U if mistake == "unnormalised_surprise" else U / total)
        return np.asarray(s, dtype=np.float32)
    monkeypatch.setattr(O, "combine", wrong)
    with pytest.raises(AssertionError):
        _all_pins()
