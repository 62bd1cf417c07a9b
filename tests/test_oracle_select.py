"""Pins of the oracle's refresh-set selection and age bookkeeping.

The selection rule: tokens whose age reached the bound are forced (WAM-Cache
§1, §4.4; RealtimeWAM App. D.3 "Recursive reuse"), forced tokens count toward
k, the rest are ranked by score with a lower-index tie-break.  Pinned here by
hand-worked examples, by exhaustive brute force on tiny inputs (every subset
of the right size checked against an independently written comparator), by
random dominance checks and by a closed-form cohort argument.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import wamc_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f(v):
    return float(v) if not isinstance(v, str) else float(v.replace("nan", "nan"))


def test_worked_examples():
    with open(os.path.join(GOLDEN, "select_worked.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        score = np.array([_f(v) for v in c["score"]], dtype=np.float32)
        age = np.array(c["age"], dtype=np.int64)
        idx, k_eff, new_age, n_forced = O.select(score, age, c["k"], c["G"])
        assert idx.tolist() == c["idx"], c
        assert k_eff == c["k_eff"]
        assert n_forced == c["n_forced"]
        assert new_age.tolist() == c["age_after"]


def _beats(i, j, forced, score):
    """Independent comparator: does token i rank strictly above token j?"""
    if forced[i] != forced[j]:
        return bool(forced[i])
    si, sj = float(score[i]), float(score[j])
    ni, nj = math.isnan(si), math.isnan(sj)
    if ni and nj:
        return i < j
    if ni != nj:
        return nj            # a number beats NaN
    if si != sj:              # -0.0 == 0.0 here
        return si > sj
    return i < j


def _brute_force(score, age, k, G):
    N = len(score)
    forced = [a >= G for a in age]
    k_eff = max(k, sum(forced))
    winners = []
    for S in itertools.combinations(range(N), k_eff):
        rest = [j for j in range(N) if j not in S]
        if all(_beats(i, j, forced, score) for i in S for j in rest):
            winners.append(list(S))
    assert len(winners) == 1, "the ranking must be a total order"
    return winners[0], k_eff


SCORE_SETS = [
    [0.5, -0.0, 0.0, float("nan"), 0.5, 1.0],
    [1.0, 1.0, 1.0, 1.0, 1.0, 1.0],
    [float("nan"), -1.0, 2.0, float("nan"), -0.0, 2.0],
]


@pytest.mark.parametrize("N,G", [(4, 2), (5, 2), (6, 1)])
def test_exhaustive_brute_force(N, G):
    for scores in SCORE_SETS:
        score = np.array(scores[:N], dtype=np.float32)
        for ages in itertools.product(range(G + 1), repeat=N):
            age = np.array(ages)
            for k in range(N + 1):
                idx, k_eff, new_age, _ = O.select(score, age, k, G)
                want, want_k = _brute_force(score, ages, k, G)
                assert idx.tolist() == want and k_eff == want_k
                assert new_age.max() <= G + 1
                refreshed = set(want)
                assert all(new_age[i] == (0 if i in refreshed else ages[i] + 1) for i in range(N))


def test_random_dominance_and_properties():
    rng = np.random.default_rng(7)
    for trial in range(200):
        N = int(rng.integers(1, 65))
        G = int(rng.integers(0, 5))
        k = int(rng.integers(0, N + 1))
        score = rng.choice(np.array([0.0, -0.0, 0.25, 0.5, np.nan, -3.0], dtype=np.float32), size=N)
        score = np.where(rng.random(N) < 0.5, score, rng.standard_normal(N).astype(np.float32))
        age = rng.integers(0, G + 2, size=N)
        idx, k_eff, new_age, n_forced = O.select(score, age, k, G)
        forced = age >= G
        S = set(idx.tolist())
        assert list(idx) == sorted(S)
        assert k_eff == max(k, int(forced.sum())) == len(S)
        assert set(np.nonzero(forced)[0].tolist()) <= S        # F subset of R
        for i in S:
            for j in set(range(N)) - S:
                assert _beats(i, j, forced, score)
        assert (new_age[list(S)] == 0).all()


def test_capacity_clamp():
    # more forced tokens than the row capacity: the cap wins, forced tokens
    # still rank first (lowest index among equals)
    score = np.array([3.0, 2.0, 1.0, 0.0], dtype=np.float32)
    age = np.array([5, 5, 5, 0])
    idx, k_eff, new_age, n_forced = O.select(score, age, 1, 2, cap=2)
    assert n_forced == 3 and k_eff == 2 and idx.tolist() == [0, 1]
    assert new_age.tolist() == [0, 0, 6, 1]


def test_cohort_closed_form():
    """If the same k tokens always top the scores, the other N-k tokens age
    together, are all forced at chunk G+1 after a dense start, and
    k_eff = max(k, N-k) there."""
    N, G = 20, 3
    for k in (3, 8, 10, 14):
        score = np.zeros(N, dtype=np.float32)
        score[:k] = 1.0
        age = np.zeros(N, dtype=np.int64)
        keffs = []
        for chunk in range(1, G + 3):
            idx, k_eff, age, _ = O.select(score, age, k, G)
            keffs.append(k_eff)
            assert age.max() <= G
        assert keffs[:G] == [k] * G
        assert keffs[G] == max(k, N - k)


def test_age_bound_zero_is_dense():
    score = np.arange(10, dtype=np.float32)
    idx, k_eff, age, _ = O.select(score, np.zeros(10, dtype=np.int64), 2, 0)
    assert k_eff == 10 and idx.tolist() == list(range(10)) and age.max() == 0


def test_planted_tie_break_mistake_is_caught(monkeypatch):
    """A wrong tie-break (higher index first) must fail the worked examples."""
    def wrong(forced, s, i):
        isnum = not math.isnan(s)
        return (forced, isnum, (s + 0.0) if isnum else 0.0, i)
    monkeypatch.setattr(O, "rank_key", wrong)
    with pytest.raises(AssertionError):
        test_worked_examples()


def test_planted_age_mistake_is_caught(monkeypatch):
    """Forgetting to reset refreshed ages must fail the cohort argument."""
    def wrong(age, idx):
        return np.asarray(age, dtype=np.int64) + 1
    monkeypatch.setattr(O, "ages_after", wrong)
    with pytest.raises(AssertionError):
        test_cohort_closed_form()
