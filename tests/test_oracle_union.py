"""Pins of the oracle's union refresh rule (WAM-Cache §1, §4.3, §4.4, §5.3):
top-ceil(b_a N) by attention mass, top-ceil(b_s N) by surprise, plus the
forced tokens, each counted once.  Checked against a brute-force formulation
(pairwise "beats" counts), set identities and closed forms."""
import math

import numpy as np
import pytest

from oracle import wamc_oracle as O


def _beats(vj, j, vi, i):
    """Does token j outrank token i?  Numbers above NaN; equal values (with
    -0 == +0) go to the lower index."""
    nj, ni = math.isnan(vj), math.isnan(vi)
    if nj != ni:
        return ni
    if nj and ni:
        return j < i
    if vj != vi:
        return vj > vi
    return j < i


def _top_brute(v, n):
    N = len(v)
    out = []
    for i in range(N):
        better = sum(1 for j in range(N) if j != i and _beats(float(v[j]), j, float(v[i]), i))
        if better < n:
            out.append(i)
    return out


def _values(rng, N):
    pool = np.array([0.0, -0.0, 1.0, 2.5, -3.0, np.nan, 1e-30, 7.0], dtype=np.float32)
    v = rng.standard_normal(N).astype(np.float32)
    m = rng.random(N) < 0.5
    v[m] = rng.choice(pool, size=int(m.sum()))
    return v


@pytest.mark.parametrize("seed", range(40))
def test_union_brute_force(seed):
    rng = np.random.default_rng(seed)
    N = int(rng.integers(1, 40))
    P, U = _values(rng, N), _values(rng, N)
    G = int(rng.integers(0, 4))
    age = rng.integers(0, 5, size=N)
    na, ns = int(rng.integers(0, N + 1)), int(rng.integers(0, N + 1))
    idx, k_eff, new_age, n_forced = O.select_union(P, U, age, na, ns, G)
    want = sorted(set(_top_brute(P, na)) | set(_top_brute(U, ns)) | {i for i in range(N) if age[i] >= G})
    assert idx.tolist() == want
    assert k_eff == len(want)
    assert n_forced == int((age >= G).sum())
    assert np.array_equal(new_age, np.where(np.isin(np.arange(N), want), 0, age + 1))


def test_union_counts_shared_tokens_once():
    """§5.3: tokens picked by both signals are counted once."""
    N = 10
    P = np.arange(N, dtype=np.float32)           # top 4 by mass: 6..9
    U = np.arange(N, dtype=np.float32)[::-1].copy()   # top 3 by surprise: 0..2
    age = np.zeros(N, dtype=np.int64)
    idx, k_eff, _, _ = O.select_union(P, U, age, 4, 3, G=2)
    assert k_eff == 7 and idx.tolist() == [0, 1, 2, 6, 7, 8, 9]     # disjoint: n_a + n_s
    idx, k_eff, _, _ = O.select_union(P, P, age, 4, 3, G=2)
    assert k_eff == 4 and idx.tolist() == [6, 7, 8, 9]               # same ranking: max(n_a, n_s)


def test_union_degenerate_budgets():
    rng = np.random.default_rng(7)
    N = 50
    P, U = rng.random(N).astype(np.float32), rng.random(N).astype(np.float32)
    age = rng.integers(0, 4, size=N)
    idx, k_eff, _, nf = O.select_union(P, U, age, 0, 0, G=2)
    assert idx.tolist() == np.flatnonzero(age >= 2).tolist() and k_eff == nf   # only the forced set
    idx, k_eff, new_age, _ = O.select_union(P, U, age, N, 0, G=2)
    assert k_eff == N and (new_age == 0).all()                                  # everything
    idx, k_eff, _, _ = O.select_union(P, U, np.zeros(N, dtype=np.int64), 5, 0, G=0)
    assert k_eff == N                                                           # G = 0: every chunk dense


def test_union_set_identities():
    rng = np.random.default_rng(11)
    for _ in range(50):
        N = int(rng.integers(5, 200))
        P, U = rng.random(N).astype(np.float32), rng.random(N).astype(np.float32)
        age = rng.integers(0, 4, size=N)
        na, ns = int(rng.integers(0, N)), int(rng.integers(0, N))
        idx, k_eff, _, nf = O.select_union(P, U, age, na, ns, 3)
        s = set(idx.tolist())
        assert set(O.top_by(P, na).tolist()) <= s and set(O.top_by(U, ns).tolist()) <= s
        assert set(np.flatnonzero(age >= 3).tolist()) <= s
        assert max(na, ns, nf) <= k_eff <= min(N, na + ns + nf)
        assert np.all(np.diff(idx) > 0)


def test_budget_counts():
    """ceil(b N) without float rounding: 0.1 * 30 is 3, not 4."""
    assert O.budget_count(0.1, 30) == 3
    assert O.budget_count(0.4, 4680) == 1872
    assert O.budget_count(0.4, 120) == 48 and O.budget_count(0.1, 120) == 12
    assert O.budget_count(0.6, 120) == 72
    assert O.budget_count(0.25, 7) == 2 and O.budget_count(0.0, 9) == 0 and O.budget_count(1.0, 9) == 9


def test_union_rollout_age_invariant():
    """With the union rule no age ever exceeds G after a chunk (R5), and the
    recompute ratio stays within [max budget share, 1]."""
    rng = np.random.default_rng(5)
    N, G = 300, 2
    na, ns = O.budget_count(0.4, N), O.budget_count(0.1, N)
    age = np.zeros(N, dtype=np.int64)
    ratios = []
    for t in range(12):
        P, U = rng.random(N).astype(np.float32), rng.random(N).astype(np.float32)
        idx, k_eff, age, _ = O.select_union(P, U, age, na, ns, G)
        assert age.max() <= G
        ratios.append(k_eff / N)
    assert min(ratios) >= na / N
