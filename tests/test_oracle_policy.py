"""Pins for oracle.policy: EMA closed form, recency, and the eviction rule
against exhaustive search over subsets on tiny segments with forced ties."""

import itertools

import numpy as np
import pytest

from oracle import policy as P


def test_ema_closed_form():
    # Constant mass a from ema = 0 for k steps: a (1 - beta^k).
    a, beta = 0.37, 0.9
    e = np.zeros(1)
    for k in range(1, 30):
        e = P.ema_update(e, a, beta)
        assert abs(e[0] - a * (1 - beta ** k)) < 1e-15


def test_recency_and_score():
    t = 99
    r = P.recency(np.array([0, 49, 99]), t)
    assert r.tolist() == [0.01, 0.5, 1.0]
    assert P.composite_score(0.2, 1.0, 1.0) == 0.2 and P.composite_score(0.2, 1.0, 0.0) == 1.0
    assert abs(P.composite_score(0.2, 1.0, 0.25) - (0.05 + 0.75)) < 1e-15


def _better(i, j, score, pos):
    return (score[i], -pos[i]) > (score[j], -pos[j])


@pytest.mark.parametrize("seed", range(40))
def test_selection_exhaustive(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 11))
    t = int(rng.integers(n - 1, n + 20))
    pos = np.sort(rng.choice(np.arange(t), size=n - 1, replace=False)) if n > 1 else np.zeros(0, int)
    pos = np.append(pos, t)
    score = rng.choice([0.1, 0.2, 0.3], size=n).astype(np.float32)      # many ties
    budget = int(rng.integers(0, n + 2))
    s, Pw = int(rng.integers(0, 3)), int(rng.integers(0, 4))
    vic = set(P.select_victims(pos, score, t, budget, s, Pw).tolist())
    prot = [i for i in range(n) if pos[i] < s or pos[i] > t - Pw]
    cand = [i for i in range(n) if i not in prot]
    if n <= budget:
        assert not vic
        return
    keep_free = max(0, budget - len(prot))
    want = None
    for S in itertools.combinations(cand, min(keep_free, len(cand))):
        if all(_better(i, j, score, pos) for i in S for j in cand if j not in S):
            assert want is None
            want = set(cand) - set(S)
    assert vic == want
    assert not vic & set(prot)
    assert n - len(vic) == max(budget, len(prot)) if keep_free <= len(cand) else True


def test_pure_recency_is_sliding_window():
    # alpha = 0: the score is recency, so the kept set is the newest `budget` rows.
    t, budget = 50, 12
    pos = np.arange(t + 1)
    score = P.composite_score(np.random.default_rng(0).random(t + 1), P.recency(pos, t), 0.0).astype(np.float32)
    vic = P.select_victims(pos, score, t, budget, 0, 4)
    kept = sorted(set(pos.tolist()) - set(pos[vic].tolist()))
    assert kept == list(range(t + 1 - budget, t + 1))


def test_negative_zero_ties_with_zero():
    pos = np.array([3, 5, 9])
    score = np.array([0.0, -0.0, 1.0], np.float32)
    assert P.select_victims(pos, score, 9, 2, 0, 1).tolist() == [1]   # tie -> higher position goes
