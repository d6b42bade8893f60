"""Pins of the sampling oracle: hand-worked draws, a library softmax, and
the stratified-frequency invariant of inverse-CDF sampling."""

import json
import os

import numpy as np
import pytest
from scipy.special import softmax

from oracle import sampling as SP

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "sampling_worked.json")))


@pytest.mark.parametrize("case", GOLDEN["greedy"], ids=lambda c: c["name"])
def test_greedy_worked(case):
    assert SP.greedy(np.array(case["logits"], dtype=np.float32)) == case["token"]


@pytest.mark.parametrize("case", GOLDEN["draw"], ids=lambda c: c["name"])
def test_draw_worked(case):
    z = np.array(case["logits"]) if "logits" in case else np.log(np.array(case["logits_are_log_of"]))
    for u, tok in case["cases"]:
        assert SP.draw(z, u) == tok, (u, tok)
        assert SP.draw_is_valid(z, u, tok, 0.0)


def test_probabilities_match_library_softmax():
    rng = np.random.default_rng(0)
    for V in (2, 17, 1000):
        z = (rng.standard_normal(V) * 6).astype(np.float32)
        np.testing.assert_allclose(SP.probabilities(z), softmax(z.astype(np.float64)), rtol=1e-13, atol=0)


def test_greedy_is_argmax_and_never_below_the_draws_mode():
    rng = np.random.default_rng(1)
    z = (rng.standard_normal(5000) * 3).astype(np.float32)
    assert SP.greedy(z) == int(np.argmax(z))
    # the greedy token is the one with the largest probability
    assert SP.probabilities(z)[SP.greedy(z)] == SP.probabilities(z).max()


def test_stratified_draws_reproduce_p():
    # u_k = (k + 1/2)/N lands on token j N p_j times, give or take one: a dropped,
    # shifted or misordered term in the cumulative sum breaks the counts
    rng = np.random.default_rng(2)
    z = (rng.standard_normal(40) * 2).astype(np.float32)
    p = softmax(z.astype(np.float64))
    N = 20000
    counts = np.zeros(z.size, dtype=np.int64)
    c = SP.cdf(z)
    for k in range(N):
        counts[SP.draw(z, (k + 0.5) / N)] += 1
    assert np.all(np.abs(counts - N * p) <= 1.0 + 1e-9)
    assert abs(c[-1] - 1.0) < 1e-12


def test_zero_probability_tokens_are_never_drawn():
    z = np.array([-2000.0, 0.0, -2000.0, 1.0, -2000.0])
    for u in np.linspace(0.0, 0.999999, 101):
        assert SP.draw(z, float(u)) in (1, 3)


def test_rejects_bad_inputs():
    with pytest.raises(ValueError):
        SP.draw([0.0, 1.0], 1.0)
    with pytest.raises(ValueError):
        SP.greedy([0.0, float("nan")])
