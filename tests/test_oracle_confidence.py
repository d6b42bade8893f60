"""Pins for oracle.confidence: closed forms of the confidence on distribution
families whose entropy, margin and top probability are known by hand."""

import math

import numpy as np
import pytest

from oracle import confidence as C


def sig(x):
    return 1.0 / (1.0 + math.exp(-x))


@pytest.mark.parametrize("V", [2, 3, 1000, 152064])
def test_uniform_logits(V):
    # Uniform p: H = log V so Hn = 1; margin 0 so sigma = 1/2; p_max = 1/V.
    z = np.full(V, 0.37, dtype=np.float32)
    Hn, margin, pmax = C.distribution_terms(z)
    assert abs(Hn - 1.0) < 1e-12 and margin == 0.0 and abs(pmax - 1.0 / V) < 1e-15
    assert abs(C.confidence(z) - (0.15 + 0.3 / V)) < 1e-12


@pytest.mark.parametrize("V", [2, 1000, 152064])
@pytest.mark.parametrize("g", [0.25, 1.0, 3.0, 10.0, 25.0])
def test_one_raised_logit_closed_form(V, g):
    # Logits (g, 0, ..., 0): p1 = 1/(1 + (V-1)e^-g), every other p_o = p1 e^-g.
    p1 = 1.0 / (1.0 + (V - 1) * math.exp(-g))
    po = p1 * math.exp(-g)
    H = -p1 * math.log(p1) - (V - 1) * po * math.log(po)
    want = 0.4 * (1 - H / math.log(V)) + 0.3 * sig(g) + 0.3 * p1
    z = np.zeros(V)
    z[V // 3] = g
    assert abs(C.confidence(z) - want) < 1e-12


def test_one_hot_limit():
    # As one logit dominates, H -> 0 and p_max -> 1, so c -> 0.7 + 0.3 sigma(margin).
    for V, g in ((1000, 40.0), (152064, 45.0)):
        z = np.zeros(V)
        z[7] = g
        assert abs(C.confidence(z) - (0.7 + 0.3 * sig(g))) < 1e-5


def test_two_candidates_closed_form():
    # V = 2: p1 = sigma(|a-b|), binary entropy, margin |a-b|.
    for a, b in ((1.0, -2.0), (0.3, 0.29), (-5.0, 4.0)):
        d = abs(a - b)
        p1 = sig(d)
        Hb = -(p1 * math.log(p1) + (1 - p1) * math.log(1 - p1))
        want = 0.4 * (1 - Hb / math.log(2)) + 0.3 * sig(d) + 0.3 * p1
        assert abs(C.confidence([a, b]) - want) < 1e-12


def test_tied_maxima_margin_zero():
    z = np.array([1.0, 5.0, 5.0, -1.0])
    _, margin, _ = C.distribution_terms(z)
    assert margin == 0.0


def test_weights_are_separately_visible():
    # Distinct families isolate each weight: a wrong weight on one term moves c.
    V = 1000
    z = np.zeros(V)
    base = C.confidence(z)
    assert abs(C.confidence(z, 0.5, 0.3, 0.3) - base) < 1e-12          # entropy term is 0 here
    assert abs(C.confidence(z, 0.4, 0.4, 0.3) - (base + 0.05)) < 1e-12  # margin term is sigma(0)=1/2
    assert abs(C.confidence(z, 0.4, 0.3, 0.4) - (base + 0.1 / V)) < 1e-12


def test_invariances():
    rng = np.random.default_rng(3)
    z = rng.normal(size=500) * 4
    c = C.confidence(z)
    assert abs(C.confidence(rng.permutation(z)) - c) < 1e-12
    assert abs(C.confidence(z + 123.25) - c) < 1e-10
    assert 0.0 < c < 1.0


def test_underflowing_probabilities_contribute_zero_entropy():
    z = np.array([0.0, -2000.0, -3000.0])
    Hn, margin, pmax = C.distribution_terms(z)
    assert Hn == 0.0 and margin == 2000.0 and pmax == 1.0


def test_gate_prose_reading_and_literal():
    assert C.gate(0.61, 0.6, 64, 128) == 64       # confident -> tight
    assert C.gate(0.59, 0.6, 64, 128) == 128      # uncertain -> loose
    assert C.gate(0.6, 0.6, 64, 128) == 64        # c == tau counts as confident
    assert C.gate(0.61, 0.6, 128, 64) == 64       # naming-independent
    assert C.gate(0.61, 0.6, 64, 128, literal=True) == 128
    assert C.gate(0.59, 0.6, 64, 128, literal=True) == 64


def test_pyramid_schedule():
    # 1.5x at the first layer, 0.5x at the last, linear, floored, non-increasing.
    L = 12
    b = [C.layer_budget(256, l, L, True) for l in range(L)]
    assert b[0] == 384 and b[-1] == 128
    assert all(x >= y for x, y in zip(b, b[1:]))
    L = 5
    assert [C.layer_budget(100, l, L, True) for l in range(L)] == [150, 125, 100, 75, 50]
    assert C.layer_budget(77, 0, 1, True) == 77
    assert C.layer_budget(77, 3, 8, False) == 77
