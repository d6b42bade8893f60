"""The oracle against hand-worked examples under tests/golden/.

Each fixture is worked out by hand from the definitions on the pages (its
`source` and `derivation` fields); no value in them comes from running code.
"""

import json
import os

import numpy as np
import pytest

from oracle import confidence as C
from oracle import kvpop as KP
from oracle import policy as P
from oracle import quant as Q

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.mark.parametrize("case", load("confidence_worked.json")["cases"], ids=lambda c: c["name"])
def test_confidence_worked(case):
    z = np.array(case["logits"], dtype=np.float64)
    c = C.confidence(z)
    assert abs(c - case["c"]) < 1e-12
    assert C.gate(c, case["tau"], case["n_low"], case["n_high"]) == case["budget_prose"]
    assert C.gate(c, case["tau"], case["n_low"], case["n_high"], literal=True) == case["budget_literal"]


def test_eviction_worked():
    g = load("eviction_worked.json")
    pos = np.array(g["pos"])
    score = P.composite_score(np.array(g["ema"]), P.recency(pos, g["t"]), g["alpha"]).astype(np.float32)
    assert score.tolist() == np.array(g["score_f32"], dtype=np.float32).tolist()
    vic = P.select_victims(pos, score, g["t"], g["budget"], g["num_sink"], g["protect_last"])
    assert pos[vic].tolist() == g["victim_pos"]
    assert sorted(set(g["pos"]) - set(pos[vic].tolist())) == g["kept_pos"]


@pytest.mark.parametrize("case", load("int8_worked.json")["cases"], ids=lambda c: str(c["scale"]))
def test_int8_worked(case):
    codes, scale = Q.quantize_row(np.array(case["x"], dtype=np.float16))
    assert float(scale) == case["scale"]
    assert codes.tolist() == case["codes"]


def test_budgets_worked():
    g = load("budget_worked.json")
    for c in g["pyramid"]:
        assert C.layer_budget(c["base"], c["layer"], c["num_layers"], True) == c["budget"], c
    for c in g["kvpop"]:
        assert KP.budget(c["num_sink"], c["window"], c["k"]) == c["budget"]


@pytest.mark.parametrize("case", load("kvpop_worked.json")["cases"], ids=lambda c: f"t{c['t']}")
def test_kvpop_worked(case):
    g = load("kvpop_worked.json")
    prio = np.array(g["prio"], dtype=np.float32)
    kept = KP.kept_closed_form(case["t"], lambda p: prio[p], g["num_sink"], g["window"], g["k"])
    assert kept == case["kept"]
    # the incremental rule over the whole history reaches the same set
    pos = []
    for t in range(case["t"] + 1):
        pos.append(t)
        arr = np.array(pos)
        vic = KP.long_range_victims(arr, prio[arr], t, g["num_sink"], g["window"], g["k"])
        pos = [p for i, p in enumerate(pos) if i not in set(vic.tolist())]
    assert pos == case["kept"]
