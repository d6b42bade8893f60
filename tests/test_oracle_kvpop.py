"""Pins for oracle.kvpop: the step-by-step rule equals the history-free
top-k closed form at every step of a stream."""

import numpy as np

from oracle import cache as OC
from oracle import kvpop as KP


def test_incremental_equals_closed_form():
    s, w, k, d = 2, 4, 5, 8
    rng = np.random.default_rng(5)
    steps = 60
    prio = rng.random(steps).astype(np.float32)
    prio[10:20] = prio[10]                                  # ties
    cfg = OC.Config(num_layers=1, batch=1, num_q_heads=1, num_kv_heads=1, head_dim=d, policy="kvpop",
                    num_sink=s, protect_last=w, fp16_window=w, kvpop_k=k, old_int8=False)
    cache = OC.OracleCache(cfg)
    for t in range(steps):
        kv = rng.normal(size=(1, 1, 1, d)).astype(np.float16)
        pr = np.array([[[prio[t - w] if t - w >= 0 else 0.0]]], np.float32)
        cache.step(q=rng.normal(size=(1, 1, 1, d)), k_new=kv, v_new=kv, prio=pr)
        kept = cache.segs[0].pos.tolist()
        assert kept == KP.kept_closed_form(t, lambda p: prio[p], s, w, k)
        assert len(kept) == min(t + 1, KP.budget(s, w, k))


def test_budget_formula():
    assert KP.budget(4, 256, 1788) == 2048
