"""End-to-end pins for oracle.cache: cases where the whole decode loop has a
closed form (no eviction -> plain attention over the history; pure recency ->
sliding window; uniform attention -> EMA series), checked against torch's
SDPA (float64, CPU, GQA grouping) and hand-derived values."""

import math

import numpy as np
import torch

from oracle import cache as OC
from oracle import quant as Q


def _cfg(**kw):
    base = dict(num_layers=1, batch=1, num_q_heads=4, num_kv_heads=2, head_dim=16, vocab=50, n_low=10 ** 6,
                n_high=10 ** 6, protect_last=2, fp16_window=10 ** 6, tau=0.6, alpha=0.5, ema_beta=0.9)
    base.update(kw)
    return OC.Config(**base)


def _sdpa_gqa(q, K, V):
    """q [Hq, d], K/V [Hkv, n, d] -> [Hq, d] via torch SDPA with GQA grouping."""
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q, dtype=torch.float64)[None, :, None, :], torch.tensor(K, dtype=torch.float64)[None],
        torch.tensor(V, dtype=torch.float64)[None], enable_gqa=True)
    return out[0, :, 0, :].numpy()


def _run(cfg, steps, seed=0, prefill=0, q_zero=False):
    rng = np.random.default_rng(seed)
    L, B, Hq, H, d = cfg.num_layers, cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    preK = rng.normal(size=(L, B, H, prefill, d)).astype(np.float16)
    preV = rng.normal(size=(L, B, H, prefill, d)).astype(np.float16)
    cache = OC.OracleCache(cfg)
    cache.init(prefill, lambda s: (preK[cache.coords(s)[0], cache.coords(s)[1], cache.coords(s)[2]],
                                   preV[cache.coords(s)[0], cache.coords(s)[1], cache.coords(s)[2]]))
    hist = []
    for i in range(steps):
        x = dict(logits=rng.normal(size=(B, cfg.vocab or 2)).astype(np.float32) * 8,
                 q=np.zeros((L, B, Hq, d), np.float16) if q_zero else rng.normal(size=(L, B, Hq, d)).astype(np.float16),
                 k_new=rng.normal(size=(L, B, H, d)).astype(np.float16),
                 v_new=rng.normal(size=(L, B, H, d)).astype(np.float16))
        rec = cache.step(**x)
        hist.append((x, rec))
    return cache, hist, preK, preV


def test_no_eviction_fp16_equals_full_attention_with_gqa():
    cfg = _cfg()
    _, hist, _, _ = _run(cfg, 12)
    Ks = np.zeros((2, 0, 16), np.float16)
    Vs = np.zeros((2, 0, 16), np.float16)
    for x, rec in hist:
        Ks = np.concatenate([Ks, x["k_new"][0, 0][:, None]], axis=1)
        Vs = np.concatenate([Vs, x["v_new"][0, 0][:, None]], axis=1)
        want = _sdpa_gqa(x["q"][0, 0].astype(np.float64), Ks.astype(np.float64), Vs.astype(np.float64))
        got = np.concatenate([rec.seg[0].out, rec.seg[1].out])
        assert np.abs(got - want).max() < 1e-12


def test_prefill_int8_split_and_attention():
    cfg = _cfg(fp16_window=5, num_kv_heads=4)
    cache, hist, preK, preV = _run(cfg, 6, prefill=9)
    t = 9
    for x, rec in hist:
        for h in range(4):
            seg = cache.segs[h] if (x, rec) is hist[-1] else None
            if seg is not None:
                assert seg.is8.tolist() == [p <= t - 5 for p in seg.pos]
        t += 1
    # first decode step: rows 0..3 were quantized at init (pos <= P0-1-W = 3)
    x, rec = hist[0]
    for h in range(4):
        k = preK[0, 0, h].copy().astype(np.float64)
        v = preV[0, 0, h].copy().astype(np.float64)
        for p in range(4):
            c, s = Q.quantize_row(preK[0, 0, h, p]); k[p] = Q.dequantize(c, s)
            c, s = Q.quantize_row(preV[0, 0, h, p]); v[p] = Q.dequantize(c, s)
        k = np.vstack([k, x["k_new"][0, 0, h].astype(np.float64)])
        v = np.vstack([v, x["v_new"][0, 0, h].astype(np.float64)])
        want = _sdpa_gqa(x["q"][0, 0, h:h + 1].astype(np.float64), k[None], v[None])
        assert np.abs(rec.seg[h].out - want).max() < 1e-12


def test_pure_recency_is_a_sliding_window():
    budget = 7
    cfg = _cfg(alpha=0.0, n_low=budget, n_high=budget, protect_last=3, num_kv_heads=4)
    cache, hist, _, _ = _run(cfg, 25)
    for t, (x, rec) in enumerate(hist):
        lo = max(0, t - budget)
        for h in range(4):
            assert rec.seg[h].pos.tolist() == list(range(lo, t + 1))         # attended rows
    for h in range(4):
        assert cache.segs[h].pos.tolist() == list(range(25 - budget, 25))


def test_ema_series_under_uniform_attention():
    # q = 0 gives every present row mass 1/n; with no eviction n = t+1, so a row
    # appended at step a has ema_t = sum_{j=a..t} (1-beta) beta^(t-j) / (j+1).
    beta = 0.9
    cfg = _cfg(ema_beta=beta)
    cache, hist, _, _ = _run(cfg, 15, q_zero=True)
    t = 14
    for a, e in zip(cache.segs[0].pos, cache.segs[0].ema):
        want = sum((1 - beta) * beta ** (t - j) / (j + 1) for j in range(a, t + 1))
        assert abs(e - want) < 1e-15


def test_budget_is_per_row_and_per_layer():
    # Row 0 gets confident logits (tight budget), row 1 flat ones (loose); the
    # pyramid shrinks the budget with depth.
    cfg = _cfg(num_layers=3, batch=2, n_low=6, n_high=12, protect_last=2, pyramid=True, num_kv_heads=1,
               num_q_heads=2, vocab=40)
    rng = np.random.default_rng(1)
    cache = OC.OracleCache(cfg)
    cache.init(0)
    for t in range(30):
        logits = np.zeros((2, 40), np.float32)
        logits[0, 3] = 30.0                       # one-hot-like -> c ~ 1
        x = dict(logits=logits, q=rng.normal(size=(3, 2, 2, 16)), k_new=rng.normal(size=(3, 2, 1, 16)),
                 v_new=rng.normal(size=(3, 2, 1, 16)))
        rec = cache.step(**x)
        assert rec.base == {0: 6, 1: 12}
    for l in range(3):
        tight = (6 * (3 * 2 - 2 * l)) // 4
        loose = (12 * (3 * 2 - 2 * l)) // 4
        assert len(cache.segs[(l * 2 + 0)]) == tight
        assert len(cache.segs[(l * 2 + 1)]) == loose


def test_protected_rows_always_survive_and_length_rule():
    cfg = _cfg(n_low=5, n_high=5, protect_last=4, num_sink=2, num_kv_heads=4)
    cache, hist, _, _ = _run(cfg, 40, seed=4)
    for t, (x, rec) in enumerate(hist):
        for h in range(4):
            r = rec.seg[h]
            kept = set(r.pos.tolist()) - set(r.victims.tolist())
            assert {p for p in r.pos if p < 2 or p > t - 4} <= kept
            n = len(r.pos)
            assert len(kept) == (n if n <= 5 else max(5, sum(1 for p in r.pos if p < 2 or p > t - 4)))
