"""Pins of oracle.kvpop_prefill, the multi-query mask of a KVpop prefill.

* Each mask row equals the rows a decode step at t = q attends to: the
  history-free kept set after step q - 1 plus row q (oracle.kvpop, itself
  pinned to the step-by-step rule).
* The running-threshold form equals brute-force top-k per query row, with
  tied priorities, k = 0, tiny and huge k, w = 0 and sinks.
* Prefill attention under the mask equals the decode oracle's output at
  every step of a stream on the same rows, queries and priorities.
* The future-attention target: identical keys give harmonic sums in closed
  form; with causal normalisers the masses add up to the number of query
  rows; explicit loops agree.
"""

import numpy as np
import pytest

from oracle import cache as OC
from oracle import kvpop as KP
from oracle import kvpop_prefill as KPP


def prios(S, seed, ties=False):
    rng = np.random.default_rng(seed)
    p = rng.random(S).astype(np.float32)
    if ties:
        p = (np.floor(p * 4) / 4).astype(np.float32)  # four distinct values
    return p


@pytest.mark.parametrize("s,w,k,ties", [(0, 4, 5, False), (2, 4, 5, True), (1, 0, 3, True), (3, 6, 0, False),
                                        (0, 3, 100, False), (4, 8, 1, True)])
def test_mask_rows_are_the_decode_attention_sets(s, w, k, ties):
    S = 70
    p = prios(S, 11 + k, ties)
    M = KPP.mask_brute_force(p, s, w, k)
    for q in range(S):
        want = set(KP.kept_closed_form(q - 1, lambda j: p[j], s, w, k)) | {q}
        assert set(np.nonzero(M[q])[0].tolist()) == want, q


@pytest.mark.parametrize("s,w,k,ties", [(0, 4, 5, False), (2, 4, 5, True), (1, 0, 3, True), (3, 6, 0, False),
                                        (0, 3, 100, False), (4, 8, 1, True), (0, 0, 1, True)])
def test_running_threshold_equals_brute_force(s, w, k, ties):
    S = 90
    p = prios(S, 23 + w, ties)
    rank = KPP.descending_ranks(p, s)
    thr = KPP.running_thresholds(rank, S, s, w, k)
    assert np.array_equal(KPP.mask_from_thresholds(rank, thr, s, w), KPP.mask_brute_force(p, s, w, k))
    # the threshold only moves down, and each row holds at most s + w + 1 + k rows
    assert np.all(np.diff(thr) <= 0)
    assert KPP.mask_brute_force(p, s, w, k).sum(axis=1).max() <= s + w + 1 + k


def test_ranks_order_priorities_then_positions():
    p = np.array([0.5, 0.9, 0.5, 0.1, 0.9], dtype=np.float32)
    assert KPP.descending_ranks(p, 1).tolist() == [-1, 0, 2, 3, 1]


def test_prefill_attention_equals_decode_steps():
    # one layer, GQA 4/2, d 16; the prefill's query t must see what decode step t sees
    s, w, k, d, S, Hq, Hkv = 2, 5, 6, 16, 48, 4, 2
    rng = np.random.default_rng(3)
    Q = rng.normal(size=(Hq, S, d)).astype(np.float16)
    K = rng.normal(size=(Hkv, S, d)).astype(np.float16)
    V = rng.normal(size=(Hkv, S, d)).astype(np.float16)
    P = rng.random((Hkv, S)).astype(np.float32)
    P[:, 10:14] = P[:, 10:11]                         # ties
    scale = 1.0 / np.sqrt(d)
    outs, lses = [], []
    for h in range(Hkv):
        M = KPP.mask_brute_force(P[h], s, w, k)
        o, l = KPP.masked_attention(Q[h * 2:(h + 1) * 2], K[h:h + 1], V[h:h + 1], M, scale)
        outs.append(o)
        lses.append(l)
    out = np.concatenate(outs)
    cfg = OC.Config(num_layers=1, batch=1, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, policy="kvpop",
                    num_sink=s, protect_last=w, fp16_window=w, kvpop_k=k, old_int8=False)
    cache = OC.OracleCache(cfg)
    cache.init(0)
    for t in range(S):
        pr = np.zeros((1, 1, Hkv), np.float32)
        if t - w >= 0:
            pr[0, 0] = P[:, t - w]
        rec = cache.step(q=Q[None, None, :, t], k_new=K[None, None, :, t], v_new=V[None, None, :, t], prio=pr)
        for h in range(Hkv):
            np.testing.assert_allclose(rec.seg[h].out, out[h * 2:(h + 1) * 2, t], rtol=0, atol=1e-12)
            np.testing.assert_allclose(rec.seg[h].lse, np.concatenate(lses)[h * 2:(h + 1) * 2, t], rtol=0, atol=1e-12)


def test_masked_attention_without_eviction_is_causal_attention():
    # k at least S: nothing is ever cut, the mask is plain causal
    S, d = 20, 8
    rng = np.random.default_rng(4)
    p = rng.random(S).astype(np.float32)
    M = KPP.mask_brute_force(p, 0, 2, S)
    assert np.array_equal(M, np.tril(np.ones((S, S), dtype=bool)))


def causal_lse(q, K, scale):
    """LSE of plain causal attention, per query head: [Hq][S]."""
    Hq, S, _ = q.shape
    G = Hq // K.shape[0]
    out = np.zeros((Hq, S))
    for hq in range(Hq):
        s_ = (np.asarray(q[hq], np.float64) @ np.asarray(K[hq // G], np.float64).T) * scale
        s_ = np.where(np.tril(np.ones((S, S), bool)), s_, -np.inf)
        m = s_.max(axis=1)
        out[hq] = m + np.log(np.exp(s_ - m[:, None]).sum(axis=1))
    return out


def test_future_target_identical_keys_is_harmonic():
    # every key equal: causal attention is uniform, p(d, t) = 1/(d+1), so the
    # target is log(G * sum_{d=t+w}^{S-1} 1/(d+1))
    S, d, G, w = 30, 8, 3, 4
    rng = np.random.default_rng(9)
    q = rng.normal(size=(G, S, d))
    K = np.tile(rng.normal(size=(1, 1, d)), (1, S, 1))
    scale = 0.25
    lse = causal_lse(q, K, scale)
    tgt = KPP.future_attention_target(q, K, lse, w, scale)
    for t in range(S):
        if t + w < S:
            want = np.log(G * sum(1.0 / (dd + 1) for dd in range(t + w, S)))
            assert tgt[0, t] == pytest.approx(want, rel=1e-12, abs=1e-12)
        else:
            assert tgt[0, t] == -np.inf


def test_future_target_masses_add_up_to_the_rows():
    # with causal LSEs each query row sums to 1: the masses over all keys add
    # up to the number of (query, head) pairs whose keys lie at least w back
    S, d, Hq, Hkv, w = 25, 8, 4, 2, 3
    rng = np.random.default_rng(10)
    q = rng.normal(size=(Hq, S, d))
    K = rng.normal(size=(Hkv, S, d))
    scale = 1 / np.sqrt(d)
    lse = causal_lse(q, K, scale)
    tgt = KPP.future_attention_target(q, K, lse, 0, scale)
    assert np.exp(tgt).sum() == pytest.approx(Hq * S, rel=1e-12)
    # brute force with explicit loops for w > 0
    tw = KPP.future_attention_target(q, K, lse, w, scale)
    G = Hq // Hkv
    for h in range(Hkv):
        for t in range(S):
            m = 0.0
            for g in range(G):
                for dd in range(t + w, S):
                    m += np.exp(scale * float(np.dot(q[h * G + g, dd], K[h, t])) - lse[h * G + g, dd])
            assert (np.log(m) if m > 0 else -np.inf) == pytest.approx(tw[h, t], rel=1e-12, abs=1e-12)
