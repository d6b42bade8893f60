"""KVpop's multi-query mask and the masked prefill attention (float64).
TEST INFRASTRUCTURE ONLY.

[KVpop summary] §2.4: at inference the k long-range slots are chosen by a
running threshold over static per-token priorities (with a Fenwick tree),
which lets the sparse mask be generated inside the attention kernel rather
than stored as a dense S x S mask. §2.1 fixes the kept set: s sinks, the w
most recent tokens, and the top-k of the older ones.

Reading: a prefill (or teacher-forced pass) over S tokens whose priorities
are all known must let query q see exactly the rows a decode step at t = q
attends to. The decode step appends row q to the rows kept after step q - 1,
so (with the delayed-scoring reading of oracle/kvpop.py)

    allowed(q, j) = j <= q and (j < s or j >= q - w or j in topk(C_q)),
    C_q = [s, q - 1 - w],

top-k by (priority descending, position ascending). This module gives the
mask by brute force per query row, the same mask through a running threshold
over priority ranks (the form a kernel evaluates), and the masked attention
of every query head of a GQA group.
"""

from __future__ import annotations

import numpy as np


def descending_ranks(prio, num_sink):
    """rank[j] for j >= s: 0 for the highest (priority, -position), ascending
    from there; -1 for the sinks (they are never ranked)."""
    pr = np.asarray(prio, dtype=np.float32).ravel()
    S = pr.size
    order = sorted(range(num_sink, S), key=lambda j: (-float(pr[j]), j))
    rank = np.full(S, -1, dtype=np.int64)
    for r, j in enumerate(order):
        rank[j] = r
    return rank


def topk_long_range(prio, q, num_sink, window, k):
    """Positions of topk(C_q), C_q = [s, q-1-w] (brute force)."""
    pr = np.asarray(prio, dtype=np.float32).ravel()
    cand = list(range(num_sink, q - window))
    ranked = sorted(cand, key=lambda j: (-float(pr[j]), j))
    return set(ranked[:k])


def mask_brute_force(prio, num_sink, window, k):
    """Boolean [S, S]: row q, column j."""
    S = np.asarray(prio).size
    M = np.zeros((S, S), dtype=bool)
    for q in range(S):
        top = topk_long_range(prio, q, num_sink, window, k)
        for j in range(q + 1):
            M[q, j] = j < num_sink or j >= q - window or j in top
    return M


def running_thresholds(rank, S, num_sink, window, k):
    """thr[q] = the k-th smallest rank among C_q = [s, q-1-w], or S (every
    candidate passes) while |C_q| < k; -1 when k = 0 (none pass).

    Computed the way a kernel can, in one pass over q: C_q gains position
    q-1-w at query q; a present-set over ranks keeps the threshold, which
    only moves down once |C_q| >= k: an inserted rank below the threshold
    pushes it to the next present rank below.
    """
    thr = np.empty(S, dtype=np.int64)
    present = np.zeros(max(S, 1), dtype=bool)
    n = 0
    t = S  # threshold rank: S while fewer than k candidates
    for q in range(S):
        p = q - 1 - window
        if p >= num_sink:
            r = int(rank[p])
            present[r] = True
            n += 1
            if k > 0:
                if n == k:
                    t = max(i for i in range(S) if present[i])
                elif n > k and r < t:
                    t = max(i for i in range(t) if present[i])
        thr[q] = t if k > 0 else -1
    return thr


def mask_from_thresholds(rank, thr, num_sink, window):
    S = rank.size
    M = np.zeros((S, S), dtype=bool)
    for q in range(S):
        for j in range(q + 1):
            M[q, j] = j < num_sink or j >= q - window or rank[j] <= thr[q]
    return M


def masked_attention(q, K, V, mask, scale):
    """q [Hq][S][d], K/V [Hkv][S][d] (fp16 values), mask [S][S]; query head
    h*G + g uses KV head h. Returns out [Hq][S][d] and lse [Hq][S] (float64)."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    Hq, S, d = q.shape
    Hkv = K.shape[0]
    G = Hq // Hkv
    out = np.zeros((Hq, S, d))
    lse = np.zeros((Hq, S))
    for hq in range(Hq):
        h = hq // G
        s_ = (q[hq] @ K[h].T) * scale
        s_ = np.where(mask, s_, -np.inf)
        m = s_.max(axis=1, keepdims=True)
        e = np.exp(s_ - m)
        l = e.sum(axis=1, keepdims=True)
        out[hq] = (e / l) @ V[h]
        lse[hq] = m[:, 0] + np.log(l[:, 0])
    return out, lse


def future_attention_target(q, K, lse, window, scale):
    """[KVpop summary] §2.2: the scorer's training target for key position t
    is the log of the attention mass that future queries d >= t + w give it.
    With each query's log-sum-exp normaliser LSE handed in (the attention
    pass already produced it), the mass needs no softmax over a dense map:

        target[h, t] = log sum_{g < G} sum_{d = t + w}^{S - 1} exp(s[d, g, t] - LSE[d, g]),
        s[d, g, t] = scale * q[h*G + g, d] . k[h, t],

    summed over the G query heads of KV head h (-inf where no query counts).
    q [Hq][S][d], K [Hkv][S][d], lse [Hq][S]. Returns [Hkv][S] float64.
    Reading: the heads of a group add up, as the rows of one KV head's
    budget serve all of them."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    Hq, S, _ = q.shape
    Hkv = K.shape[0]
    G = Hq // Hkv
    d_idx = np.arange(S)[:, None]
    t_idx = np.arange(S)[None, :]
    future = d_idx >= t_idx + window                      # [query d, key t]
    out = np.full((Hkv, S), -np.inf)
    for h in range(Hkv):
        mass = np.zeros(S)
        for g in range(G):
            s_ = (q[h * G + g] @ K[h].T) * scale             # [d, t]
            p = np.where(future, np.exp(s_ - lse[h * G + g][:, None]), 0.0)
            mass += p.sum(axis=0)
        with np.errstate(divide="ignore"):
            out[h] = np.log(mass)
    return out
