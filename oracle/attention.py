"""Single-query decode attention over a segment's retained rows (float64).

[CONF-KV abstract] pairs the eviction policy with blockwise online-softmax
attention; [Conf-KV post] names the INT8 dequantization inside the attention
kernel as one of the hard parts. What the attention computes is plain softmax
attention of each query head of a GQA group against the segment's keys:

    s_gi = (q_g . k_i) * scale,   p_gi = exp(s_gi - LSE_g),   o_g = sum_i p_gi v_i

with scale = 1/sqrt(d). Three evaluation orders are given here — two-pass,
blockwise online (running max and sum, rescaled per block), and split with a
log-sum-exp combine — and the tests pin them equal to each other and to a
library routine. The step oracle uses the two-pass form.
"""

from __future__ import annotations

import numpy as np


def scores(q, K, scale):
    """s[g, i] = scale * q_g . k_i for q [G, d], K [n, d]."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    return (q @ K.T) * scale


def attend_two_pass(q, K, V, scale):
    """Two-pass softmax attention. Returns (o [G, d], lse [G], p [G, n])."""
    s = scores(q, K, scale)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    p = e / l
    o = p @ np.asarray(V, dtype=np.float64)
    lse = m[:, 0] + np.log(l[:, 0])
    return o, lse, p


def attend_online(q, K, V, scale, block):
    """Blockwise online softmax: one pass over blocks of rows, carrying a
    running max m, running sum l and unnormalized accumulator, rescaled by
    exp(m_old - m_new) whenever the max grows. Returns (o, lse)."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    G, d = q.shape
    m = np.full(G, -np.inf)
    l = np.zeros(G)
    acc = np.zeros((G, V.shape[1]))
    for start in range(0, K.shape[0], block):
        s = scores(q, K[start:start + block], scale)
        m_new = np.maximum(m, s.max(axis=1))
        corr = np.exp(m - m_new)
        e = np.exp(s - m_new[:, None])
        l = l * corr + e.sum(axis=1)
        acc = acc * corr[:, None] + e @ V[start:start + block]
        m = m_new
    return acc / l[:, None], m + np.log(l)


def attend_split(q, K, V, scale, num_splits):
    """Split the rows into contiguous parts, attend to each part alone, then
    merge the partial results through their log-sum-exps. Returns (o, lse)."""
    n = np.asarray(K).shape[0]
    bounds = np.linspace(0, n, num_splits + 1).astype(int)
    parts = []
    for a, b in zip(bounds[:-1], bounds[1:]):
        if b > a:
            o_i, lse_i, _ = attend_two_pass(q, K[a:b], V[a:b], scale)
            parts.append((o_i, lse_i))
    lses = np.stack([p[1] for p in parts])            # [S, G]
    lse = np.logaddexp.reduce(lses, axis=0)           # [G]
    w = np.exp(lses - lse[None, :])                   # [S, G]
    o = sum(w[i][:, None] * parts[i][0] for i in range(len(parts)))
    return o, lse


def attention_mass(p):
    """Attention mass a token receives in one step: the mean over the query
    heads of its GQA group of that head's softmax probability. Reading (the
    pages say only "attention mass"): eviction is per KV head, so the G query
    heads sharing a KV head are averaged; G = 1 is plain multi-head."""
    return np.asarray(p, dtype=np.float64).mean(axis=0)
