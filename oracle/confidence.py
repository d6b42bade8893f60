"""Confidence score and the gated per-step budget (float64).

Follows [Conf-KV post], method paragraph and decoding-loop pseudocode: the
next-token distribution p = softmax(logits) is mixed into one scalar from
three signals — normalized entropy, the sigmoid of the log-probability gap
between the two best candidates, and the top probability — with weights
0.4 / 0.3 / 0.3. [CONF-KV abstract] states the same three-way mix.

Readings where the pages are silent:
* natural log for the entropy; the base cancels in H / log V;
* V is the length of the logits vector handed in;
* temperature 1 (p is the plain softmax of the logits);
* margin = z(1) - z(2) on the logits, which equals log p(1) - log p(2)
  exactly and stays finite when p rounds to one-hot; a tied maximum gives 0;
* sigma is the logistic function.
"""

from __future__ import annotations

import math

import numpy as np

W_ENTROPY = 0.4
W_MARGIN = 0.3
W_PMAX = 0.3


def distribution_terms(logits):
    """Return (Hn, margin, pmax) of p = softmax(logits), all float64.

    H = -sum_i p_i log p_i with 0 log 0 = 0, written through log p_i = z_i - lse
    so that a p_i that underflows to 0 contributes exactly 0.
    """
    z = np.asarray(logits, dtype=np.float64).ravel()
    V = z.size
    if V < 2:
        raise ValueError("the confidence needs at least two candidates")
    m = z.max()
    lse = m + math.log(np.exp(z - m).sum())
    logp = z - lse
    p = np.exp(logp)
    H = -float(np.sum(np.where(p > 0.0, p * logp, 0.0)))
    Hn = H / math.log(V)
    top2 = np.sort(z)[-2:]
    margin = float(top2[1] - top2[0])
    pmax = math.exp(float(top2[1]) - lse)
    return Hn, margin, pmax


def sigmoid(x: float) -> float:
    if x >= 0:
        return 1.0 / (1.0 + math.exp(-x))
    e = math.exp(x)
    return e / (1.0 + e)


def confidence(logits, w_entropy=W_ENTROPY, w_margin=W_MARGIN, w_pmax=W_PMAX) -> float:
    """c = w_e (1 - H/log V) + w_m sigma(margin) + w_p p_max  ([Conf-KV post], pseudocode)."""
    Hn, margin, pmax = distribution_terms(logits)
    return w_entropy * (1.0 - Hn) + w_margin * sigmoid(margin) + w_pmax * pmax


def gate(c: float, tau: float, n_low: int, n_high: int, literal: bool = False) -> int:
    """Pick the step's base budget from the confidence.

    The prose of both CONF-KV pages says a confident step prunes hard (a tight
    budget) and an uncertain one keeps more context; the pseudocode's variable
    names say the opposite. Default reading (prose): c >= tau -> the smaller of
    the two budgets, c < tau -> the larger; c == tau counts as confident, as the
    pseudocode's comparison does. ``literal=True`` takes the pseudocode as
    printed (c >= tau -> n_high).
    """
    confident = c >= tau
    if literal:
        return int(n_high if confident else n_low)
    return int(min(n_low, n_high) if confident else max(n_low, n_high))


def layer_budget(base: int, layer: int, num_layers: int, pyramid: bool) -> int:
    """Per-layer budget. [Conf-KV post] and [CONF-KV abstract]: an optional
    pyramidal variant gives deeper layers smaller budgets. Reading: linear in
    depth from 1.5x the base at the first layer to 0.5x at the last, rounded
    down: floor(base * (3(L-1) - 2l) / (2(L-1))). One layer keeps the base.
    """
    if not pyramid or num_layers <= 1:
        return int(base)
    L1 = num_layers - 1
    return int((base * (3 * L1 - 2 * layer)) // (2 * L1))
