"""Ranking and eviction inside the chosen budget.

[Conf-KV post], method paragraph and pseudocode; [CONF-KV abstract]: within a
budget, tokens are ranked by a blend of recency and an exponential moving
average of the attention mass they received, alpha * ema + (1 - alpha) *
recency; a fixed window of the most recent tokens is never evicted; when a
layer holds more tokens than the budget, the lowest-ranked ones are dropped.

Readings where the pages are silent:
* EMA: ema <- beta * ema + (1 - beta) * mass, every present row (the new one
  included) each step; a row starts at 0 when appended and keeps its value
  through compaction.
* recency(pos, t) = (pos + 1) / (t + 1): linear, in (0, 1], 1 for the newest.
* Eviction is per (layer, batch row, KV head) segment; the budget counts the
  rows of one segment.
* Protected rows: sinks (pos < num_sink; none by default for CONF-KV) and
  the last P positions, pos > t - P, the new token included. If the budget
  is below the protected count, exactly the protected rows stay.
* Order: score descending, then position ascending — among equal scores the
  lower position is kept first. Scores are compared as float32 values (the
  precision the cache stores them in); -0.0 equals +0.0.

Rankers the Conf-KV post compares in its matched-rate ablation (the budget
schedule unchanged, only the choice of victims differs):
* recency only and attention only are alpha = 0 and alpha = 1 of the blend;
* random victims: each step every row gets a fresh uniform rank in [0, 1)
  and the lowest ranks go, so the victims are a uniform random subset of the
  candidates of the size the schedule fixes. The rank is drawn from a
  counter-based generator so that any (seed, t, segment, position) gives the
  same number on every implementation: SplitMix64 (Steele, Lea and Flood,
  "Fast splittable pseudorandom number generators", OOPSLA 2014), whose n-th
  output from seed k is mix64(k + n * 0x9E3779B97F4A7C15), chained as
  k1 = out(seed, t+1), k2 = out(k1, segment+1), x = out(k2, pos+1), and the
  rank is the top 24 bits of x times 2^-24 (exact in float32).
"""

from __future__ import annotations

import numpy as np


def ema_update(ema, mass, beta):
    return beta * np.asarray(ema, dtype=np.float64) + (1.0 - beta) * np.asarray(mass, dtype=np.float64)


def recency(pos, t):
    return (np.asarray(pos, dtype=np.float64) + 1.0) / (float(t) + 1.0)


def composite_score(ema, rec, alpha):
    return alpha * np.asarray(ema, dtype=np.float64) + (1.0 - alpha) * np.asarray(rec, dtype=np.float64)


def protected_mask(pos, t, num_sink, protect_last):
    pos = np.asarray(pos, dtype=np.int64)
    return (pos < num_sink) | (pos > t - protect_last)


def select_victims(pos, score32, t, budget, num_sink, protect_last):
    """Indices (into pos) of the rows evicted this step, ascending.

    No eviction unless the segment holds more rows than the budget. Otherwise
    keep every protected row plus the best (budget - #protected) of the rest
    by (score desc, pos asc), evict the remainder.
    """
    pos = np.asarray(pos, dtype=np.int64)
    n = pos.size
    if n <= budget:
        return np.zeros(0, dtype=np.int64)
    prot = protected_mask(pos, t, num_sink, protect_last)
    keep_free = max(0, int(budget) - int(prot.sum()))
    cand = [int(i) for i in np.nonzero(~prot)[0]]
    sc = np.asarray(score32, dtype=np.float32)
    ranked = sorted(cand, key=lambda i: (-float(sc[i]), int(pos[i])))
    return np.array(sorted(ranked[keep_free:]), dtype=np.int64)


_MASK64 = (1 << 64) - 1
GOLDEN_GAMMA = 0x9E3779B97F4A7C15


def mix64(z: int) -> int:
    """SplitMix64's output function (two xor-shift-multiply rounds and a final xor-shift)."""
    z &= _MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
    return z ^ (z >> 31)


def splitmix64(seed: int, n: int) -> int:
    """The n-th output (n >= 1) of SplitMix64 started from state `seed`."""
    return mix64((seed + n * GOLDEN_GAMMA) & _MASK64)


def random_rank(seed, t, segment, pos):
    """float32 uniform rank in [0, 1) of each position at step t of a segment."""
    k2 = splitmix64(splitmix64(int(seed), int(t) + 1), int(segment) + 1)
    out = [splitmix64(k2, int(p) + 1) >> 40 for p in np.asarray(pos, dtype=np.int64).ravel()]
    return np.asarray(out, dtype=np.float64).astype(np.float32) * np.float32(2.0 ** -24)
