"""KVpop fixed budget: sinks + protected window + long-range top-k.

[KVpop summary] §2.1: each KV head keeps a bounded cache of B = s + w + k
rows: the first s tokens (attention sinks) are always kept, the w most recent
tokens are protected, and older tokens compete for k long-range slots by an
importance score. §2.3: a token is scored only when it leaves the protected
window (delayed scoring). §2.4: at inference the k slots are filled by a
running threshold over static per-token priorities.

The learned scorer is out of scope; its output is replaced by a given static
float32 priority per token. Reading of the delayed scoring: the priority of
the token at position t - w arrives at step t, the step on which that token
stops being protected. Long-range order: priority descending, then position
ascending (lower position kept on ties).
"""

from __future__ import annotations

import numpy as np


def budget(num_sink: int, window: int, k: int) -> int:
    """B = s + w + k ([KVpop summary] §2.1)."""
    return int(num_sink) + int(window) + int(k)


def long_range_victims(pos, prio32, t, num_sink, window, k):
    """Indices into pos of the long-range rows evicted at step t.

    The long-range set is R = {s <= pos <= t - w}. While |R| <= k nothing is
    evicted; otherwise the |R| - k rows of lowest (priority, then highest
    position) leave.
    """
    pos = np.asarray(pos, dtype=np.int64)
    pr = np.asarray(prio32, dtype=np.float32)
    R = [int(i) for i in np.nonzero((pos >= num_sink) & (pos <= t - window))[0]]
    if len(R) <= k:
        return np.zeros(0, dtype=np.int64)
    ranked = sorted(R, key=lambda i: (-float(pr[i]), int(pos[i])))
    return np.array(sorted(ranked[k:]), dtype=np.int64)


def kept_closed_form(t, prio_of_pos, num_sink, window, k):
    """History-free form of the same rule: after step t the kept positions
    are the sinks, the window (t-w, t], and the top-k by (priority desc,
    position asc) of every position in [s, t-w]. A priority is static and the
    candidate set only grows, so an evicted row can never re-enter the top-k
    and the incremental rule reaches exactly this set.

    prio_of_pos: callable pos -> float32 priority.
    """
    sinks = [p for p in range(0, min(num_sink, t + 1))]
    win = [p for p in range(max(num_sink, t - window + 1), t + 1)]
    cand = list(range(num_sink, t - window + 1))
    ranked = sorted(cand, key=lambda p: (-float(np.float32(prio_of_pos(p))), p))
    return sorted(set(sinks) | set(win) | set(ranked[:k]))
