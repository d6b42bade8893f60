"""Next-token choice from the step's logits (float64). TEST INFRASTRUCTURE ONLY.

[Conf-KV post], decoding-loop pseudocode: after the cache update the next
token is drawn from the same p = softmax(logits) that the confidence reads.

Readings where the pages are silent:
* temperature 1, no truncation (p is the plain softmax of the logits);
* greedy decoding takes the largest logit, the lowest index among equal
  maxima;
* a random draw is an inverse-CDF draw with one uniform u in [0, 1) per batch
  row, handed in by the caller: the token is the smallest j whose cumulative
  probability p_0 + ... + p_j exceeds u;
* should u reach past the last cumulative sum through rounding, the draw is
  the last token with p_j > 0.
"""

from __future__ import annotations

import numpy as np


def greedy(logits) -> int:
    """argmax z, lowest index on ties."""
    z = np.asarray(logits, dtype=np.float32).ravel()
    if not np.all(np.isfinite(z)):
        raise ValueError("non-finite logits")
    m = z.max()
    return int(np.flatnonzero(z == m)[0])


def probabilities(logits) -> np.ndarray:
    """p = softmax(z) in float64, p_i = exp(z_i - m) / sum_j exp(z_j - m)."""
    z = np.asarray(logits, dtype=np.float64).ravel()
    if not np.all(np.isfinite(z)):
        raise ValueError("non-finite logits")
    e = np.exp(z - z.max())
    return e / e.sum()


def cdf(logits) -> np.ndarray:
    """Running sums p_0 + ... + p_j, accumulated in index order (numpy's
    cumulative sum adds one term at a time)."""
    return np.cumsum(probabilities(logits))


def draw(logits, u: float) -> int:
    """Smallest j with cdf_j > u (inverse-CDF sampling)."""
    if not 0.0 <= u < 1.0:
        raise ValueError("u must lie in [0, 1)")
    c = cdf(logits)
    above = np.flatnonzero(c > u)
    if above.size:
        return int(above[0])
    return int(np.flatnonzero(probabilities(logits) > 0.0)[-1])


def draw_is_valid(logits, u: float, j: int, eps: float) -> bool:
    """Whether token j is a correct draw for u once the cumulative sums may be
    off by eps (another summation order): cdf_{j-1} <= u + eps < ... and
    cdf_j > u - eps, with p_j > 0."""
    c = cdf(logits)
    p = probabilities(logits)
    lo = c[j - 1] if j > 0 else 0.0
    return bool(p[j] > 0.0 and lo <= u + eps and c[j] > u - eps)
