"""Per-token, per-head absmax INT8 quantizer, emulated with exact IEEE float32.

[CONF-KV abstract] and [Conf-KV post] keep the recent window in FP16 and store
older retained tokens as INT8. The pages fix neither the scale nor the rounding;
the reading taken (symmetric absmax, one float32 scale per token and head,
separately for keys and values, round to nearest even) is:

    amax  = max_j |x_j|                       (exact: fp16 -> fp32 widening)
    scale = fl32(amax / 127)                  (IEEE float32 division)
    code  = clamp(rne(fl32(x_j / scale)), -127, 127)
    amax == 0  ->  scale = 0, all codes 0
    dequantized value = fl32(code * scale)

NumPy float32 scalars and arrays divide and multiply with IEEE single
precision, so every step above is bit-exact float32 arithmetic.
"""

from __future__ import annotations

import numpy as np


def quantize_row(x16):
    """x16: float16 vector. Returns (codes int8 [d], scale float32)."""
    x = np.asarray(x16, dtype=np.float16).astype(np.float32)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
    if amax == np.float32(0):
        return np.zeros(x.shape, dtype=np.int8), np.float32(0)
    scale = np.float32(amax / np.float32(127.0))
    q = np.divide(x, scale, dtype=np.float32)
    code = np.clip(np.rint(q), -127, 127).astype(np.int8)
    return code, scale


def quantize_rows(x16):
    """Row-wise quantize_row over a [n, d] float16 array."""
    x16 = np.asarray(x16, dtype=np.float16)
    codes = np.zeros(x16.shape, dtype=np.int8)
    scales = np.zeros(x16.shape[0], dtype=np.float32)
    for i in range(x16.shape[0]):
        codes[i], scales[i] = quantize_row(x16[i])
    return codes, scales


def dequantize(codes, scales):
    """fl32(code * scale) per element; scales broadcast over the last axis."""
    c = np.asarray(codes, dtype=np.float32)
    s = np.asarray(scales, dtype=np.float32)
    if c.ndim == 2:
        s = s[:, None]
    return np.multiply(c, s, dtype=np.float32)
