"""Pins for oracle.quant: every code against exact rational arithmetic, plus
the absmax properties. float(Fraction) rounds the exact quotient correctly to
binary64, and rounding that to binary32 equals the correctly rounded binary32
quotient (p' = 53 >= 2p + 2 = 50, so double rounding is innocuous for
division); the code is then the round-half-even of that binary32 value."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import quant as Q


def _exact_codes(x16):
    x = [Fraction(float(v)) for v in np.asarray(x16, np.float16).astype(np.float32)]
    amax = max(abs(v) for v in x)
    if amax == 0:
        return [0] * len(x), 0.0
    scale = float(np.float32(float(amax / 127)))        # correctly rounded fp32 of amax/127
    codes = []
    for v in x:
        qf = float(np.float32(float(v / Fraction(scale))))
        fl = Fraction(qf)
        lo = fl.numerator // fl.denominator                 # floor
        rem = fl - lo
        r = lo + (1 if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1) else 0)
        codes.append(max(-127, min(127, r)))
    return codes, scale


@pytest.mark.parametrize("seed", range(6))
def test_codes_match_exact_arithmetic(seed):
    rng = np.random.default_rng(seed)
    x = (rng.normal(size=(8, 128)) * rng.choice([1e-3, 1.0, 30.0])).astype(np.float16)
    codes, scales = Q.quantize_rows(x)
    for i in range(x.shape[0]):
        want, s = _exact_codes(x[i])
        assert scales[i] == np.float32(s)
        assert codes[i].tolist() == want


def test_round_half_even():
    # amax 127 -> scale exactly 1, so x/scale is exact and x.5 cases are real ties.
    x = np.array([127, 2.5, 3.5, -2.5, -3.5, 0.5, -0.5, 1.5] + [0] * 56, dtype=np.float16)
    codes, scale = Q.quantize_row(x)
    assert scale == np.float32(1.0)
    assert codes[:8].tolist() == [127, 2, 4, -2, -4, 0, 0, 2]


def test_absmax_properties():
    rng = np.random.default_rng(9)
    for _ in range(50):
        x = (rng.normal(size=64) * 5).astype(np.float16)
        codes, scale = Q.quantize_row(x)
        xf = x.astype(np.float64)
        j = int(np.argmax(np.abs(xf)))
        assert abs(int(codes[j])) == 127 and np.sign(codes[j]) == np.sign(xf[j])
        assert codes.min() >= -127 and codes.max() <= 127
        deq = Q.dequantize(codes, scale).astype(np.float64)
        assert np.all(np.abs(deq - xf) <= float(scale) * (0.5 + 1e-6) + 1e-30)


def test_zero_row():
    codes, scale = Q.quantize_row(np.zeros(128, np.float16))
    assert scale == 0 and not codes.any()
    assert not Q.dequantize(codes, scale).any()
