"""Pins for oracle.attention: the three evaluation orders agree, agree with
torch's scaled_dot_product_attention (float64, CPU), and hit closed forms."""

import numpy as np
import pytest
import torch

from oracle import attention as A


def _rand(n, G=4, d=64, seed=0, spread=3.0):
    rng = np.random.default_rng(seed)
    return rng.normal(size=(G, d)) * spread, rng.normal(size=(n, d)), rng.normal(size=(n, d))


@pytest.mark.parametrize("n", [1, 2, 7, 64, 301])
def test_orders_agree(n):
    q, K, V = _rand(n, seed=n)
    o2, lse2, p = A.attend_two_pass(q, K, V, 0.125)
    for block in (1, 5, 64):
        oo, lo = A.attend_online(q, K, V, 0.125, block)
        assert np.abs(oo - o2).max() < 1e-12 and np.abs(lo - lse2).max() < 1e-12
    for splits in (1, 2, 3, 7):
        if splits <= n:
            os_, ls = A.attend_split(q, K, V, 0.125, splits)
            assert np.abs(os_ - o2).max() < 1e-12 and np.abs(ls - lse2).max() < 1e-12
    assert np.abs(p.sum(axis=1) - 1).max() < 1e-12


@pytest.mark.parametrize("n,d", [(1, 64), (33, 64), (500, 128)])
def test_matches_library_sdpa(n, d):
    q, K, V = _rand(n, G=5, d=d, seed=11 + n)
    o, _, _ = A.attend_two_pass(q, K, V, 1 / np.sqrt(d))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q)[None, :, None, :], torch.tensor(K)[None, None].expand(1, 5, n, d),
        torch.tensor(V)[None, None].expand(1, 5, n, d))[0, :, 0, :].numpy()
    assert np.abs(o - ref).max() < 1e-12


def test_closed_forms():
    q, K, V = _rand(9)
    o, lse, _ = A.attend_two_pass(np.zeros_like(q), K, V, 0.3)      # q = 0: uniform weights
    assert np.abs(o - V.mean(axis=0)).max() < 1e-12 and np.abs(lse - np.log(9)).max() < 1e-12
    o, _, _ = A.attend_two_pass(q, K[:1], V[:1], 0.3)                 # one row: o = v
    assert np.abs(o - V[0]).max() < 1e-15
    K2 = K.copy()
    K2[4] = q[0] * 50                                                  # one dominant key for head 0
    o, _, p = A.attend_two_pass(q, K2, V, 1.0)
    assert abs(p[0, 4] - 1) < 1e-12 and np.abs(o[0] - V[4]).max() < 1e-10


def test_mass_is_group_mean():
    q, K, V = _rand(40, G=4)
    _, _, p = A.attend_two_pass(q, K, V, 0.2)
    m = A.attention_mass(p)
    assert abs(m.sum() - 1) < 1e-12                                   # a sum over heads would give G
    _, _, p1 = A.attend_two_pass(q[:1], K, V, 0.2)
    assert np.abs(A.attention_mass(p1) - p1[0]).max() == 0           # G = 1 is the head's own p
