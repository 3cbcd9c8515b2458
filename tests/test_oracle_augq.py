"""Pins of the augmented-Q oracle (CPU).

SwiGLU gating and the three projections are checked against torch's silu
and matmul in float64 (independent library routines), a pure-Python brute
force on tiny shapes, closed forms of silu, and structural special cases.
"""

import math

import numpy as np
import torch

import oracle


def _w(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def test_silu_closed_forms():
    assert oracle.silu(0.0) == 0.0
    np.testing.assert_allclose(oracle.silu(1.0), 1.0 / (1.0 + math.exp(-1.0)), rtol=1e-15)
    np.testing.assert_allclose(oracle.silu(np.log(3.0)), np.log(3.0) * 0.75, rtol=1e-15)
    assert abs(oracle.silu(-50.0)) < 1e-19 and abs(oracle.silu(50.0) - 50.0) < 1e-19


def test_augq_matches_torch_float64():
    h, wg, wu, wd = _w(1, 5, 48), _w(2, 80, 48), _w(3, 80, 48), _w(4, 32, 80)
    q, a = oracle.augq(h, wg, wu, wd)
    t = lambda x: torch.from_numpy(x)
    g = t(h) @ t(wg).T
    ref_a = torch.nn.functional.silu(g) * (t(h) @ t(wu).T)
    ref_q = ref_a @ t(wd).T
    np.testing.assert_allclose(a, ref_a.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(q, ref_q.numpy(), rtol=1e-12, atol=1e-12)


def test_augq_brute_force_tiny():
    h, wg, wu, wd = _w(5, 2, 3), _w(6, 4, 3), _w(7, 4, 3), _w(8, 2, 4)
    q, _ = oracle.augq(h, wg, wu, wd)
    for m in range(2):
        acts = []
        for i in range(4):
            g = sum(h[m][j] * wg[i][j] for j in range(3))
            u = sum(h[m][j] * wu[i][j] for j in range(3))
            acts.append(g / (1 + math.exp(-g)) * u)
        for o in range(2):
            assert abs(q[m][o] - sum(acts[i] * wd[o][i] for i in range(4))) < 1e-12


def test_augq_structure():
    h, wg, wu, wd = _w(9, 3, 16), _w(10, 24, 16), _w(11, 24, 16), _w(12, 8, 24)
    q, a = oracle.augq(h, wg, wu, wd)
    # Linear in the up and down weights; a zero gate (silu(0) = 0) or a zero
    # up projection closes every channel.
    q2, _ = oracle.augq(h, wg, 2 * wu, wd)
    np.testing.assert_allclose(q2, 2 * q, rtol=1e-13)
    q3, _ = oracle.augq(h, wg, wu, -3 * wd)
    np.testing.assert_allclose(q3, -3 * q, rtol=1e-13)
    assert (oracle.augq(h, 0 * wg, wu, wd)[0] == 0).all()
    assert (oracle.augq(h, wg, 0 * wu, wd)[0] == 0).all()
    # Rows of h are independent tokens.
    q_row, _ = oracle.augq(h[1:2], wg, wu, wd)
    np.testing.assert_allclose(q_row[0], q[1], rtol=1e-13)
    # A gate far positive turns silu into the identity: a ~= g * u.
    big = 1e3
    _, a_big = oracle.augq(np.abs(h) + 1.0, big * np.abs(wg) + big, wu, wd)
    g = (np.abs(h) + 1.0) @ (big * np.abs(wg) + big).T
    u = (np.abs(h) + 1.0) @ wu.T
    np.testing.assert_allclose(a_big, g * u, rtol=1e-12)
