"""Pins of the oracle's projections and SwiGLU."""
import math

import numpy as np
import torch
import torch.nn.functional as F

import oracle


def test_linear_triple_loop():
    g = np.random.default_rng(0)
    a, w = g.standard_normal((5, 7)), g.standard_normal((3, 7))
    got = oracle.linear(a, w)
    for i in range(5):
        for j in range(3):
            assert abs(got[i, j] - sum(a[i, k] * w[j, k] for k in range(7))) < 1e-12


def test_silu_closed_forms():
    assert oracle.silu(0.0) == 0.0
    assert abs(oracle.silu(1.0) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    assert abs(oracle.silu(1.0) - 0.7310585786300049) < 1e-15
    assert abs(oracle.silu(40.0) - 40.0) < 1e-12
    assert abs(oracle.silu(-40.0)) < 1e-15
    assert oracle.silu(-800.0) == 0.0
    z = np.linspace(-20, 20, 401)
    np.testing.assert_allclose(oracle.silu(z), F.silu(torch.from_numpy(z)).numpy(), rtol=1e-14, atol=1e-300)


def test_swiglu_gate_then_up():
    g = np.random.default_rng(1)
    F_ = 6
    gate, up = g.standard_normal((4, F_)), g.standard_normal((4, F_))
    got = oracle.swiglu(np.concatenate([gate, up], 1), F_)
    np.testing.assert_allclose(got, gate / (1 + np.exp(-gate)) * up, rtol=1e-15)
    ones = oracle.swiglu(np.concatenate([gate, np.ones((4, F_))], 1), F_)
    np.testing.assert_allclose(ones, oracle.silu(gate), rtol=0)
