"""Pins of the oracle's attention: pure-Python brute force on tiny inputs,
torch scaled_dot_product_attention in fp64, and closed-form special cases."""
import math

import numpy as np
import torch
import torch.nn.functional as F

import oracle


def _brute(q, k, v, scale):
    """Explicit softmax attention with Python loops, one head."""
    n, m, dv = len(q), len(k), len(v[0])
    out = []
    for i in range(n):
        logits = [scale * sum(q[i][c] * k[j][c] for c in range(len(q[i]))) for j in range(m)]
        mx = max(logits)
        w = [math.exp(z - mx) for z in logits]
        tot = sum(w)
        out.append([sum(w[j] * v[j][c] for j in range(m)) / tot for c in range(dv)])
    return out


def test_brute_force_tiny():
    g = np.random.default_rng(0)
    H, d, n = 2, 8, 13
    q, k, v = (g.standard_normal((n, H * d)) for _ in range(3))
    got = oracle.attention(q, k, v, H, d, 0.37, chunk=5)
    for h in range(H):
        sl = slice(h * d, (h + 1) * d)
        want = _brute(q[:, sl].tolist(), k[:, sl].tolist(), v[:, sl].tolist(), 0.37)
        np.testing.assert_allclose(got[:, sl], np.array(want), rtol=1e-12, atol=1e-13)


def test_matches_torch_sdpa_fp64():
    g = np.random.default_rng(1)
    H, d, n = 4, 64, 128
    q, k, v = (g.standard_normal((n, H * d)) * 2 for _ in range(3))
    got = oracle.attention(q, k, v, H, d, 1 / 8.0, chunk=37)
    tq, tk, tv = (torch.from_numpy(a.reshape(n, H, d)).transpose(0, 1) for a in (q, k, v))
    ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=False).transpose(0, 1).reshape(n, H * d)
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-11, atol=1e-12)


def test_zero_query_gives_mean_of_values():
    g = np.random.default_rng(2)
    H, d, n = 2, 16, 40
    k, v = g.standard_normal((n, H * d)), g.standard_normal((n, H * d))
    got = oracle.attention(np.zeros((3, H * d)), k, v, H, d, 0.25, rows=np.array([0, 5, 9]))
    np.testing.assert_allclose(got, np.tile(v.mean(axis=0), (3, 1)), rtol=1e-13, atol=1e-14)


def test_dominant_key_selects_its_value():
    g = np.random.default_rng(3)
    H, d, n = 1, 16, 30
    k = g.standard_normal((n, d)) * 0.01
    k[17] = 50.0
    q = np.ones((2, d))
    v = g.standard_normal((n, d))
    got = oracle.attention(q, k, v, H, d, 1.0)
    np.testing.assert_allclose(got, np.tile(v[17], (2, 1)), atol=1e-12)


def test_probability_rows_sum_to_one_and_key_order_is_free():
    g = np.random.default_rng(4)
    H, d, n = 3, 32, 50
    q, k = g.standard_normal((n, H * d)) * 3, g.standard_normal((n, H * d)) * 3
    got = oracle.attention(q, k, np.ones((n, H * d)), H, d, 0.2)
    np.testing.assert_allclose(got, 1.0, rtol=1e-13)
    v = g.standard_normal((n, H * d))
    perm = g.permutation(n)
    a = oracle.attention(q, k, v, H, d, 0.2)
    b = oracle.attention(q, k[perm], v[perm], H, d, 0.2)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


def test_row_subset_equals_full():
    g = np.random.default_rng(5)
    H, d, n = 2, 32, 70
    q, k, v = (g.standard_normal((n, H * d)) for _ in range(3))
    rows = np.array([0, 3, 69, 40])
    full = oracle.attention(q, k, v, H, d, 0.3)
    sub = oracle.attention(q[rows], k, v, H, d, 0.3, rows=rows)
    np.testing.assert_allclose(sub, full[rows], rtol=1e-13)
