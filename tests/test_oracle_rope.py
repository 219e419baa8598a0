"""Pins of the oracle's interval decode and 3-D MM-RoPE.

Closed forms (frequencies, a unit vector rotated by 1 rad), the 1-D RoFormer
formula in complex form, and the invariants: norm preservation, position 0
is the identity, R(p)R(p') = R(p + p'), and shifting every position by a
constant leaves all q.k dot products unchanged.
"""
import numpy as np

import oracle
from video_audio_diffusion_amd import inputs

H, d = 2, 64
SPLIT = (16, 24, 24)
BASE = 10000.0


def test_token_table_matches_unravel_index():
    for idx in (1, 2):
        c = inputs.CONFIGS[idx]
        mod_set, pos = oracle.token_table(c.segments, c.n_tok)
        for s in c.segments:
            l = np.arange(s.length)
            t, h, w = np.unravel_index(l, (s.T, s.H, s.W))
            assert np.array_equal(pos[s.start:s.start + s.length], np.stack([t, h, w], 1))
            assert np.all(mod_set[s.start:s.start + s.length] == s.mod_set)
    c = inputs.CONFIGS[1]
    _, pos = oracle.token_table(c.segments, c.n_tok)
    assert pos[15].tolist() == [15, 0, 0]     # last text token, time axis only
    assert pos[23].tolist() == [7, 0, 0]      # last audio token
    assert pos[24 + 6 * 4 + 6 + 5].tolist() == [1, 1, 5]


def test_inv_freq_closed_form():
    np.testing.assert_allclose(oracle.rope_inv_freq(4, 1e4), [1.0, 0.01], rtol=1e-15)
    np.testing.assert_allclose(oracle.rope_inv_freq(8, 1e4), [1.0, 0.1, 0.01, 0.001], rtol=1e-14)


def test_unit_vector_rotates_counterclockwise():
    x = np.zeros((1, d))
    x[0, 0] = 1.0                     # first t pair, freq 1
    got = oracle.rope3d(x, np.array([[1, 0, 0]]), 1, d, SPLIT, BASE)
    want = np.zeros(d)
    want[0], want[1] = np.cos(1.0), np.sin(1.0)
    np.testing.assert_allclose(got[0], want, atol=1e-15)
    y = np.zeros((1, d))
    y[0, 17] = 1.0                    # odd slot of the first h pair
    got = oracle.rope3d(y, np.array([[0, 2, 0]]), 1, d, SPLIT, BASE)
    want = np.zeros(d)
    want[16], want[17] = -np.sin(2.0), np.cos(2.0)
    np.testing.assert_allclose(got[0], want, atol=1e-15)


def test_t_chunk_is_complex_roformer():
    g = np.random.default_rng(0)
    x = g.standard_normal((5, d))
    pos = np.stack([np.arange(5) * 3, np.zeros(5, int), np.zeros(5, int)], 1)
    got = oracle.rope3d(x, pos, 1, d, SPLIT, BASE)
    z = x[:, 0:16:2] + 1j * x[:, 1:16:2]
    theta = 1.0 / BASE ** (np.arange(0, 16, 2) / 16.0)
    zr = z * np.exp(1j * pos[:, :1] * theta[None, :])
    np.testing.assert_allclose(got[:, 0:16:2], zr.real, atol=1e-13)
    np.testing.assert_allclose(got[:, 1:16:2], zr.imag, atol=1e-13)
    np.testing.assert_allclose(got[:, 16:], x[:, 16:], atol=0)     # h = w = 0: untouched


def test_axis_chunks_are_t_h_w_in_order():
    g = np.random.default_rng(1)
    x = g.standard_normal((3, d))
    pos = np.array([[5, 0, 0], [0, 5, 0], [0, 0, 5]])
    got = oracle.rope3d(x, pos, 1, d, SPLIT, BASE)
    changed = np.abs(got - x) > 1e-12
    assert changed[0, :16].any() and not changed[0, 16:].any()
    assert changed[1, 16:40].any() and not changed[1, :16].any() and not changed[1, 40:].any()
    assert changed[2, 40:].any() and not changed[2, :40].any()


def test_norm_preserved_and_zero_position_identity():
    g = np.random.default_rng(2)
    x = g.standard_normal((40, H * d))
    pos = g.integers(0, 100, size=(40, 3))
    got = oracle.rope3d(x, pos, H, d, SPLIT, BASE)
    pairs = lambda a: (a.reshape(40, -1, 2) ** 2).sum(-1)
    np.testing.assert_allclose(pairs(got), pairs(x), rtol=1e-12)
    assert np.array_equal(oracle.rope3d(x, np.zeros((40, 3), int), H, d, SPLIT, BASE), x)


def test_composition():
    g = np.random.default_rng(3)
    x = g.standard_normal((10, H * d))
    p1 = g.integers(0, 50, size=(10, 3))
    p2 = g.integers(0, 50, size=(10, 3))
    twice = oracle.rope3d(oracle.rope3d(x, p1, H, d, SPLIT, BASE), p2, H, d, SPLIT, BASE)
    once = oracle.rope3d(x, p1 + p2, H, d, SPLIT, BASE)
    np.testing.assert_allclose(twice, once, atol=1e-11)


def test_relative_position_invariance():
    g = np.random.default_rng(4)
    n = 24
    q = g.standard_normal((n, H * d))
    k = g.standard_normal((n, H * d))
    pos = g.integers(0, 60, size=(n, 3))
    shift = np.array([7, 3, 11])
    def scores(p):
        qr = oracle.rope3d(q, p, H, d, SPLIT, BASE).reshape(n, H, d)
        kr = oracle.rope3d(k, p, H, d, SPLIT, BASE).reshape(n, H, d)
        return np.einsum("ihd,jhd->hij", qr, kr)
    np.testing.assert_allclose(scores(pos + shift), scores(pos), atol=1e-10)
    # and the scores do depend on the relative offsets
    assert np.abs(scores(pos) - np.einsum("ihd,jhd->hij", q.reshape(n, H, d), k.reshape(n, H, d))).max() > 1e-3
