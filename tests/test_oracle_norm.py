"""Pins of the oracle's modulated norm, QK-norm and gated residual.

Special cases that reduce to a library routine or a closed form:
shift = scale = 0 is plain RMSNorm (torch rms_norm, fp64); a row with RMS 1
gives (1 + scale) * x + shift exactly; gate = 0 is the identity residual.
"""
import numpy as np
import torch
import torch.nn.functional as F

import oracle
from video_audio_diffusion_amd import inputs

CFG = inputs.CONFIGS[1]


def _mod(seed=0, zero=()):
    g = np.random.default_rng(seed)
    m = g.standard_normal((3, 6, CFG.dim))
    for c in zero:
        m[:, c, :] = 0.0
    return m


def test_zero_shift_scale_is_rmsnorm():
    x = np.random.default_rng(1).standard_normal((CFG.n_tok, CFG.dim)) * 3.0
    m = _mod(zero=(0, 1, 3, 4))
    for br in (oracle.BRANCH_ATTN, oracle.BRANCH_FFN):
        got = oracle.adaln_modulate(x, m, br, CFG.segments, 1e-6)
        ref = F.rms_norm(torch.from_numpy(x), (CFG.dim,), eps=1e-6).numpy()
        np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-13)
        rms = np.sqrt((oracle.adaln_modulate(x, m, br, CFG.segments, 0.0) ** 2).mean(axis=1))
        np.testing.assert_allclose(rms, 1.0, rtol=1e-13)


def test_unit_rms_row_closed_form():
    # rows of +-1 have RMS exactly 1, so with eps = 0 the norm is the identity
    sign = np.where(np.arange(CFG.dim) % 3 == 0, -1.0, 1.0)
    x = np.tile(sign, (CFG.n_tok, 1))
    m = _mod(seed=2)
    got = oracle.adaln_modulate(x, m, oracle.BRANCH_FFN, CFG.segments, 0.0)
    for s in CFG.segments:
        for i in range(s.start, s.start + s.length):
            want = x[i] * (1.0 + m[s.mod_set, 4]) + m[s.mod_set, 3]
            np.testing.assert_allclose(got[i], want, rtol=1e-15, atol=1e-15)


def test_two_element_rms():
    x = np.array([[3.0, 4.0]])
    got = oracle.rms_normalize(x, 0.5)
    np.testing.assert_allclose(got, x / np.sqrt(12.5 + 0.5), rtol=1e-15)


def test_interval_selects_its_modality_row():
    x = np.ones((CFG.n_tok, CFG.dim))
    m = np.zeros((3, 6, CFG.dim))
    for s in range(3):
        m[s, 0] = 10.0 * (s + 1)        # shift1 identifies the set
    got = oracle.adaln_modulate(x, m, oracle.BRANCH_ATTN, CFG.segments, 0.0)
    kinds = {inputs.MOD_TEXT: 10.0, inputs.MOD_AUDIO: 30.0, inputs.MOD_VISUAL: 20.0}
    for seg in CFG.segments:
        want = 1.0 + kinds[seg.mod_set]
        assert np.all(got[seg.start:seg.start + seg.length] == want), seg.kind


def test_branch_picks_its_chunks():
    x = np.random.default_rng(3).standard_normal((CFG.n_tok, CFG.dim))
    m = _mod(seed=4)
    m_attn_only = m.copy()
    m_attn_only[:, 3:6] = 99.0          # FFN chunks must not affect the attention branch
    a1 = oracle.adaln_modulate(x, m, oracle.BRANCH_ATTN, CFG.segments, 1e-6)
    a2 = oracle.adaln_modulate(x, m_attn_only, oracle.BRANCH_ATTN, CFG.segments, 1e-6)
    assert np.array_equal(a1, a2)
    y = np.random.default_rng(5).standard_normal(x.shape)
    g1 = oracle.gate_residual(x, y, m, oracle.BRANCH_ATTN, CFG.segments)
    g2 = oracle.gate_residual(x, y, m_attn_only, oracle.BRANCH_ATTN, CFG.segments)
    assert np.array_equal(g1, g2)


def test_gate_zero_identity_and_gate_one_sum():
    x = np.random.default_rng(6).standard_normal((CFG.n_tok, CFG.dim))
    y = np.random.default_rng(7).standard_normal((CFG.n_tok, CFG.dim))
    m = _mod(seed=8)
    m[:, 2] = 0.0
    m[:, 5] = 1.0
    assert np.array_equal(oracle.gate_residual(x, y, m, oracle.BRANCH_ATTN, CFG.segments), x)
    np.testing.assert_allclose(oracle.gate_residual(x, y, m, oracle.BRANCH_FFN, CFG.segments), x + y,
                               rtol=0, atol=0)


def test_gate_hand_example():
    x = np.array([[1.0, 2.0]] * 72)
    y = np.array([[10.0, 20.0]] * 72)
    m = np.zeros((3, 6, 2))
    m[:, 2, :] = [[0.5, -1.0], [2.0, 0.0], [0.0, 3.0]]
    c = inputs.CONFIGS[1]
    got = oracle.gate_residual(x, y, m, oracle.BRANCH_ATTN, c.segments)
    assert got[0].tolist() == [6.0, -18.0]          # text
    assert got[16].tolist() == [1.0, 62.0]          # audio (set 2)
    assert got[24].tolist() == [21.0, 2.0]          # video (set 1)


def test_qk_rmsnorm():
    H, d = 4, 64
    q = np.random.default_rng(9).standard_normal((50, H * d)) * 7.0
    out = oracle.qk_rmsnorm(q, H, d, np.ones(d), 0.0).reshape(50, H, d)
    np.testing.assert_allclose(np.sqrt((out ** 2).mean(axis=2)), 1.0, rtol=1e-13)
    # invariant to a positive per-row scale, equal to torch rms_norm per head
    out2 = oracle.qk_rmsnorm(q * 3.5, H, d, np.ones(d), 0.0).reshape(50, H, d)
    np.testing.assert_allclose(out2, out, rtol=1e-13)
    gamma = np.random.default_rng(10).standard_normal(d)
    got = oracle.qk_rmsnorm(q, H, d, gamma, 1e-6)
    ref = F.rms_norm(torch.from_numpy(q.reshape(50, H, d)), (d,), weight=torch.from_numpy(gamma), eps=1e-6)
    np.testing.assert_allclose(got, ref.reshape(50, H * d).numpy(), rtol=1e-13, atol=1e-13)
    # heads are normalized on their own: scaling one head leaves the others alone
    q2 = q.copy()
    q2[:, :d] *= 100.0
    o2 = oracle.qk_rmsnorm(q2, H, d, np.ones(d), 0.0)
    np.testing.assert_allclose(o2, oracle.qk_rmsnorm(q, H, d, np.ones(d), 0.0), rtol=1e-12)
