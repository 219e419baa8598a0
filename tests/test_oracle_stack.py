"""Pins of the oracle's sampler step and 50-block stack, and of the host
schedule the product path passes to h3_euler_update.

Shifted schedule (a reading: the pages name the shifts, 12 for video and 3
for audio, but print no formula): sigma(t) = s t / (1 + (s - 1) t).  Pinned
by what any such time shift must satisfy -- identity at s = 1, the fixed end
points, odds scaled by exactly s, monotonicity -- and by hand values.
"""
import numpy as np
import pytest

import oracle
from torch_block import torch_block
from video_audio_diffusion_amd import inputs, sampler


def test_shift_one_is_identity_and_end_points_fixed():
    t = np.linspace(0.0, 1.0, 11)
    np.testing.assert_allclose(oracle.shifted_sigma(t, 1.0), t, rtol=0, atol=1e-15)
    for s in (3.0, 12.0):
        assert oracle.shifted_sigma(0.0, s) == 0.0
        assert oracle.shifted_sigma(1.0, s) == 1.0


def test_shift_scales_the_odds():
    t = np.linspace(0.05, 0.95, 19)
    for s in (3.0, 12.0):
        sig = oracle.shifted_sigma(t, s)
        np.testing.assert_allclose(sig / (1 - sig), s * t / (1 - t), rtol=1e-12)
        assert np.all(np.diff(sig) > 0) and np.all(sig >= t)


def test_hand_values():
    assert abs(oracle.shifted_sigma(0.5, 3.0) - 0.75) < 1e-15
    assert abs(oracle.shifted_sigma(0.98, 12.0) - 11.76 / 11.78) < 1e-15


def test_first_step_coefficients_closed_form():
    # step 0 of 50: sigma(t1) - sigma(1) = (t1 - 1) / (1 + (s - 1) t1), t1 = 0.98
    c = oracle.euler_coefficients(inputs.CONFIGS[3].segments, 0, 50, dict(inputs.TARGET_SHIFTS))
    text, audio, video = inputs.CONFIGS[3].segments
    assert np.all(c[text.start:text.start + text.length] == 0.0)
    assert abs(c[audio.start] - (-0.02 / (1 + 2 * 0.98))) < 1e-15
    assert abs(c[video.start] - (-0.02 / (1 + 11 * 0.98))) < 1e-15


def test_coefficients_telescope_to_minus_one():
    segs = inputs.CONFIGS[3].segments
    total = sum(oracle.euler_coefficients(segs, k, 50, dict(inputs.TARGET_SHIFTS)) for k in range(50))
    np.testing.assert_allclose(total[segs[1].start:], -1.0, rtol=0, atol=1e-12)
    assert np.all(total[:segs[1].start] == 0.0)


def test_reference_intervals_stay_fixed():
    segs = inputs.CONFIGS[4].segments
    c = oracle.euler_coefficients(segs, 7, 50, dict(inputs.TARGET_SHIFTS))
    for s in segs:
        part = c[s.start:s.start + s.length]
        if s.kind in ("video", "audio"):
            assert np.all(part < 0)
        else:
            assert np.all(part == 0.0), s.kind


def test_euler_update_is_x_plus_c_v():
    g = np.random.default_rng(3)
    x, v = g.standard_normal((6, 5)), g.standard_normal((6, 5))
    c = np.array([0.0, 1.0, -0.5, 0.0, 2.0, 0.25])
    out = oracle.euler_update(x, v, c)
    assert np.array_equal(out[[0, 3]], x[[0, 3]])
    np.testing.assert_allclose(out[1], x[1] + v[1], rtol=1e-15)
    np.testing.assert_allclose(out[2], x[2] - 0.5 * v[2], rtol=1e-15)


def test_stack_with_zero_gates_is_identity_then_scaled():
    """Every block is the identity when both gates are 0, so v = x and the
    step gives x (1 + c)."""
    c = inputs.STACK_TINY
    b = c.block
    x = inputs.widen(inputs.make_inputs(b, ("x",))["x"], b.dtype)
    blocks = []
    for i in range(3):
        t = {k: v.astype(np.float64) for k, v in inputs.make_stack_block(b, i).items()}
        t["mod"][:, 2] = 0.0
        t["mod"][:, 5] = 0.0
        blocks.append(t)
    xn, v = oracle.stack_forward(x, blocks, b, 0, 50, dict(c.shifts))
    assert np.array_equal(v, x)
    coef = oracle.euler_coefficients(b.segments, 0, 50, dict(c.shifts))
    np.testing.assert_allclose(xn, x * (1 + coef[:, None]), rtol=1e-15)


def test_host_schedule_matches_closed_form():
    """The product path's host coefficients (one per interval)."""
    segs = inputs.CONFIGS[3].segments
    got = sampler.step_coefficients(segs, 0, 50, dict(inputs.TARGET_SHIFTS))
    assert got[0] == 0.0
    assert abs(got[1] - (-0.02 / (1 + 2 * 0.98))) < 1e-15
    assert abs(got[2] - (-0.02 / (1 + 11 * 0.98))) < 1e-15
    tot = np.sum([sampler.step_coefficients(segs, k, 50, dict(inputs.TARGET_SHIFTS)) for k in range(50)], axis=0)
    np.testing.assert_allclose(tot, [0.0, -1.0, -1.0], atol=1e-12)
    with pytest.raises(ValueError):
        sampler.step_coefficients(segs, 50, 50, dict(inputs.TARGET_SHIFTS))


def _stack_blocks(b, n):
    """n blocks of the tiny stack, each with its own seeded weights and
    non-zero gates (fp64 copies)."""
    return [{k: (inputs.widen(v, b.dtype) if k.startswith("w_") else v.astype(np.float64))
             for k, v in inputs.make_stack_block(b, i).items()} for i in range(n)]


def test_stack_is_the_blocks_in_order_then_the_update_of_x():
    """Three blocks with distinct, non-zero gates: the velocity is the
    blocks applied one after another to x (assembled independently from
    torch library routines), and the step moves x -- the stack's input, not
    the velocity -- by coef * v."""
    c = inputs.STACK_TINY
    b = c.block
    x = inputs.widen(inputs.make_inputs(b, ("x",))["x"], b.dtype)
    blocks = _stack_blocks(b, 3)
    for t in blocks:   # both branches of every block contribute
        assert np.abs(t["mod"][:, 2]).mean() > 0.1 and np.abs(t["mod"][:, 5]).mean() > 0.1
    assert not np.array_equal(blocks[0]["w_qkv"], blocks[1]["w_qkv"])
    xn, v = oracle.stack_forward(x, blocks, b, 3, 50, dict(c.shifts))
    h = x
    for t in blocks:
        h = torch_block(dict(t, x=h), b)
    np.testing.assert_allclose(v, h, rtol=1e-10, atol=1e-10)
    # the update: hand-evaluated coefficients of step 3 (t 0.94 -> 0.92)
    t0, t1 = 0.94, 0.92
    sig = lambda t, s: s * t / (1 + (s - 1) * t)
    coef = np.zeros(b.n_tok)
    for s in b.segments:
        if s.kind in dict(c.shifts):
            sh = dict(c.shifts)[s.kind]
            coef[s.start:s.start + s.length] = sig(t1, sh) - sig(t0, sh)
    assert np.count_nonzero(coef) and np.count_nonzero(coef == 0.0)
    np.testing.assert_allclose(xn, x + coef[:, None] * h, rtol=1e-10, atol=1e-10)
    # an update applied to the velocity instead of x would differ
    assert np.abs((h + coef[:, None] * h) - xn).max() > 1e-2


def test_stack_order_matters():
    """The blocks differ, so running them in another order gives another
    velocity (a stack that ignored its order, or applied every block to the
    original x, would not see this)."""
    c = inputs.STACK_TINY
    b = c.block
    x = inputs.widen(inputs.make_inputs(b, ("x",))["x"], b.dtype)
    blocks = _stack_blocks(b, 3)
    _, v = oracle.stack_forward(x, blocks, b, 0, 50, dict(c.shifts))
    _, v_rev = oracle.stack_forward(x, blocks[::-1], b, 0, 50, dict(c.shifts))
    assert np.abs(v - v_rev).max() > 1e-2
    # applying every block to the original x and keeping the last is also different
    last_only = torch_block(dict(blocks[-1], x=x), b)
    assert np.abs(v - last_only).max() > 1e-2
