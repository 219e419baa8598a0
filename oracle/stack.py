"""fp64 oracle of the 50-block backbone and one Euler step of the sampler.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources: "MiniMax-H3: native audio-video joint generation" notes, section
3.2 (50 backbone blocks), section 5 (an update mask separates generated
latents from fixed reference latents) and section 6 (video and audio follow
separately configured schedulers with shifts 12 and 3, and each takes an
Euler update from its velocity prediction).

Readings (the pages print no schedule and no output heads):
* time t falls from 1 to 0 in n_steps equal steps; a modality with shift s
  sits at noise level sigma(t) = s t / (1 + (s - 1) t), the rectified-flow
  time shift, which scales the odds sigma / (1 - sigma) by s;
* the velocity is the last block's output in hidden space;
* step k moves each target interval by (sigma(t_{k+1}) - sigma(t_k)) * v and
  leaves text and reference intervals unchanged.
"""
import numpy as np

from .block import block_forward


def shifted_sigma(t, shift):
    t = np.asarray(t, dtype=np.float64)
    return shift * t / (1.0 + (shift - 1.0) * t)


def euler_coefficients(segments, step, n_steps, shifts):
    """Per-token coefficient sigma(t_{k+1}) - sigma(t_k) (0 off the targets)."""
    n = segments[-1].start + segments[-1].length
    t0 = 1.0 - step / n_steps
    t1 = 1.0 - (step + 1) / n_steps
    c = np.zeros(n)
    for s in segments:
        if s.kind in shifts:
            c[s.start:s.start + s.length] = shifted_sigma(t1, shifts[s.kind]) - shifted_sigma(t0, shifts[s.kind])
    return c


def euler_update(x, v, coef):
    """x + coef[:, None] * v."""
    x = np.asarray(x, dtype=np.float64)
    return x + np.asarray(coef, dtype=np.float64)[:, None] * np.asarray(v, dtype=np.float64)


def stack_forward(x, blocks, cfg, step, n_steps, shifts):
    """Run every block (block b takes the dict blocks[b] of its weights,
    modulation table and gains) on x, then the Euler step.  Returns
    (x_next, v)."""
    h = np.asarray(x, dtype=np.float64)
    for t in blocks:
        h = block_forward(dict(t, x=h), cfg)["out"]
    c = euler_coefficients(cfg.segments, step, n_steps, shifts)
    return euler_update(x, h, c), h
