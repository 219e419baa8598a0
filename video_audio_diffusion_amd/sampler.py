"""One Euler step of the flow sampler, as per-interval coefficients for
h3_euler_update.

[notes] section 6 ("MiniMax-H3: native audio-video joint generation"): video
and audio latents follow separately configured schedulers, with shifts 12 and
3, and each receives an Euler update from its velocity prediction; section 5:
an update mask keeps the fixed reference intervals as they are.  The pages do
not print the schedule, so it is read plainly: sampling time t runs from 1 to
0 in n_steps equal steps and each modality's noise level is the shifted time

    sigma(t) = s t / (1 + (s - 1) t),

the usual rectified-flow shift (it multiplies the odds sigma / (1 - sigma) by
s).  Step k then moves a target interval by sigma(t_{k+1}) - sigma(t_k) times
the velocity, and every other interval by 0.
"""
from __future__ import annotations

from typing import Dict, List, Sequence


def shifted_sigma(t: float, shift: float) -> float:
    return shift * t / (1.0 + (shift - 1.0) * t)


def step_times(step: int, n_steps: int):
    if not 0 <= step < n_steps:
        raise ValueError(f"step {step} outside [0, {n_steps})")
    return 1.0 - step / n_steps, 1.0 - (step + 1) / n_steps


def step_coefficients(segments: Sequence, step: int, n_steps: int, shifts: Dict[str, float]) -> List[float]:
    """sigma_next - sigma for every interval whose kind has a schedule, else 0."""
    t0, t1 = step_times(step, n_steps)
    out = []
    for s in segments:
        shift = shifts.get(s.kind)
        out.append(0.0 if shift is None else shifted_sigma(t1, shift) - shifted_sigma(t0, shift))
    return out
