"""GPU parity of the Euler step (h3_euler_update) and of the 50-block stack
with its Euler step, against the fp64 oracle.

* h3_euler_update: fp32 at the tiny workload and bf16 at the 4 s workload
  (25616 x 5376), with a coefficient per interval including zeros; rows of
  a zero-coefficient interval must come back bit for bit.
* The 50-block stack at tiny width (fp32, 72 tokens): the velocity (last
  block output) and the updated latent within 1e-5.  The stack is well
  conditioned (a 1e-7 relative change of the input moves the velocity by
  about 1e-7), so fp32 rounding over 50 blocks stays near 50 x 1e-7.
"""
import numpy as np
import pytest

import oracle
from video_audio_diffusion_amd import blk, inputs, sampler
from video_audio_diffusion_amd.block import BlockWeights, H3Stack, device_inputs, host_array

from gpu_util import TOL, assert_close, assert_delta_close

pytestmark = pytest.mark.gpu


def _dev(a):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.mark.parametrize("cfg_index,dtype", [(1, "f32"), (2, "bf16")])
def test_euler_update(cfg_index, dtype):
    import torch
    c = inputs.CONFIGS[cfg_index]
    N, D = c.n_tok, c.dim
    x = inputs.draw_rows(c, (N, D), seed=900 + cfg_index, dtype=dtype)
    v = inputs.draw_rows(c, (N, D), seed=910 + cfg_index, dtype=dtype)
    coef_vals = [0.0] + [-0.25 * (i + 1) for i in range(len(c.segments) - 1)]
    xd, vd = _dev(x), _dev(v)
    dt = blk.H3_BF16 if dtype == "bf16" else blk.H3_F32
    blk.h3_euler_update(xd, vd, N, D, blk.coefficients(coef_vals), blk.segments(c.segments), len(c.segments), dt)
    torch.cuda.synchronize()
    got = host_array(xd, dtype)
    s0 = c.segments[0]
    assert np.array_equal(got[s0.start:s0.start + s0.length], x[s0.start:s0.start + s0.length])
    rows = inputs.sample_rows(c, n_random=512) if N > 4096 else np.arange(N)
    coef = np.zeros(N)
    for s, cv in zip(c.segments, coef_vals):
        coef[s.start:s.start + s.length] = cv
    ref = oracle.euler_update(inputs.widen(x[rows], dtype), inputs.widen(v[rows], dtype), coef[rows])
    assert_close(f"euler_{dtype}", inputs.widen(got[rows], dtype), ref, TOL[dtype])


def test_tiny_stack_f32():
    import torch
    sc = inputs.STACK_TINY
    b = sc.block
    blocks = [inputs.make_stack_block(b, i) for i in range(sc.n_blocks)]
    x = inputs.make_inputs(b, ("x",))["x"]
    weights = []
    for t in blocks:
        d = device_inputs(b, t)
        weights.append(BlockWeights(d["w_qkv"], d["w_o"], d["w_gu"], d["w_d"], d["mod"], d["gamma_q"], d["gamma_k"]))
    stack = H3Stack(sc, weights)
    xd = _dev(x)
    stack.forward(xd)
    torch.cuda.synchronize()
    v_got = host_array(stack.block.buf["out"], b.dtype)
    x_got = host_array(xd, b.dtype)
    t64 = [{k: a.astype(np.float64) for k, a in t.items()} for t in blocks]
    x_ref, v_ref = oracle.stack_forward(x.astype(np.float64), t64, b, sc.step, sc.n_steps, dict(sc.shifts))
    assert_close("stack_velocity", v_got, v_ref, TOL["f32"])
    assert_close("stack_step", x_got, x_ref, TOL["f32"])
    assert_delta_close("stack_step_delta", x_got, x_ref, x, TOL["f32"], "f32")
    np.testing.assert_allclose(stack.coef_values,
                               [0.0, -0.02 / (1 + 2 * 0.98), -0.02 / (1 + 11 * 0.98)], rtol=0, atol=1e-15)
