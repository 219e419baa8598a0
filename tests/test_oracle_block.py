"""Block-level pins of the oracle (tiny fp32 workload, widened to fp64).

The pages print no numeric example of the block, so its values are pinned
through the step pins, these invariants, and an independent assembly of the
block from torch library routines (rms_norm, scaled_dot_product_attention,
silu, complex-number RoPE)."""
import numpy as np

import oracle
from torch_block import torch_block
from video_audio_diffusion_amd import inputs

CFG = inputs.CONFIGS[1]


def _t(cfg=CFG):
    raw = inputs.make_inputs(cfg)
    return {k: (inputs.widen(v, cfg.dtype) if k not in ("mod", "gamma_q", "gamma_k") else v.astype(np.float64))
            for k, v in raw.items()}


def test_zero_gates_give_identity_block():
    t = _t()
    t["mod"][:, 2] = 0.0
    t["mod"][:, 5] = 0.0
    r = oracle.block_forward(t, CFG)
    assert np.array_equal(r["out"], t["x"])


def test_zero_output_projections_give_identity_block():
    t = _t()
    t["w_o"][:] = 0.0
    t["w_d"][:] = 0.0
    assert np.array_equal(oracle.block_forward(t, CFG)["out"], t["x"])


def test_ffn_residual_starts_from_attention_residual():
    t = _t()
    t["w_d"][:] = 0.0
    r = oracle.block_forward(t, CFG)
    assert np.array_equal(r["out"], r["x1"])
    assert np.abs(r["x1"] - t["x"]).max() > 1e-3


def test_rows_mode_matches_full():
    t = _t()
    full = oracle.block_forward(t, CFG)
    rows = np.array([0, 15, 16, 23, 24, 50, 71])
    sub = oracle.block_forward(t, CFG, rows=rows)
    for key in ("a", "q_rope", "o", "x1", "gu", "out"):
        np.testing.assert_allclose(sub[key], full[key][rows], rtol=1e-12, atol=1e-12)


def test_segment_permutation_equivariance():
    t = _t()
    full = oracle.block_forward(t, CFG)["out"]
    for order in ((2, 0, 1), (1, 2, 0)):
        pcfg, rows = inputs.permuted(CFG, order)
        tp = dict(t)
        tp["x"] = t["x"][rows]
        got = oracle.block_forward(tp, pcfg)["out"]
        np.testing.assert_allclose(got, full[rows], rtol=1e-11, atol=1e-12)


def test_block_matches_library_assembly():
    t = _t()
    got = oracle.block_forward(t, CFG)["out"]
    ref = torch_block(t, CFG)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-11)
    # the same with a peaked softmax (Q/K gains 4, logits of std about 16)
    c2 = inputs.BlockConfig(**{**CFG.__dict__, "gamma": 4.0})
    t2 = _t(c2)
    np.testing.assert_allclose(oracle.block_forward(t2, c2)["out"], torch_block(t2, c2), rtol=1e-10, atol=1e-10)
