"""GPU parity on the tiny fp32 workload (hidden 192, 4 heads x 64, 72
tokens): every call and the whole block against the fp64 oracle at 1e-5."""
import numpy as np
import pytest

import oracle
from video_audio_diffusion_amd import blk, inputs

from gpu_util import TOL, assert_close, assert_delta_close, make_device, oracle_inputs, run_block_steps, widen

pytestmark = pytest.mark.gpu
CFG = inputs.CONFIGS[1]


@pytest.fixture(scope="module")
def state():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    blk.load()
    host = inputs.make_inputs(CFG)
    dev = make_device(CFG, host)
    print(f"[tiny] running block on {torch.cuda.get_device_name(0)}", flush=True)
    r = run_block_steps(CFG, dev)
    return host, dev, r


def test_steps_match_oracle(state):
    host, dev, r = state
    c = CFG
    t = oracle_inputs(c, host)
    W = lambda k: widen(r[k], c.dtype)
    tol = TOL[c.dtype]
    _, pos = oracle.token_table(c.segments, c.n_tok)
    assert_close("adaln_attn", W("a"), oracle.adaln_modulate(t["x"], t["mod"], 0, c.segments, c.eps), tol)
    assert_close("gemm_qkv", W("qkv_raw"), oracle.linear(W("a"), t["w_qkv"]), tol)
    raw = W("qkv_raw")
    I = c.inner
    qr = oracle.rope3d(oracle.qk_rmsnorm(raw[:, :I], c.heads, c.head_dim, t["gamma_q"], c.eps), pos, c.heads,
                       c.head_dim, c.rope_split, c.rope_base)
    kr = oracle.rope3d(oracle.qk_rmsnorm(raw[:, I:2 * I], c.heads, c.head_dim, t["gamma_k"], c.eps), pos,
                       c.heads, c.head_dim, c.rope_split, c.rope_base)
    qkv = W("qkv")
    assert_close("qknorm_rope_q", qkv[:, :I], qr, tol)
    assert_close("qknorm_rope_k", qkv[:, I:2 * I], kr, tol)
    assert np.array_equal(qkv[:, 2 * I:], raw[:, 2 * I:])      # v untouched
    assert_close("attention", W("o"), oracle.attention(qkv[:, :I], qkv[:, I:2 * I], qkv[:, 2 * I:], c.heads,
                                                       c.head_dim, c.scale), tol)
    assert_close("gemm_o", W("y"), oracle.linear(W("o"), t["w_o"]), tol)
    assert_close("gate_attn", W("x1"), oracle.gate_residual(t["x"], W("y"), t["mod"], 0, c.segments), tol)
    assert_close("adaln_ffn", W("a2"), oracle.adaln_modulate(W("x1"), t["mod"], 1, c.segments, c.eps), tol)
    assert_close("gemm_gu", W("gu"), oracle.linear(W("a2"), t["w_gu"]), tol)
    assert_close("swiglu", W("h"), oracle.swiglu(W("gu"), c.ffn), tol)
    assert_close("gemm_d", W("f"), oracle.linear(W("h"), t["w_d"]), tol)
    assert_close("gate_ffn", W("out"), oracle.gate_residual(W("x1"), W("f"), t["mod"], 1, c.segments), tol)


def test_block_matches_oracle(state):
    host, dev, r = state
    ref = oracle.block_forward(oracle_inputs(CFG, host), CFG)
    x = inputs.widen(host["x"], CFG.dtype)
    got = widen(r["out"], CFG.dtype)
    assert_close("block_out", got, ref["out"], TOL["f32"])
    assert_delta_close("block_delta", got, ref["out"], x, TOL["f32"], "f32")


def test_attention_lse(state):
    import torch
    host, dev, r = state
    c = CFG
    I = c.inner
    q, k, v = r["qkv"][:, :I], r["qkv"][:, I:2 * I], r["qkv"][:, 2 * I:]
    o = torch.empty(c.n_tok, I, dtype=torch.float32, device="cuda")
    lse = torch.empty(c.heads, c.n_tok, dtype=torch.float32, device="cuda")
    blk.h3_attention_fwd(q, k, v, 3 * I, o, I, c.n_tok, c.heads, c.head_dim, c.scale, lse, blk.H3_F32)
    torch.cuda.synchronize()
    qh = widen(q, "f32").reshape(c.n_tok, c.heads, c.head_dim)
    kh = widen(k, "f32").reshape(c.n_tok, c.heads, c.head_dim)
    s = np.einsum("ihd,jhd->hij", qh, kh) * c.scale
    ref = s.max(-1) + np.log(np.exp(s - s.max(-1, keepdims=True)).sum(-1))
    np.testing.assert_allclose(lse.cpu().numpy(), ref, rtol=1e-5, atol=1e-5)
    assert np.array_equal(o.cpu().numpy(), r["o"].cpu().numpy())


def test_zero_gate_is_bit_exact_identity(state):
    import torch
    host, dev, r = state
    c = CFG
    mod = dev["mod"].clone()
    mod[:, 2] = 0.0
    out = torch.empty_like(dev["x"])
    blk.h3_gate_residual(dev["x"], r["y"], out, c.n_tok, c.dim, mod, 3, blk.H3_BRANCH_ATTN,
                         blk.segments(c.segments), len(c.segments), blk.H3_F32)
    torch.cuda.synchronize()
    assert torch.equal(out, dev["x"])


def test_in_place_gate_residual(state):
    import torch
    host, dev, r = state
    c = CFG
    x = dev["x"].clone()
    blk.h3_gate_residual(x, r["y"], x, c.n_tok, c.dim, dev["mod"], 3, blk.H3_BRANCH_ATTN,
                         blk.segments(c.segments), len(c.segments), blk.H3_F32)
    torch.cuda.synchronize()
    assert torch.equal(x, r["x1"])
