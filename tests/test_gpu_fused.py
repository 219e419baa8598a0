"""GPU parity of the fused projection epilogues against the fp64 oracle.

* h3_gemm_gate_residual: out = x + gate[s(row)] * A.W^T with 1 to 6
  modulation sets, tiles inside one interval and tiles crossing several,
  both branches, in place and out of place, strided views, ragged M and N,
  bf16 and fp32.
* h3_gemm_swiglu: SiLU(gate) * up from the 32-row interleaved weight, F
  below and above one 256-column tile, ragged M, bf16 and fp32.
* The seven-call fused block (QKV projection with q/k norm and RoPE in its
  epilogue): end to end at a ragged 117-token width-256
  block, and at the 15 s 768p workload (92840 tokens, full width, the launch
  configuration the benchmark times) every call on sampled rows against the
  oracle applied to the GPU's own inputs to that call, attention over all
  keys of every head, and the whole block end to end on sampled rows
  against the oracle's block from the same input.
"""
import numpy as np
import pytest

import oracle
from video_audio_diffusion_amd import blk, inputs
from video_audio_diffusion_amd.block import BlockWeights, H3Block, device_inputs, host_array, interleave_gate_up

from gpu_util import TOL, assert_close, assert_delta_close, make_device, oracle_inputs, widen

pytestmark = pytest.mark.gpu


def _segments(M, n_sets):
    """Intervals of a 1-D sequence of M tokens cycling through the sets."""
    cuts = sorted({0, M} | {max(1, min(M - 1, (M * i) // 5)) for i in range(1, 5)}) if M > 5 else [0, M]
    segs = []
    for i, (a, b) in enumerate(zip(cuts[:-1], cuts[1:])):
        segs.append(inputs.Segment(start=a, length=b - a, mod_set=(i * 3 + 1) % n_sets, T=b - a, kind="audio"))
    return segs


def _dev(a):
    return device_inputs(None, {"a": a})["a"]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("M,N,K,n_sets,br,inplace,pad", [
    (1, 8, 64, 1, 0, False, 0), (300, 264, 128, 4, 0, True, 0), (257, 520, 192, 3, 1, False, 8),
    (513, 256, 64, 4, 1, True, 16), (1536, 512, 64, 6, 0, False, 0), (1280, 264, 128, 2, 1, True, 8),
    (300, 264, 8256, 3, 1, True, 8)])    # K past the LDS-DMA loop's limit: the register-staged loop
def test_gemm_gate_residual(dtype, M, N, K, n_sets, br, inplace, pad):
    import torch
    ldo = N + pad
    a_h = inputs.draw_rows(None, (M, K), 31 + M, dtype=dtype)
    w_h = inputs.draw_rows(None, (N, K), 32 + N, dtype=dtype)
    x_h = inputs.draw_rows(None, (M, ldo), 33 + K, dtype=dtype)
    mod = np.random.Generator(np.random.PCG64(34)).standard_normal((n_sets, 6, N)).astype(np.float32)
    segs = _segments(M, n_sets)
    A, W, x, modd = _dev(a_h), _dev(w_h), _dev(x_h), _dev(mod)
    dt = blk.H3_BF16 if dtype == "bf16" else blk.H3_F32
    out = x if inplace else torch.full_like(x, float("nan"))
    blk.h3_gemm_gate_residual(A, K, W, K, x, out, ldo, M, N, K, modd, n_sets, br, blk.segments(segs),
                              len(segs), dt)
    torch.cuda.synchronize()
    got = widen(out, dtype)
    x64 = inputs.widen(x_h, dtype)
    ref = oracle.gate_residual(x64[:, :N], oracle.linear(inputs.widen(a_h, dtype), inputs.widen(w_h, dtype)),
                               mod.astype(np.float64), br, segs)
    name = f"gemm_gate {dtype} {M}x{N}x{K} sets{n_sets} br{br}{' inplace' if inplace else ''}"
    assert_close(name, got[:, :N], ref, TOL[dtype])
    assert_delta_close(name + " delta", got[:, :N], ref, x64[:, :N], TOL[dtype], dtype)
    if pad:
        pad_got = host_array(out, dtype)[:, N:]
        if inplace:
            assert np.array_equal(pad_got, x_h[:, N:]), "columns beyond N were written"
        else:
            assert np.all(np.isnan(inputs.widen(pad_got, dtype))), "columns beyond N were written"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("M,F,K,pad", [(1, 32, 64, 0), (257, 96, 128, 0), (300, 160, 192, 8), (513, 288, 64, 0),
                                        (257, 96, 8256, 8)])
def test_gemm_swiglu(dtype, M, F, K, pad):
    import torch
    a_h = inputs.draw_rows(None, (M, K), 41 + M, dtype=dtype)
    w_h = inputs.draw_rows(None, (2 * F, K), 42 + F, dtype=dtype)
    il = np.asarray(blk.interleave_gate_up_rows(F))
    A, Wil = _dev(a_h), _dev(np.ascontiguousarray(w_h[il]))
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    H = torch.zeros(M, F + pad, dtype=tdt, device="cuda")
    dt = blk.H3_BF16 if dtype == "bf16" else blk.H3_F32
    blk.h3_gemm_swiglu(A, K, Wil, K, H, F + pad, M, F, K, dt)
    torch.cuda.synchronize()
    ref = oracle.swiglu(oracle.linear(inputs.widen(a_h, dtype), inputs.widen(w_h, dtype)), F)
    got = widen(H, dtype)
    assert_close(f"gemm_swiglu {dtype} {M}x{F}x{K}", got[:, :F], ref, TOL[dtype])
    assert np.all(got[:, F:] == 0), "columns beyond F were written"


def test_interleave_rows():
    rows = blk.interleave_gate_up_rows(64)
    assert rows[:32] == list(range(32)) and rows[32:64] == list(range(64, 96))
    assert rows[64:96] == list(range(32, 64)) and rows[96:] == list(range(96, 128))
    assert sorted(rows) == list(range(128))
    with pytest.raises(ValueError):
        blk.interleave_gate_up_rows(48)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("F,K,pad_src,pad_dst", [(32, 8, 0, 0), (96, 64, 8, 0), (288, 136, 0, 24), (14336, 64, 0, 8)])
def test_interleave_gate_up_copy(dtype, F, K, pad_src, pad_dst):
    """h3_interleave_gate_up moves every row whole to the slot the 32-row
    interleave names (bit-exact), strided source and destination; the
    padding columns of the destination stay as they were."""
    import torch
    ls, ld = K + pad_src, K + pad_dst
    w_h = inputs.draw_rows(None, (2 * F, ls), 40 + F, dtype=dtype)
    w = _dev(w_h)
    il = torch.full((2 * F, ld), -7.0, dtype=w.dtype, device="cuda")
    dt = blk.H3_BF16 if dtype == "bf16" else blk.H3_F32
    blk.h3_interleave_gate_up(w, ls, il, ld, F, K, dt)
    torch.cuda.synchronize()
    got = host_array(il, dtype)
    src = host_array(w, dtype)
    rows = np.asarray(blk.interleave_gate_up_rows(F))
    assert np.array_equal(got[:, :K].view(np.uint8), src[rows, :K].view(np.uint8))
    assert np.all(widen(il, dtype)[:, K:] == -7.0)


def _small():
    return inputs.BlockConfig(
        name="ragged-bf16", index=11, dim=256, heads=2, head_dim=128, ffn=512, rope_split=(64, 32, 32),
        rope_base=10000.0, dtype="bf16", gamma=1.0,
        segments=inputs.pack([("text", 0, 7, 1, 1), ("audio", 2, 5, 1, 1), ("video", 1, 3, 5, 7)]))


def _fused_block(cfg, dev):
    w = BlockWeights(dev["w_qkv"], dev["w_o"], dev["w_gu"], dev["w_d"], dev["mod"], dev["gamma_q"], dev["gamma_k"])
    return H3Block(cfg, interleave_gate_up(w, keep_plain=False), fused=True)


def test_small_fused_block():
    import torch
    cfg = _small()
    host = inputs.make_inputs(cfg)
    dev = make_device(cfg, host)
    block = _fused_block(cfg, dev)
    block.forward(dev["x"])
    torch.cuda.synchronize()
    ref = oracle.block_forward(oracle_inputs(cfg, host), cfg)
    x = inputs.widen(host["x"], "bf16")
    got = widen(block.buf["out"], "bf16")
    assert_close("fused_small_out", got, ref["out"], TOL["bf16"])
    assert_delta_close("fused_small_delta", got, ref["out"], x, TOL["bf16"], "bf16")
    assert_close("fused_small_x1", widen(block.buf["x1"], "bf16"), ref["x1"], TOL["bf16"])
    assert_close("fused_small_h", widen(block.buf["h"], "bf16"), ref["h"], TOL["bf16"])


def test_fused_block_in_place_matches_out_of_place():
    """x may be the block's own output buffer: the stack feeds each block's
    output to the next."""
    import torch
    cfg = _small()
    host = inputs.make_inputs(cfg)
    dev = make_device(cfg, host)
    block = _fused_block(cfg, dev)
    ref = block.forward(dev["x"]).clone()
    block.buf["out"].copy_(dev["x"])
    block.forward(block.buf["out"])
    torch.cuda.synchronize()
    assert torch.equal(block.buf["out"], ref)


C3 = inputs.CONFIGS[3]


def _rows(t, rows):
    import torch
    idx = torch.from_numpy(np.asarray(rows, dtype=np.int64)).to(t.device)
    return inputs.widen(host_array(t.index_select(0, idx), "bf16"), "bf16")


@pytest.fixture(scope="module")
def c3_run():
    """The benchmark's workload and launch configuration: the fused block at
    92840 tokens, run once; its buffers hold the last value of each: qkv
    (after norm and rotation), o, x1, a (= a2), h and out."""
    import torch
    print(f"[c3] drawing inputs for {C3.n_tok} tokens", flush=True)
    host = inputs.make_inputs(C3)
    dev = make_device(C3, host)
    block = _fused_block(C3, dev)
    print("[c3] running the fused block", flush=True)
    block.forward(dev["x"])
    torch.cuda.synchronize()
    return host, dev, block, inputs.sample_rows(C3, n_random=160)


def test_c3_fused_each_call(c3_run):
    """Every call of the fused block at 92840 tokens against the oracle
    applied to the GPU's own inputs to that call."""
    host, dev, block, rows = c3_run
    c = C3
    I, TB = c.inner, TOL["bf16"]
    b = block.buf
    t = oracle_inputs(c, {k: host[k] for k in ("mod", "gamma_q", "gamma_k")})
    mod = t["mod"]
    _, pos = oracle.token_table(c.segments, c.n_tok)
    x = inputs.widen(host["x"][rows], "bf16")

    a = oracle.adaln_modulate(x, mod, 0, c.segments, c.eps, rows=rows)
    raw = oracle.linear(a, inputs.widen(host["w_qkv"], "bf16"))
    qkv = _rows(b["qkv"], rows)
    for name, sl, gam in (("q", slice(0, I), t["gamma_q"]), ("k", slice(I, 2 * I), t["gamma_k"])):
        ref = oracle.rope3d(oracle.qk_rmsnorm(raw[:, sl], c.heads, c.head_dim, gam, c.eps), pos[rows],
                            c.heads, c.head_dim, c.rope_split, c.rope_base)
        assert_close("adaln_gemm_qknorm_rope_" + name, qkv[:, sl], ref, TB)
    assert_close("gemm_qkv_v", qkv[:, 2 * I:], raw[:, 2 * I:], TB)

    arows = rows[:: max(1, len(rows) // 32)]
    q = _rows(b["qkv"], arows)[:, :I]
    kv = host_array(b["qkv"][:, I:], "bf16")
    d = c.head_dim
    o_ref = np.empty((len(arows), I))
    for h in range(c.heads):
        kh = inputs.widen(kv[:, h * d:(h + 1) * d], "bf16")
        vh = inputs.widen(kv[:, I + h * d:I + (h + 1) * d], "bf16")
        o_ref[:, h * d:(h + 1) * d] = oracle.attention(q[:, h * d:(h + 1) * d], kh, vh, 1, d, c.scale)
    del kv
    assert_close("attention", _rows(b["o"], arows), o_ref, TB)

    o = _rows(b["o"], rows)
    x1 = _rows(b["x1"], rows)
    ref = oracle.gate_residual(x, oracle.linear(o, inputs.widen(host["w_o"], "bf16")), mod, 0, c.segments,
                               rows=rows)
    assert_close("gemm_o_gate", x1, ref, TB)
    assert_delta_close("gemm_o_gate delta", x1, ref, x, TB, "bf16")
    a2 = _rows(b["a"], rows)
    assert_close("adaln_ffn", a2, oracle.adaln_modulate(x1, mod, 1, c.segments, c.eps, rows=rows), TB)
    hh = _rows(b["h"], rows)
    assert_close("gemm_gu_swiglu", hh, oracle.swiglu(oracle.linear(a2, inputs.widen(host["w_gu"], "bf16")),
                                                      c.ffn), TB)
    out = _rows(b["out"], rows)
    ref = oracle.gate_residual(x1, oracle.linear(hh, inputs.widen(host["w_d"], "bf16")), mod, 1, c.segments,
                               rows=rows)
    assert_close("gemm_d_gate", out, ref, TB)
    assert_delta_close("gemm_d_gate delta", out, ref, x1, TB, "bf16")


def test_c3_fused_end_to_end(c3_run):
    """The whole fused block at 92840 tokens against the oracle's block from
    the same x: the oracle computes K and V for every token (about 1.4e13
    fp64 flop on the host) and every other step only for the sampled rows
    (rows are independent given K and V).  out and the block's update
    out - x within 2e-2 (the update beyond the bf16 rounding of out)."""
    host, dev, block, rows = c3_run
    c = C3
    print(f"[c3] oracle block on {len(rows)} rows (K and V for all {c.n_tok} tokens)", flush=True)
    ref = oracle.block_forward(oracle_inputs(c, host), c, rows=rows)
    x = inputs.widen(host["x"][rows], "bf16")
    b = block.buf
    assert_close("c3_block_out", _rows(b["out"], rows), ref["out"], TOL["bf16"])
    assert_delta_close("c3_block_delta", _rows(b["out"], rows), ref["out"], x, TOL["bf16"], "bf16")
    assert_close("c3_block_x1", _rows(b["x1"], rows), ref["x1"], TOL["bf16"])
    assert_close("c3_block_o", _rows(b["o"], rows), ref["o"], TOL["bf16"])
