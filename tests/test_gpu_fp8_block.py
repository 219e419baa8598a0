"""GPU parity of the FP8 block (H3BlockFP8) and of its two fused fp8
projections against the oracle.

* h3_gemm_fp8_gate_residual and h3_gemm_fp8_swiglu against the oracle's
  gated residual and SwiGLU of the oracle's product of the GPU's own codes
  and scales (the products are exact, the fp8 MFMA's sums carry about 2^-16,
  then one bf16 rounding): 4e-3 on the output, and on the branch delta
  beyond the output's own rounding; ragged shapes, several intervals, in
  place.
* The twelve calls of the block replayed with a buffer per intermediate
  (the driver's output must equal the replay bit for bit), each call
  against the oracle on the GPU's own inputs to it with that call's bound:
  quantisers bit for bit, fp8 products 4e-3, the fp8 attention 2^-4 (see
  test_gpu_fp8_attention), the bf16 norm / RoPE / AdaLN passes 2e-2.  At a
  ragged 117-token width-256 block, and at the 15 s 768p workload (92840
  tokens, full width) on sampled rows.
* End to end against the unquantised fp64 block (117 tokens): every
  quantised operand carries its own rounding, so the block's update out - x
  moves by the per-call bounds combined along each branch: attention branch
  sqrt(6e-2^2 (QKV) + 7.5e-2^2 (attention) + 6e-2^2 (output projection)) =
  0.113, FFN branch sqrt((sqrt(2) 6e-2)^2 (gate and up into SwiGLU) +
  6e-2^2 (down)) = 0.104; held to 0.12 in the Frobenius norm of out - x.
"""
import numpy as np
import pytest

import oracle
from fp8_layout import vt_key
from video_audio_diffusion_amd import blk, inputs
from video_audio_diffusion_amd.block import (BlockWeights, H3BlockFP8, device_inputs, host_array,
                                             interleave_gate_up)

from gpu_util import TOL, assert_close, assert_delta_close, make_device, oracle_inputs, widen

pytestmark = pytest.mark.gpu
TB = TOL["bf16"]
T8 = 4e-3          # fp8 product of the same codes, bf16 out
TOL_P = 2.0 ** -4  # fp8 attention against the attention of its dequantised operands
TOL_BLOCK = 0.12   # block update against the unquantised block


def _dev(a):
    return device_inputs(None, {"a": a})["a"]


def _quant(x_dev, K):
    import torch
    n = x_dev.shape[0]
    q = torch.empty(n, K, dtype=torch.uint8, device="cuda")
    s = torch.empty(n, dtype=torch.float32, device="cuda")
    blk.h3_quantize_fp8(x_dev, x_dev.stride(0), n, K, q, K, s, blk.H3_BF16)
    return q, s


def _segments(M, n_sets):
    cuts = sorted({0, M} | {max(1, min(M - 1, (M * i) // 5)) for i in range(1, 5)}) if M > 5 else [0, M]
    return [inputs.Segment(start=a, length=b - a, mod_set=(i * 3 + 1) % n_sets, T=b - a, kind="audio")
            for i, (a, b) in enumerate(zip(cuts[:-1], cuts[1:]))]


@pytest.mark.parametrize("M,N,K,n_sets,br,inplace", [(1, 8, 128, 1, 0, False), (300, 264, 384, 4, 0, True),
                                                     (257, 520, 256, 3, 1, False), (1280, 264, 1024, 2, 1, True)])
def test_gemm_fp8_gate_residual(M, N, K, n_sets, br, inplace):
    import torch
    a_h = inputs.draw_rows(None, (M, K), 61 + M, dtype="bf16")
    w_h = inputs.draw_rows(None, (N, K), 62 + N, dtype="bf16")
    x_h = inputs.draw_rows(None, (M, N), 63 + K, dtype="bf16")
    mod = np.random.Generator(np.random.PCG64(64)).standard_normal((n_sets, 6, N)).astype(np.float32)
    segs = _segments(M, n_sets)
    qa, sa = _quant(_dev(a_h), K)
    qw, sw = _quant(_dev(w_h), K)
    x = _dev(x_h)
    out = x if inplace else torch.full_like(x, float("nan"))
    blk.h3_gemm_fp8_gate_residual(qa, K, sa, qw, K, sw, x, out, N, M, N, K, _dev(mod), n_sets, br,
                                  blk.segments(segs), len(segs))
    torch.cuda.synchronize()
    y = oracle.gemm_fp8(qa.cpu().numpy(), sa.cpu().numpy(), qw.cpu().numpy(), sw.cpu().numpy())
    x64 = inputs.widen(x_h, "bf16")
    ref = oracle.gate_residual(x64, y, mod.astype(np.float64), br, segs)
    got = widen(out, "bf16")
    name = f"gemm_fp8_gate {M}x{N}x{K} sets{n_sets} br{br}{' inplace' if inplace else ''}"
    assert_close(name, got, ref, T8)
    assert_delta_close(name + " delta", got, ref, x64, T8, "bf16")


@pytest.mark.parametrize("M,F,K", [(1, 32, 128), (257, 96, 256), (300, 160, 384), (513, 288, 1024)])
def test_gemm_fp8_swiglu(M, F, K):
    import torch
    a_h = inputs.draw_rows(None, (M, K), 71 + M, dtype="bf16")
    w_h = inputs.draw_rows(None, (2 * F, K), 72 + F, dtype="bf16")
    il = np.asarray(blk.interleave_gate_up_rows(F))
    qa, sa = _quant(_dev(a_h), K)
    qw, sw = _quant(_dev(w_h), K)                      # plain [gate | up] rows; per-row codes permute with rows
    idx = torch.from_numpy(il).cuda()
    qw_il, sw_il = qw.index_select(0, idx).contiguous(), sw.index_select(0, idx).contiguous()
    H = torch.zeros(M, F, dtype=torch.bfloat16, device="cuda")
    blk.h3_gemm_fp8_swiglu(qa, K, sa, qw_il, K, sw_il, H, F, M, F, K)
    torch.cuda.synchronize()
    gu = oracle.gemm_fp8(qa.cpu().numpy(), sa.cpu().numpy(), qw.cpu().numpy(), sw.cpu().numpy())
    assert_close(f"gemm_fp8_swiglu {M}x{F}x{K}", widen(H, "bf16"), oracle.swiglu(gu, F), T8)


# ------------------------------------------------------------------ the block

def _small():
    return inputs.BlockConfig(
        name="ragged-bf16", index=11, dim=256, heads=2, head_dim=128, ffn=512, rope_split=(64, 32, 32),
        rope_base=10000.0, dtype="bf16", gamma=1.0,
        segments=inputs.pack([("text", 0, 7, 1, 1), ("audio", 2, 5, 1, 1), ("video", 1, 3, 5, 7)]))


def _block(cfg, dev):
    w = BlockWeights(dev["w_qkv"], dev["w_o"], dev["w_gu"], dev["w_d"], dev["mod"], dev["gamma_q"], dev["gamma_k"])
    return H3BlockFP8(cfg, interleave_gate_up(w, keep_plain=False))


def _replay(cfg, block, x):
    """The block's twelve calls with a separate buffer per intermediate
    (qkv_raw is the plain QKV product of the same codes, h3_gemm_fp8, which
    the fused call norms and rotates in its epilogue)."""
    import torch
    c, w, wq = cfg, block.w, block.wq
    N, D, H, d, I, F = c.n_tok, c.dim, c.heads, c.head_dim, c.inner, c.ffn
    segs, ns, nset = block.segs, block.n_segs, block.n_sets
    BF = blk.H3_BF16
    b16 = lambda *s: torch.empty(*s, dtype=torch.bfloat16, device="cuda")
    r = {"a": b16(N, D), "qkv": b16(N, 3 * I), "o": b16(N, I), "x1": b16(N, D), "a2": b16(N, D), "h": b16(N, F),
         "out": b16(N, D)}
    n_pad = block.n_pad
    r.update(q8=torch.empty(N, I, dtype=torch.uint8, device="cuda"), k8=torch.empty(N, I, dtype=torch.uint8, device="cuda"),
             vt=torch.empty(I, n_pad, dtype=torch.uint8, device="cuda"),
             sq=torch.empty(H, N, dtype=torch.float32, device="cuda"), sk=torch.empty(H, dtype=torch.float32, device="cuda"),
             sv=torch.empty(H, dtype=torch.float32, device="cuda"))
    blk.h3_adaln_modulate(x, r["a"], N, D, w.mod, nset, blk.H3_BRANCH_ATTN, segs, ns, c.eps, BF)
    r["a8"], r["sa"] = _quant(r["a"], D)
    # the plain product as well, for the GEMM's own check
    r["qkv_raw"] = b16(N, 3 * I)
    blk.h3_gemm_fp8(r["a8"], D, r["sa"], wq["qkv"][0], D, wq["qkv"][1], r["qkv_raw"], 3 * I, N, 3 * I, D, BF)
    blk.h3_gemm_fp8_qknorm_rope(r["a8"], D, r["sa"], wq["qkv"][0], D, wq["qkv"][1], r["qkv"], 3 * I, N, 3 * I, D, H, d,
                                w.gamma_q, w.gamma_k, c.eps, *c.rope_split, c.rope_base, segs, ns)
    q, k, v = r["qkv"][:, :I], r["qkv"][:, I:2 * I], r["qkv"][:, 2 * I:]
    blk.h3_quantize_qkv_fp8(q, k, v, 3 * I, N, H, d, r["q8"], r["k8"], r["vt"], n_pad, r["sq"], r["sk"], r["sv"], BF)
    blk.h3_attention_fp8(r["q8"], r["k8"], r["vt"], n_pad, r["sq"], r["sk"], r["sv"], r["o"], I, N, H, d, c.scale)
    r["o8"], r["so"] = _quant(r["o"], I)
    blk.h3_gemm_fp8_gate_residual(r["o8"], I, r["so"], wq["o"][0], I, wq["o"][1], x, r["x1"], D, N, D, I, w.mod, nset,
                                  blk.H3_BRANCH_ATTN, segs, ns)
    blk.h3_adaln_modulate(r["x1"], r["a2"], N, D, w.mod, nset, blk.H3_BRANCH_FFN, segs, ns, c.eps, BF)
    r["a28"], r["sa2"] = _quant(r["a2"], D)
    blk.h3_gemm_fp8_swiglu(r["a28"], D, r["sa2"], wq["gu"][0], D, wq["gu"][1], r["h"], F, N, F, D)
    r["h8"], r["sh"] = _quant(r["h"], F)
    blk.h3_gemm_fp8_gate_residual(r["h8"], F, r["sh"], wq["d"][0], F, wq["d"][1], r["x1"], r["out"], D, N, D, F,
                                  w.mod, nset, blk.H3_BRANCH_FFN, segs, ns)
    return r


def _select(t, rows):
    import torch
    if rows is None:
        return t
    return t.index_select(0, torch.from_numpy(np.asarray(rows, dtype=np.int64)).to(t.device))


def _host_rows(t, rows):
    return _select(t, rows).cpu().numpy()


def _b16(t, rows=None):
    return inputs.widen(host_array(_select(t, rows), "bf16"), "bf16")


def _check_calls(cfg, host, block, r, rows=None, attn_heads=None):
    """Every call against the oracle on the GPU's own inputs to it (on
    `rows` if given)."""
    c = cfg
    N, D, H, d, I, F = c.n_tok, c.dim, c.heads, c.head_dim, c.inner, c.ffn
    R = np.arange(N) if rows is None else np.asarray(rows)
    t = oracle_inputs(c, {k: host[k] for k in ("mod", "gamma_q", "gamma_k")})
    mod = t["mod"]
    _, pos = oracle.token_table(c.segments, N)
    wq = {k: (v[0].cpu().numpy(), v[1].cpu().numpy()) for k, v in block.wq.items()}
    x = inputs.widen(host["x"][R], "bf16")

    a = _b16(r["a"], rows)
    assert_close("adaln_attn", a, oracle.adaln_modulate(x, mod, 0, c.segments, c.eps, rows=R), TB)
    qa, sa = oracle.quantize_rows(a)
    assert np.array_equal(_host_rows(r["a8"], rows), qa) and np.array_equal(_host_rows(r["sa"], rows), sa)
    raw = _b16(r["qkv_raw"], rows)
    assert_close("gemm_fp8_qkv", raw, oracle.gemm_fp8(qa, sa, *wq["qkv"]), T8)
    assert np.array_equal(host_array(_select(r["qkv"], rows), "bf16")[:, 2 * I:],
                          host_array(_select(r["qkv_raw"], rows), "bf16")[:, 2 * I:]), "v differs from the plain product"
    qkv = _b16(r["qkv"], rows)
    for name, sl, gam in (("q", slice(0, I), t["gamma_q"]), ("k", slice(I, 2 * I), t["gamma_k"])):
        ref = oracle.rope3d(oracle.qk_rmsnorm(raw[:, sl], H, d, gam, c.eps), pos[R], H, d, c.rope_split, c.rope_base)
        assert_close("gemm_fp8_qknorm_rope_" + name, qkv[:, sl], ref, TB)

    # q/k/v codes: per-token q codes and scales on the rows; k and v with the
    # whole sequence's per-head scales
    q8, sq, _, _, _, _ = oracle.quantize_qkv(qkv[:, :I], qkv[:, I:2 * I], qkv[:, 2 * I:], H, d)
    assert np.array_equal(_host_rows(r["q8"], rows), q8)
    assert np.array_equal(r["sq"].cpu().numpy()[:, R], sq)
    sk, sv = r["sk"].cpu().numpy(), r["sv"].cpu().numpy()
    qkv_all = host_array(r["qkv"], "bf16")
    mag = (qkv_all.reshape(N, 3, H, d)[:, 1:] & 0x7FFF).max(axis=(0, 3))          # finite bf16: bits order like values
    amax = inputs.widen(mag.astype(np.uint16), "bf16").astype(np.float32)
    assert np.array_equal(sk, np.where(amax[0] > 0, amax[0] / np.float32(448), np.float32(1)).astype(np.float32))
    assert np.array_equal(sv, np.where(amax[1] > 0, amax[1] / np.float32(448), np.float32(1)).astype(np.float32))
    k8 = oracle.e4m3_encode((qkv[:, I:2 * I].reshape(-1, H, d).astype(np.float32) / sk[None, :, None]).reshape(len(R), I))
    assert np.array_equal(_host_rows(r["k8"], rows), k8)

    # attention on the dequantised codes, head by head over all keys
    o = _b16(r["o"], rows)
    heads = range(H) if attn_heads is None else attn_heads
    k8_all, vt_all, q8_rows = r["k8"].cpu().numpy(), r["vt"].cpu().numpy(), _host_rows(r["q8"], rows)
    src = (np.arange(block.n_pad) // 64) * 64 + vt_key(np.arange(block.n_pad) % 64)
    ok = src < N
    for hh in heads:
        sl = slice(hh * d, (hh + 1) * d)
        kd = oracle.e4m3_decode(k8_all[:, sl]) * float(sk[hh])
        vd = np.empty((N, d))
        vd[src[ok]] = oracle.e4m3_decode(vt_all[hh * d:(hh + 1) * d][:, ok].T) * float(sv[hh])
        qd = oracle.e4m3_decode(q8_rows[:, sl]) * r["sq"].cpu().numpy()[hh, R][:, None].astype(np.float64)
        ref = oracle.attention(qd, kd, vd, 1, d, c.scale)
        err = np.linalg.norm(o[:, sl] - ref) / np.linalg.norm(ref)
        err_v = np.abs(o[:, sl] - ref).max() / np.abs(vd).max()
        print(f"  attention_fp8 head {hh}: e_F={err:.3e} e_max/max|v|={err_v:.3e} (tol {TOL_P:g})", flush=True)
        assert err <= TOL_P and err_v <= TOL_P

    qo, so = oracle.quantize_rows(o)
    assert np.array_equal(_host_rows(r["o8"], rows), qo) and np.array_equal(_host_rows(r["so"], rows), so)
    x1 = _b16(r["x1"], rows)
    ref = oracle.gate_residual(x, oracle.gemm_fp8(qo, so, *wq["o"]), mod, 0, c.segments, rows=R)
    assert_close("gemm_fp8_o_gate", x1, ref, T8)
    assert_delta_close("gemm_fp8_o_gate delta", x1, ref, x, T8, "bf16")
    a2 = _b16(r["a2"], rows)
    assert_close("adaln_ffn", a2, oracle.adaln_modulate(x1, mod, 1, c.segments, c.eps, rows=R), TB)
    qa2, sa2 = oracle.quantize_rows(a2)
    assert np.array_equal(_host_rows(r["a28"], rows), qa2) and np.array_equal(_host_rows(r["sa2"], rows), sa2)
    il = np.asarray(blk.interleave_gate_up_rows(F))
    wgu, sgu = np.empty_like(wq["gu"][0]), np.empty_like(wq["gu"][1])
    wgu[il], sgu[il] = wq["gu"][0], wq["gu"][1]                     # back to [gate | up] row order
    h = _b16(r["h"], rows)
    assert_close("gemm_fp8_gu_swiglu", h, oracle.swiglu(oracle.gemm_fp8(qa2, sa2, wgu, sgu), F), T8)
    qh, sh = oracle.quantize_rows(h)
    assert np.array_equal(_host_rows(r["h8"], rows), qh) and np.array_equal(_host_rows(r["sh"], rows), sh)
    out = _b16(r["out"], rows)
    ref = oracle.gate_residual(x1, oracle.gemm_fp8(qh, sh, *wq["d"]), mod, 1, c.segments, rows=R)
    assert_close("gemm_fp8_d_gate", out, ref, T8)
    assert_delta_close("gemm_fp8_d_gate delta", out, ref, x1, T8, "bf16")


def test_small_fp8_block():
    import torch
    cfg = _small()
    host = inputs.make_inputs(cfg)
    dev = make_device(cfg, host)
    block = _block(cfg, dev)
    got = block.forward(dev["x"]).clone()
    r = _replay(cfg, block, dev["x"])
    torch.cuda.synchronize()
    assert torch.equal(got, r["out"]), "the driver and the call-by-call replay differ"
    _check_calls(cfg, host, block, r)
    ref = oracle.block_forward(oracle_inputs(cfg, host), cfg)
    x = inputs.widen(host["x"], "bf16")
    d_got, d_ref = widen(got, "bf16") - x, ref["out"] - x
    e_f = np.linalg.norm(d_got - d_ref) / np.linalg.norm(d_ref)
    print(f"  fp8 block update vs unquantised: e_F={e_f:.3e} (tol {TOL_BLOCK:g})", flush=True)
    assert e_f <= TOL_BLOCK


def test_fp8_block_in_place():
    """x may be the block's own output buffer (the stack feeds each block's
    output to the next)."""
    import torch
    cfg = _small()
    host = inputs.make_inputs(cfg)
    dev = make_device(cfg, host)
    block = _block(cfg, dev)
    ref = block.forward(dev["x"]).clone()
    block.buf["out"].copy_(dev["x"])
    block.forward(block.buf["out"])
    torch.cuda.synchronize()
    assert torch.equal(block.buf["out"], ref)


def test_768p15s_fp8_block_each_call():
    """The benchmark's FP8 workload: 92840 tokens at full width, every call
    on sampled rows; attention on 8 of the 56 heads over all keys (the
    kernel is checked on every head in test_gpu_fp8_attention)."""
    import torch
    c = inputs.CONFIGS[3]
    print(f"[c3 fp8] drawing inputs for {c.n_tok} tokens", flush=True)
    host = inputs.make_inputs(c)
    dev = make_device(c, host)
    block = _block(c, dev)
    print("[c3 fp8] running the block and the replay", flush=True)
    got = block.forward(dev["x"]).clone()
    r = _replay(c, block, dev["x"])
    torch.cuda.synchronize()
    assert torch.equal(got, r["out"])
    rows = inputs.sample_rows(c, n_random=48)
    _check_calls(c, host, block, r, rows=rows, attn_heads=(0, 7, 13, 22, 31, 40, 47, 55))


def test_small_fp8_stack():
    """Four FP8 blocks and the Euler step at the ragged 117-token width-256
    block: the stack's velocity equals the blocks run one after another (bit
    for bit); the Euler update of the GPU's own velocity against the oracle
    (bf16, 2e-2 on the delta beyond output rounding); and the stack's total
    update v - x against the unquantised fp64 stack within the block bound,
    since each block's quantisation error is its own."""
    import torch
    from video_audio_diffusion_amd.block import H3Stack
    b = _small()
    sc = inputs.StackConfig(name="stack4-ragged-bf16", block=b, n_blocks=4, description="fp8 stack parity")
    blocks = [inputs.make_stack_block(b, i) for i in range(sc.n_blocks)]
    x = inputs.make_inputs(b, ("x",))["x"]
    weights = []
    for t in blocks:
        d = device_inputs(b, t)
        weights.append(interleave_gate_up(BlockWeights(d["w_qkv"], d["w_o"], d["w_gu"], d["w_d"], d["mod"],
                                                       d["gamma_q"], d["gamma_k"]), keep_plain=False))
    stack = H3Stack(sc, weights, fp8=True)
    xd = _dev(x)
    stack.forward(xd)
    v = stack.block.buf["out"].clone()
    one = H3BlockFP8(b, stack.weights[0])
    h = _dev(x)
    for w in stack.weights:
        h = one.forward(h, weights=w).clone()
    torch.cuda.synchronize()
    assert torch.equal(v, h), "the stack differs from its blocks run one after another"
    coef = np.zeros(b.n_tok)
    for s, cv in zip(b.segments, stack.coef_values):
        coef[s.start:s.start + s.length] = cv
    x64, v64 = inputs.widen(x, "bf16"), widen(v, "bf16")
    ref = oracle.euler_update(x64, v64, coef)
    got = widen(xd, "bf16")
    assert_close("fp8 stack euler", got, ref, TB)
    assert_delta_close("fp8 stack euler delta", got, ref, x64, TB, "bf16")
    t64 = [{k: inputs.widen(a, "bf16") if a.dtype == np.uint16 else a.astype(np.float64) for k, a in t.items()}
           for t in blocks]
    _, v_ref = oracle.stack_forward(x64, t64, b, sc.step, sc.n_steps, dict(sc.shifts))
    e_f = np.linalg.norm((v64 - x64) - (v_ref - x64)) / np.linalg.norm(v_ref - x64)
    print(f"  fp8 stack update vs unquantised: e_F={e_f:.3e} (tol {TOL_BLOCK:g})", flush=True)
    assert e_f <= TOL_BLOCK
