"""One H3-Omni-Transformer block forward as eleven libh3blk calls, as
seven with the fused projection epilogues, or (H3BlockFP8) as twelve with
FP8 projections and attention.

This driver only allocates device buffers (torch) and issues the calls in
the block order of the "MiniMax-H3: native audio-video joint generation"
notes, section 3; every step runs in the library's kernels.

Buffers (row-major, tokens as rows):
    a   [N, D]    modulated norm output (reused for a2)
    qkv [N, 3I]   [q heads | k heads | v heads]; q and k are normed and
                  rotated in place
    o   [N, I]    attention output
    y   [N, D]    projection output (reused for the FFN down projection)
    x1  [N, D]    residual after attention
    gu  [N, 2F]   [gate | up]
    h   [N, F]    SwiGLU output
    out [N, D]
The fused mode writes neither y nor gu and does not read q and k back: the
QKV projection norms and rotates q and k in its epilogue, the output and down
projections add their gated residual there, and the gate/up projection (its
weight rows interleaved once, `interleave_gate_up`) applies SwiGLU there.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Optional

from . import blk


@dataclass
class BlockWeights:
    w_qkv: object   # [3I, D]
    w_o: object     # [D, I]
    w_gu: object    # [2F, D]
    w_d: object     # [D, F]
    mod: object     # fp32 [n_sets, 6, D]
    gamma_q: object = None   # fp32 [head_dim] or None
    gamma_k: object = None
    w_gu_il: object = None   # [2F, D] w_gu rows in h3_gemm_swiglu's interleaved order


def interleave_gate_up(weights: BlockWeights, keep_plain: bool = True) -> BlockWeights:
    """Weights with the gate/up rows permuted into the 32-row interleave the
    fused SwiGLU projection reads (a one-time weight layout step,
    h3_interleave_gate_up on the current stream).  keep_plain=False drops
    the plain [gate | up] copy."""
    import dataclasses

    import torch
    w = weights.w_gu
    if w.dtype not in (torch.bfloat16, torch.float32) or w.dim() != 2 or w.stride(1) != 1:
        raise ValueError("w_gu must be a [2F, K] bf16 or fp32 matrix with unit column stride")
    F, K = w.shape[0] // 2, w.shape[1]
    il = torch.empty(2 * F, K, dtype=w.dtype, device=w.device)
    blk.h3_interleave_gate_up(w, w.stride(0), il, K, F, K, blk.H3_BF16 if w.dtype == torch.bfloat16 else blk.H3_F32)
    return dataclasses.replace(weights, w_gu_il=il, w_gu=w if keep_plain else None)


class H3Block:
    STEPS = ("adaln_attn", "gemm_qkv", "qknorm_rope", "attention", "gemm_o", "gate_attn",
             "adaln_ffn", "gemm_gu", "swiglu", "gemm_d", "gate_ffn")
    STEPS_FUSED = ("adaln_attn", "gemm_qkv_rope", "attention", "gemm_o_gate", "adaln_ffn", "gemm_gu_swiglu",
                   "gemm_d_gate")

    def __init__(self, cfg, weights: BlockWeights, device="cuda", fused: bool = False):
        import torch
        self.cfg = cfg
        self.w = weights
        self.fused = fused
        self.steps = self.STEPS_FUSED if fused else self.STEPS
        self.dt = blk.H3_BF16 if cfg.dtype == "bf16" else blk.H3_F32
        tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        N, D, I, F = cfg.n_tok, cfg.dim, cfg.inner, cfg.ffn
        e = lambda *s: torch.empty(*s, dtype=tdt, device=device)
        self.buf: Dict[str, object] = {"a": e(N, D), "qkv": e(N, 3 * I), "o": e(N, I), "x1": e(N, D),
                                       "h": e(N, F), "out": e(N, D)}
        if not fused:
            self.buf.update(y=e(N, D), gu=e(N, 2 * F))
        self.segs = blk.segments(cfg.segments)
        self.n_segs = len(cfg.segments)
        self.n_sets = int(weights.mod.shape[0])

    def forward(self, x, stream: Optional[int] = None, events=None, weights: Optional[BlockWeights] = None):
        """Run the block on x [N, D]; returns the `out` buffer.  x may be the
        `out` buffer itself (it is read before `out` is written).  `weights`
        replaces the block's own for this call; with `events` (a list of
        len(self.steps) + 1 torch.cuda.Event), event i is recorded before
        step i and the last one after the final step."""
        c, b = self.cfg, self.buf
        w = self.w if weights is None else weights
        if self.fused:
            return self._forward_fused(x, stream, events, w)
        N, D, H, d, I, F = c.n_tok, c.dim, c.heads, c.head_dim, c.inner, c.ffn
        dt, segs, ns, nset = self.dt, self.segs, self.n_segs, self.n_sets
        st = blk.current_stream() if stream is None else stream
        qkv = b["qkv"]
        q, k, v = qkv[:, :I], qkv[:, I:2 * I], qkv[:, 2 * I:]
        rec = (lambda i: events[i].record()) if events is not None else (lambda i: None)

        rec(0)
        blk.h3_adaln_modulate(x, b["a"], N, D, w.mod, nset, blk.H3_BRANCH_ATTN, segs, ns, c.eps, dt, st)
        rec(1)
        blk.h3_gemm_bf16(b["a"], D, w.w_qkv, D, qkv, 3 * I, N, 3 * I, D, dt, st)
        rec(2)
        blk.h3_qknorm_rope3d(q, k, 3 * I, N, H, d, w.gamma_q, w.gamma_k, c.eps, *c.rope_split, c.rope_base,
                             segs, ns, dt, st)
        rec(3)
        blk.h3_attention_fwd(q, k, v, 3 * I, b["o"], I, N, H, d, c.scale, None, dt, st)
        rec(4)
        blk.h3_gemm_bf16(b["o"], I, w.w_o, I, b["y"], D, N, D, I, dt, st)
        rec(5)
        blk.h3_gate_residual(x, b["y"], b["x1"], N, D, w.mod, nset, blk.H3_BRANCH_ATTN, segs, ns, dt, st)
        rec(6)
        blk.h3_adaln_modulate(b["x1"], b["a"], N, D, w.mod, nset, blk.H3_BRANCH_FFN, segs, ns, c.eps, dt, st)
        rec(7)
        blk.h3_gemm_bf16(b["a"], D, w.w_gu, D, b["gu"], 2 * F, N, 2 * F, D, dt, st)
        rec(8)
        blk.h3_swiglu(b["gu"], b["h"], N, F, dt, st)
        rec(9)
        blk.h3_gemm_bf16(b["h"], F, w.w_d, F, b["y"], D, N, D, F, dt, st)
        rec(10)
        blk.h3_gate_residual(b["x1"], b["y"], b["out"], N, D, w.mod, nset, blk.H3_BRANCH_FFN, segs, ns, dt, st)
        rec(11)
        return b["out"]

    def _forward_fused(self, x, stream, events, w):
        if w.w_gu_il is None:
            raise ValueError("the fused block needs interleaved gate/up weights (interleave_gate_up)")
        c, b = self.cfg, self.buf
        N, D, H, d, I, F = c.n_tok, c.dim, c.heads, c.head_dim, c.inner, c.ffn
        dt, segs, ns, nset = self.dt, self.segs, self.n_segs, self.n_sets
        st = blk.current_stream() if stream is None else stream
        qkv = b["qkv"]
        q, k, v = qkv[:, :I], qkv[:, I:2 * I], qkv[:, 2 * I:]
        rec = (lambda i: events[i].record()) if events is not None else (lambda i: None)

        rec(0)
        blk.h3_adaln_modulate(x, b["a"], N, D, w.mod, nset, blk.H3_BRANCH_ATTN, segs, ns, c.eps, dt, st)
        rec(1)
        blk.h3_gemm_qknorm_rope(b["a"], D, w.w_qkv, D, qkv, 3 * I, N, 3 * I, D, H, d, w.gamma_q, w.gamma_k, c.eps,
                                *c.rope_split, c.rope_base, segs, ns, dt, st)
        rec(2)
        blk.h3_attention_fwd(q, k, v, 3 * I, b["o"], I, N, H, d, c.scale, None, dt, st)
        rec(3)
        blk.h3_gemm_gate_residual(b["o"], I, w.w_o, I, x, b["x1"], D, N, D, I, w.mod, nset, blk.H3_BRANCH_ATTN,
                                  segs, ns, dt, st)
        rec(4)
        blk.h3_adaln_modulate(b["x1"], b["a"], N, D, w.mod, nset, blk.H3_BRANCH_FFN, segs, ns, c.eps, dt, st)
        rec(5)
        blk.h3_gemm_swiglu(b["a"], D, w.w_gu_il, D, b["h"], F, N, F, D, dt, st)
        rec(6)
        blk.h3_gemm_gate_residual(b["h"], F, w.w_d, F, b["x1"], b["out"], D, N, D, F, w.mod, nset,
                                  blk.H3_BRANCH_FFN, segs, ns, dt, st)
        rec(7)
        return b["out"]


def quantize_rows_fp8(w, stream: Optional[int] = None):
    """A bf16 [rows, K] device tensor -> (e4m3 codes [rows, K] uint8, fp32
    scale per row) by h3_quantize_fp8 (weights: one scale per output
    channel)."""
    import torch
    rows, K = w.shape
    q = torch.empty(rows, K, dtype=torch.uint8, device=w.device)
    sc = torch.empty(rows, dtype=torch.float32, device=w.device)
    blk.h3_quantize_fp8(w, w.stride(0), rows, K, q, K, sc, blk.H3_BF16, stream)
    return q, sc


@dataclass
class FP8Weights:
    """One block's weights for H3BlockFP8: e4m3 codes and fp32 per-output-
    channel scales of W_qkv, W_o, the interleaved W_gu and W_d (keys qkv, o,
    gu, d), plus the modulation table and the q/k gains as in BlockWeights."""
    q: Dict[str, object]
    mod: object
    gamma_q: object = None
    gamma_k: object = None


def quantize_block_weights(weights: BlockWeights) -> FP8Weights:
    """BlockWeights (with the interleaved gate/up copy) -> FP8Weights; a
    one-time weight step on the device."""
    if weights.w_gu_il is None:
        raise ValueError("the FP8 block needs interleaved gate/up weights (interleave_gate_up)")
    return FP8Weights({"qkv": quantize_rows_fp8(weights.w_qkv), "o": quantize_rows_fp8(weights.w_o),
                       "gu": quantize_rows_fp8(weights.w_gu_il), "d": quantize_rows_fp8(weights.w_d)},
                      weights.mod, weights.gamma_q, weights.gamma_k)


class H3BlockFP8:
    """The block with its four projections and its attention on FP8 (OCP
    e4m3) operands -- the quantised variant of the fused block: every GEMM
    input is quantised per row just before its GEMM (weights once, per
    output channel, at construction), q/k/v per token-head and per head; the
    norms, RoPE, the softmax's sums and every epilogue stay in fp32/bf16.

    Buffers beyond the fused block's: a8/sa (quantised a and a2), q8, k8,
    vt, sq, sk, sv (attention operands), o8/so, h8/sh.  bf16, head_dim 128,
    D, I and F multiples of 128."""

    STEPS = ("adaln_attn", "quant_a", "gemm_qkv_rope", "quant_qkv", "attention", "quant_o", "gemm_o_gate",
             "adaln_ffn", "quant_a2", "gemm_gu_swiglu", "quant_h", "gemm_d_gate")

    def __init__(self, cfg, weights, device="cuda"):
        """`weights`: BlockWeights (quantised here) or FP8Weights."""
        import torch
        if cfg.dtype != "bf16" or cfg.head_dim != 128 or any(v % 128 for v in (cfg.dim, cfg.inner, cfg.ffn)):
            raise ValueError("the FP8 block takes bf16, head_dim 128 and widths that are multiples of 128")
        self.cfg = cfg
        self.w = weights if isinstance(weights, FP8Weights) else quantize_block_weights(weights)
        self.wq = self.w.q
        self.dt = blk.H3_BF16
        self.steps = self.STEPS
        N, D, I, F, H = cfg.n_tok, cfg.dim, cfg.inner, cfg.ffn, cfg.heads
        self.n_pad = -(-N // 64) * 64
        b16 = lambda *sh: torch.empty(*sh, dtype=torch.bfloat16, device=device)
        u8 = lambda *sh: torch.empty(*sh, dtype=torch.uint8, device=device)
        f32 = lambda *sh: torch.empty(*sh, dtype=torch.float32, device=device)
        self.buf: Dict[str, object] = {
            "a": b16(N, D), "qkv": b16(N, 3 * I), "o": b16(N, I), "x1": b16(N, D), "h": b16(N, F), "out": b16(N, D),
            "a8": u8(N, D), "sa": f32(N), "q8": u8(N, I), "k8": u8(N, I), "vt": u8(I, self.n_pad),
            "sq": f32(H, N), "sk": f32(H), "sv": f32(H), "o8": u8(N, I), "so": f32(N), "h8": u8(N, F), "sh": f32(N)}
        self.segs = blk.segments(cfg.segments)
        self.n_segs = len(cfg.segments)
        self.n_sets = int(self.w.mod.shape[0])

    def forward(self, x, stream: Optional[int] = None, events=None, weights: Optional[FP8Weights] = None):
        """Run the block on x [N, D]; returns the `out` buffer (x may be it).
        `weights` replaces the block's own for this call.  With `events`
        (len(STEPS) + 1 torch.cuda.Event), event i is recorded before step i
        and the last after the final step."""
        c, b = self.cfg, self.buf
        w = self.w if weights is None else weights
        wq = w.q
        N, D, H, d, I, F = c.n_tok, c.dim, c.heads, c.head_dim, c.inner, c.ffn
        segs, ns, nset = self.segs, self.n_segs, self.n_sets
        BF = blk.H3_BF16
        st = blk.current_stream() if stream is None else stream
        qkv = b["qkv"]
        q, k, v = qkv[:, :I], qkv[:, I:2 * I], qkv[:, 2 * I:]
        rec = (lambda i: events[i].record()) if events is not None else (lambda i: None)

        rec(0)
        blk.h3_adaln_modulate(x, b["a"], N, D, w.mod, nset, blk.H3_BRANCH_ATTN, segs, ns, c.eps, BF, st)
        rec(1)
        blk.h3_quantize_fp8(b["a"], D, N, D, b["a8"], D, b["sa"], BF, st)
        rec(2)
        blk.h3_gemm_fp8_qknorm_rope(b["a8"], D, b["sa"], wq["qkv"][0], D, wq["qkv"][1], qkv, 3 * I, N, 3 * I, D, H, d,
                                    w.gamma_q, w.gamma_k, c.eps, *c.rope_split, c.rope_base, segs, ns, st)
        rec(3)
        blk.h3_quantize_qkv_fp8(q, k, v, 3 * I, N, H, d, b["q8"], b["k8"], b["vt"], self.n_pad, b["sq"], b["sk"],
                                b["sv"], BF, st)
        rec(4)
        blk.h3_attention_fp8(b["q8"], b["k8"], b["vt"], self.n_pad, b["sq"], b["sk"], b["sv"], b["o"], I, N, H, d,
                             c.scale, st)
        rec(5)
        blk.h3_quantize_fp8(b["o"], I, N, I, b["o8"], I, b["so"], BF, st)
        rec(6)
        blk.h3_gemm_fp8_gate_residual(b["o8"], I, b["so"], wq["o"][0], I, wq["o"][1], x, b["x1"], D, N, D, I, w.mod,
                                      nset, blk.H3_BRANCH_ATTN, segs, ns, st)
        rec(7)
        blk.h3_adaln_modulate(b["x1"], b["a"], N, D, w.mod, nset, blk.H3_BRANCH_FFN, segs, ns, c.eps, BF, st)
        rec(8)
        blk.h3_quantize_fp8(b["a"], D, N, D, b["a8"], D, b["sa"], BF, st)
        rec(9)
        blk.h3_gemm_fp8_swiglu(b["a8"], D, b["sa"], wq["gu"][0], D, wq["gu"][1], b["h"], F, N, F, D, st)
        rec(10)
        blk.h3_quantize_fp8(b["h"], F, N, F, b["h8"], F, b["sh"], BF, st)
        rec(11)
        blk.h3_gemm_fp8_gate_residual(b["h8"], F, b["sh"], wq["d"][0], F, wq["d"][1], b["x1"], b["out"], D, N, D, F,
                                      w.mod, nset, blk.H3_BRANCH_FFN, segs, ns, st)
        rec(12)
        return b["out"]


def device_inputs(cfg, host: Dict, device="cuda"):
    """Host arrays from `inputs.make_inputs` -> device tensors (bf16 bits are
    reinterpreted, not converted)."""
    import numpy as np
    import torch

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)

    out = {k: dev(v) for k, v in host.items()}
    return out


def host_array(t, dtype: str):
    """Device tensor -> host numpy (bf16 kept as uint16 bits)."""
    import numpy as np
    import torch
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


class H3Stack:
    """The backbone of n_blocks blocks and one Euler step of the sampler
    ([notes] section 3.2: 50 blocks; section 6: one velocity prediction per
    step).  The blocks share one set of activation buffers; the velocity is
    the last block's output, and h3_euler_update moves the target intervals
    of the input latent by the step's coefficients (sampler.py)."""

    def __init__(self, stack_cfg, weights, device="cuda", fused: bool = False, fp8: bool = False):
        """`weights`: one BlockWeights per block (interleaved gate/up copies
        for the fused and FP8 blocks) or, with fp8, FP8Weights.  With fp8
        every block is H3BlockFP8 and only the quantised weights are kept;
        BlockWeights given here are quantised as they are taken, so a caller
        that passes a generator never holds more than one block's bf16
        weights."""
        from . import sampler
        self.cfg = stack_cfg
        if fp8:
            self.weights = [w if isinstance(w, FP8Weights) else quantize_block_weights(w) for w in weights]
        else:
            self.weights = list(weights)
        if len(self.weights) != stack_cfg.n_blocks:
            raise ValueError(f"{len(self.weights)} weight sets for {stack_cfg.n_blocks} blocks")
        self.block = (H3BlockFP8(stack_cfg.block, self.weights[0], device) if fp8 else
                      H3Block(stack_cfg.block, self.weights[0], device, fused=fused))
        self.coef_values = sampler.step_coefficients(stack_cfg.block.segments, stack_cfg.step,
                                                     stack_cfg.n_steps, dict(stack_cfg.shifts))
        self.coef = blk.coefficients(self.coef_values)

    def forward(self, x, stream: Optional[int] = None, block_events=None):
        """Velocity of latent x [N, D] through every block, then x += coef * v
        in place; returns x.  With `block_events` (one list of
        len(self.block.steps) + 1 events per block) each block records its
        per-step events."""
        c = self.cfg.block
        st = blk.current_stream() if stream is None else stream
        h = x
        for i, w in enumerate(self.weights):
            h = self.block.forward(h, st, events=None if block_events is None else block_events[i], weights=w)
        blk.h3_euler_update(x, h, c.n_tok, c.dim, self.coef, self.block.segs, self.block.n_segs, self.block.dt, st)
        return x
