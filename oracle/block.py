"""Plain fp64 statement of one H3-Omni-Transformer block forward.

TEST INFRASTRUCTURE ONLY (see the package docstring): slow, obviously correct,
numpy float64 throughout, no intermediate rounding, no blocking or fusion
beyond what a definition states.

Sources (cited by short name below):
  [notes]   "05 · MiniMax-H3: native audio-video joint generation"
            (note.shouss.top/research/video_generation/minimax_h3/)
  [reading] "MiniMax-H3 paper reading" (gojay.top/paper-reading/minimax-h3.html)

Block order, [notes] section 3 (the five-line block diagram):
  modulated norm -> shared self-attention -> modality gate + residual
  -> modulated norm -> shared gated FFN -> modality gate + residual.
Per-modality modulation picked per token interval: [notes] section 3.1.
Inner width 56 x 128 = 7168 differs from the residual width 5376; per-head
RMSNorm on Q and K before the positional encoding; SiLU(gate) * up FFN:
[notes] section 3.2 and the paragraph after its table.
3-D MM-RoPE, per-axis standard RoPE concatenated, audio/text on the time
axis with h = w = 0: [reading] sections 5 and 7.4.
Non-causal attention over all valid tokens: [notes] section 5.

Readings taken where the pages are silent (each is a parameter or a stated
convention, listed again in the design notes):
  * the modulated norm is RMSNorm without affine, eps 1e-6, modulated as
    norm(x) * (1 + scale) + shift;
  * the gate is applied as x + gate * branch;
  * AdaLN table layout [set][chunk][D], chunks (shift1, scale1, gate1,
    shift2, scale2, gate2), sets (text, visual, audio);
  * QK-norm: RMSNorm over each head's 128 values, eps 1e-6, gain [head_dim];
  * RoPE: RoFormer adjacent pairs (2j, 2j+1) inside each axis chunk, chunks
    ordered [t | h | w], frequency base^(-2j/d_axis);
  * token positions: video (t0 + l // (H*W), h0 + (l // W) % H, w0 + l % W),
    text/audio (t0 + l, 0, 0) with l the index inside the interval;
  * attention scale 1/sqrt(head_dim), no mask, no padding tokens;
  * no biases; W_qkv rows [q | k | v], W_gu rows [gate | up].
"""
from __future__ import annotations

import numpy as np

BRANCH_ATTN, BRANCH_FFN = 0, 1
SHIFT, SCALE, GATE = 0, 1, 2


# ------------------------------------------------------------ a0: intervals

def token_table(segments, n_tok):
    """Modality set and (t, h, w) position of every token of the packed
    sequence.  [notes] 2.2 keeps an index range per interval; [reading] 7.3
    flattens the (t, h, w) grid with t slowest; [reading] 7.4 puts text and
    audio on the time axis with h = w = 0."""
    mod_set = np.full(n_tok, -1, dtype=np.int64)
    pos = np.zeros((n_tok, 3), dtype=np.int64)
    for s in segments:
        for l in range(s.length):
            i = s.start + l
            if mod_set[i] != -1:
                raise ValueError("overlapping intervals")
            mod_set[i] = s.mod_set
            pos[i, 0] = s.t0 + l // (s.H * s.W)
            pos[i, 1] = s.h0 + (l // s.W) % s.H
            pos[i, 2] = s.w0 + l % s.W
    if (mod_set < 0).any():
        raise ValueError("intervals do not cover the sequence")
    return mod_set, pos


# ------------------------------------------------------------ a1 / a7

def rms_normalize(x, eps):
    """x / sqrt(mean(x^2) + eps) over the last axis."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def adaln_modulate(x, mod, branch, segments, eps, rows=None):
    """Modulated norm of [notes] section 3: normalize, then the token's own
    modality shift and scale (chosen by interval, [notes] 3.1)."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[0] if rows is None else None
    mod_set, _ = token_table(segments, sum(s.length for s in segments))
    sets = mod_set if rows is None else mod_set[rows]
    if n is not None and n != len(sets):
        raise ValueError("x rows do not match the intervals")
    mod = np.asarray(mod, dtype=np.float64)
    shift = mod[sets, 3 * branch + SHIFT, :]
    scale = mod[sets, 3 * branch + SCALE, :]
    return rms_normalize(x, eps) * (1.0 + scale) + shift


# ------------------------------------------------------------ a2 a5 a8 a10

def linear(a, w):
    """a . w^T, w stored [out, in] (no bias)."""
    return np.asarray(a, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T


# ------------------------------------------------------------ a3

def qk_rmsnorm(q, heads, head_dim, gamma, eps):
    """Per-head RMSNorm of [notes] 3.2: each head's head_dim values are
    normalized on their own, then multiplied by the gain."""
    q = np.asarray(q, dtype=np.float64).reshape(-1, heads, head_dim)
    out = rms_normalize(q, eps) * np.asarray(gamma, dtype=np.float64)
    return out.reshape(-1, heads * head_dim)


def rope_inv_freq(d_axis, base):
    """Standard RoPE frequencies base^(-2j/d_axis), j < d_axis/2."""
    j = np.arange(d_axis // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * j / d_axis)


def rope3d(x, pos, heads, head_dim, split, base):
    """3-D MM-RoPE ([reading] 7.4): the head dimension is cut into t, h and
    w chunks; each chunk gets standard 1-D RoPE driven by its own axis
    position, rotating adjacent pairs (2j, 2j+1) by pos * freq_j."""
    if sum(split) != head_dim or any(d % 2 for d in split):
        raise ValueError("RoPE split must be even and sum to head_dim")
    x = np.asarray(x, dtype=np.float64).reshape(-1, heads, head_dim)
    pos = np.asarray(pos, dtype=np.float64)
    out = x.copy()
    offset = 0
    for axis, d_axis in enumerate(split):
        if d_axis == 0:
            continue
        ang = pos[:, axis:axis + 1] * rope_inv_freq(d_axis, base)[None, :]   # [n, d_axis/2]
        c = np.cos(ang)[:, None, :]
        s = np.sin(ang)[:, None, :]
        even = x[:, :, offset:offset + d_axis:2]
        odd = x[:, :, offset + 1:offset + d_axis:2]
        out[:, :, offset:offset + d_axis:2] = even * c - odd * s
        out[:, :, offset + 1:offset + d_axis:2] = even * s + odd * c
        offset += d_axis
    return out.reshape(-1, heads * head_dim)


# ------------------------------------------------------------ a4

def attention(q, k, v, heads, head_dim, scale, rows=None, chunk=256):
    """Full bidirectional softmax attention per head ([notes] section 5:
    non-causal, every valid token sees every other).  q holds all tokens or,
    with `rows`, only the query rows listed there; k and v hold all tokens.
    The softmax is written out: subtract the row max, exponentiate, divide
    by the row sum."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64).reshape(-1, heads, head_dim)
    v = np.asarray(v, dtype=np.float64).reshape(-1, heads, head_dim)
    if rows is not None:
        q = q.reshape(len(rows), heads, head_dim)
    else:
        q = q.reshape(-1, heads, head_dim)
    out = np.empty_like(q)
    for h in range(heads):
        kh, vh = k[:, h, :], v[:, h, :]
        for c0 in range(0, q.shape[0], chunk):
            s = (q[c0:c0 + chunk, h, :] @ kh.T) * scale
            s -= s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            out[c0:c0 + chunk, h, :] = p @ vh
    return out.reshape(out.shape[0], heads * head_dim)


# ------------------------------------------------------------ a9

def silu(z):
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu(gu, ffn):
    """SiLU(gate) * up ([notes] 3.2); gu holds [gate | up] along columns."""
    gu = np.asarray(gu, dtype=np.float64)
    return silu(gu[:, :ffn]) * gu[:, ffn:2 * ffn]


# ------------------------------------------------------------ a6 / a11

def gate_residual(x, y, mod, branch, segments, rows=None):
    """Residual with the token's modality gate ([notes] section 3)."""
    mod_set, _ = token_table(segments, sum(s.length for s in segments))
    sets = mod_set if rows is None else mod_set[rows]
    gate = np.asarray(mod, dtype=np.float64)[sets, 3 * branch + GATE, :]
    return np.asarray(x, dtype=np.float64) + gate * np.asarray(y, dtype=np.float64)


# ------------------------------------------------------------ the block

def block_forward(t, cfg, rows=None):
    """One block forward in fp64.

    `t` maps x, mod, w_qkv, w_o, w_gu, w_d, gamma_q, gamma_k to float64
    arrays.  With `rows` given, K and V are computed for every token (each
    query row needs all of them) and everything else only for the listed
    rows.  Returns every intermediate, keyed by the step it ends."""
    D, H, d, F = cfg.dim, cfg.heads, cfg.head_dim, cfg.ffn
    I = H * d
    segs = cfg.segments
    n = cfg.n_tok
    mod_set, pos = token_table(segs, n)
    x = np.asarray(t["x"], dtype=np.float64)
    w_qkv = np.asarray(t["w_qkv"], dtype=np.float64)
    r = np.arange(n) if rows is None else np.asarray(rows)

    a_all = adaln_modulate(x, t["mod"], BRANCH_ATTN, segs, cfg.eps)
    kv = linear(a_all, w_qkv[I:3 * I])
    k_all = rope3d(qk_rmsnorm(kv[:, :I], H, d, t["gamma_k"], cfg.eps), pos, H, d,
                   cfg.rope_split, cfg.rope_base)
    v_all = kv[:, I:]
    a = a_all[r]
    q = linear(a, w_qkv[:I])
    q_r = rope3d(qk_rmsnorm(q, H, d, t["gamma_q"], cfg.eps), pos[r], H, d,
                 cfg.rope_split, cfg.rope_base)
    o = attention(q_r, k_all, v_all, H, d, cfg.scale, rows=r)
    y = linear(o, t["w_o"])
    x1 = gate_residual(x[r], y, t["mod"], BRANCH_ATTN, segs, rows=r)
    a2 = adaln_modulate(x1, t["mod"], BRANCH_FFN, segs, cfg.eps, rows=r)
    gu = linear(a2, t["w_gu"])
    h = swiglu(gu, F)
    f = linear(h, t["w_d"])
    out = gate_residual(x1, f, t["mod"], BRANCH_FFN, segs, rows=r)
    return {"a": a, "q": q, "kv": kv[r], "q_rope": q_r, "k_rope": k_all[r], "v": v_all[r],
            "o": o, "y": y, "x1": x1, "a2": a2, "gu": gu, "h": h, "f": f, "out": out,
            "k_all": k_all, "v_all": v_all}
