"""The H3 block assembled from torch fp64 library routines (rms_norm,
scaled_dot_product_attention, silu, complex-number RoPE): an assembly
independent of the oracle's own step functions, used to pin the oracle's
block and its 50-block composition."""
import numpy as np
import torch
import torch.nn.functional as F


def torch_block(t, cfg):
    """The block assembled from torch fp64 library routines."""
    D, H, d, Fw = cfg.dim, cfg.heads, cfg.head_dim, cfg.ffn
    I = H * d
    T = {k: torch.from_numpy(np.ascontiguousarray(v)) for k, v in t.items()}
    n = cfg.n_tok
    sets = torch.zeros(n, dtype=torch.long)
    pos = torch.zeros(n, 3, dtype=torch.float64)
    for s in cfg.segments:
        sets[s.start:s.start + s.length] = s.mod_set
        g = torch.stack(torch.meshgrid(torch.arange(s.T), torch.arange(s.H), torch.arange(s.W),
                                       indexing="ij"), -1).reshape(-1, 3)
        pos[s.start:s.start + s.length] = g.double()
    m = T["mod"][sets]                                   # [n, 6, D]
    x = T["x"]
    a = F.rms_norm(x, (D,), eps=cfg.eps) * (1 + m[:, 1]) + m[:, 0]
    qkv = a @ T["w_qkv"].T
    q, k, v = (qkv[:, i * I:(i + 1) * I].reshape(n, H, d) for i in range(3))
    q = F.rms_norm(q, (d,), weight=T["gamma_q"], eps=cfg.eps)
    k = F.rms_norm(k, (d,), weight=T["gamma_k"], eps=cfg.eps)

    def rope(z):
        parts, off = [], 0
        for ax, da in enumerate(cfg.rope_split):
            zc = torch.view_as_complex(z[..., off:off + da].reshape(n, H, da // 2, 2).contiguous())
            freq = cfg.rope_base ** (-torch.arange(0, da, 2, dtype=torch.float64) / da)
            rot = torch.polar(torch.ones(n, da // 2, dtype=torch.float64), pos[:, ax:ax + 1] * freq)
            parts.append(torch.view_as_real(zc * rot[:, None, :]).reshape(n, H, da))
            off += da
        return torch.cat(parts, -1)

    q, k = rope(q), rope(k)
    o = F.scaled_dot_product_attention(q.transpose(0, 1), k.transpose(0, 1), v.transpose(0, 1))
    o = o.transpose(0, 1).reshape(n, I)
    x1 = x + m[:, 2] * (o @ T["w_o"].T)
    a2 = F.rms_norm(x1, (D,), eps=cfg.eps) * (1 + m[:, 4]) + m[:, 3]
    gu = a2 @ T["w_gu"].T
    hdn = F.silu(gu[:, :Fw]) * gu[:, Fw:]
    return (x1 + m[:, 5] * (hdn @ T["w_d"].T)).numpy()
