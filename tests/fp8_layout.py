"""Layout helper of the FP8 attention's transposed v operand (a property
of the GPU kernel's buffer layout, not of the method): h3_quantize_qkv_fp8
stores v transposed to [heads][head_dim][n_pad] with each 64-key group
permuted so that a lane's packed softmax weights line up with the v^T bytes
it reads.  The tests use it to compare that buffer with the oracle's
quantised v in plain [n][heads*head_dim] form."""
import numpy as np


def vt_key(p):
    """Key (within its group of 64) stored at position p of the transposed
    fp8 v: p = 32 g + b holds key 32 (b // 16) + 8 ((b % 16) // 4) + 4 g + b % 4."""
    p = np.asarray(p)
    g, b = p // 32, p % 32
    return 32 * (b // 16) + 8 * ((b % 16) // 4) + 4 * g + b % 4


def vt_layout(v8, heads, head_dim, n_pad):
    """Codes v8 [n, heads*head_dim] -> [heads, head_dim, n_pad]: transposed,
    each 64-key group in vt_key order, zero past n."""
    n = v8.shape[0]
    full = np.zeros((n_pad, heads, head_dim), np.uint8)
    full[:n] = v8.reshape(n, heads, head_dim)
    pos = np.arange(n_pad)
    src = (pos // 64) * 64 + vt_key(pos % 64)
    return full[src].transpose(1, 2, 0).copy()
