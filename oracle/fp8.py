"""Oracle of the FP8 (OCP e4m3) projections.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages only say that the community runs the model with FP8 quantisation
(H3 omni-modal commentary); they fix no format, scaling or error bound.
Readings, stated as such:
* format: OCP e4m3 -- sign bit, 4 exponent bits with bias 7, 3 mantissa
  bits, subnormals m/8 * 2^-6 below 2^-6, largest finite value 448, no
  infinities, NaN codes 0x7F / 0xFF (the format the gfx950 FP8 MFMA reads);
* rounding: to the nearest e4m3 value, ties to the even code, saturating at
  +-448; NaN stays NaN;
* scales: one per row, max|x| / 448 computed in fp32 (1 for an all-zero
  row); activations are quantised per token, weights [out][in] per output
  channel, so C = diag(sa) (Qa . Qw^T) diag(sw);
* the quantised operands' products are exact and summed in fp64 here.
"""
import numpy as np

from .block import linear

E4M3_MAX = 448.0


def e4m3_decode(codes):
    """Code(s) 0..255 -> fp64 value (NaN for 0x7F and 0xFF)."""
    c = np.asarray(codes, dtype=np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e.astype(np.float64) - 7))
    mag = np.where((e == 15) & ((c & 7) == 7), np.nan, mag)
    return s * mag


_POS_CODES = np.arange(0x7F)                 # 0 .. 0x7E: the non-negative finite values, increasing
_POS_VALUES = e4m3_decode(_POS_CODES)


def e4m3_encode(x):
    """Values -> e4m3 codes: the nearest representable value, ties to the
    even code, magnitudes at or above 448 saturate to +-448, NaN -> 0x7F."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    hi = np.clip(np.searchsorted(_POS_VALUES, a, side="left"), 0, len(_POS_VALUES) - 1)
    lo = np.clip(hi - 1, 0, len(_POS_VALUES) - 1)
    d_lo = np.abs(a - _POS_VALUES[lo])
    d_hi = np.abs(_POS_VALUES[hi] - a)
    pick = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where(_POS_CODES[lo] % 2 == 0, lo, hi)))
    code = _POS_CODES[pick]
    code = np.where(a >= E4M3_MAX, 0x7E, code)
    code = code | np.where(np.signbit(x), 0x80, 0)
    code = np.where(np.isnan(x), 0x7F, code)
    return code.astype(np.uint8)


def quantize_rows(x):
    """x [n, K] (fp32-representable values) -> (codes uint8 [n, K], scales
    fp32 [n]): scale = max|x| / 448 and x / scale, both in fp32."""
    x32 = np.asarray(x, dtype=np.float32)
    mx = np.max(np.abs(x32), axis=1)
    scales = np.where(mx > 0, mx / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    return e4m3_encode(x32 / scales[:, None]), scales


def gemm_fp8(qa, sa, qw, sw):
    """C = diag(sa) (decode(qa) . decode(qw)^T) diag(sw) in fp64."""
    return linear(e4m3_decode(qa), e4m3_decode(qw)) * np.asarray(sa, np.float64)[:, None] \
        * np.asarray(sw, np.float64)[None, :]


# ------------------------------------------------------------------ attention
# Readings for the fp8 attention (the pages give none): q is quantised per
# (token, head), k and v per head (their scales are constants of the head);
# the reference is the exact softmax attention of the dequantised operands.
# Rounding the softmax weights to e4m3 inside the kernel is an approximation
# the tolerance covers, not part of this definition.

def quantize_qkv(q, k, v, heads, head_dim):
    """q, k, v [n, heads*head_dim] (fp32-representable) -> codes of the same
    shape, sq [heads, n], sk [heads], sv [heads] (fp32 scales max/448)."""
    n = np.asarray(q).shape[0]
    q32 = np.asarray(q, np.float32).reshape(n, heads, head_dim)
    mx = np.max(np.abs(q32), axis=2)                                     # [n, heads]
    sq = np.where(mx > 0, mx / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    q8 = e4m3_encode(q32 / sq[:, :, None]).reshape(n, heads * head_dim)
    out = [q8, sq.T.copy()]
    for x in (k, v):
        x32 = np.asarray(x, np.float32).reshape(n, heads, head_dim)
        m = np.max(np.abs(x32), axis=(0, 2))
        s = np.where(m > 0, m / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
        out += [e4m3_encode(x32 / s[None, :, None]).reshape(n, heads * head_dim), s]
    q8, sq, k8, sk, v8, sv = out
    return q8, sq, k8, sk, v8, sv


def dequantize_qkv(q8, sq, k8, sk, v8, sv, heads, head_dim):
    n = q8.shape[0]
    q = e4m3_decode(q8).reshape(n, heads, head_dim) * np.asarray(sq, np.float64).T[:, :, None]
    k = e4m3_decode(k8).reshape(n, heads, head_dim) * np.asarray(sk, np.float64)[None, :, None]
    v = e4m3_decode(v8).reshape(n, heads, head_dim) * np.asarray(sv, np.float64)[None, :, None]
    return tuple(a.reshape(n, heads * head_dim) for a in (q, k, v))
