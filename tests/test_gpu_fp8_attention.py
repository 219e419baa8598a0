"""GPU parity of the FP8 attention (h3_quantize_qkv_fp8, h3_attention_fp8)
against the oracle.

* Quantiser: codes and fp32 scales bit for bit against the oracle's (both
  divide in fp32 and round by the format's definition), the transposed and
  permuted V layout included, zeros past n_tok; ragged n, strided views, a
  zero query row and an all-zero head (scale 1).
* Attention: against the oracle's fp64 attention of the dequantised
  operands (the GPU's own codes and scales).  The kernel also rounds each
  softmax weight to e4m3 (relative error at most 2^-4, RMS at most
  2^-4 / sqrt(3) = 3.6 %) and normalises by the sum of the rounded weights,
  which moves o by sum_j p_j e_j (v_j - o) / sum_j p_j: held to 2^-4 in the
  Frobenius norm relative to |o|, and to 2^-4 of max |v| per element.
* A key that dominates every query, placed at the last key and at tile
  edges: the running reference is overtaken (the exponential overflows and
  the tile is redone) and a lost or misplaced key shows at once.  Peaked
  logits (std 16), an LDS poisoned beforehand, ragged tiles.
* End to end (quantise, then attend) against the unquantised attention:
  three roundings of RMS at most 2^-4 / sqrt(3) plus the logit term
  sqrt(2) of one at logits of RMS 1, 2 * 2^-4 / sqrt(3) = 7.2 % -> 7.5e-2.
* The 15 s 768p shape (92840 tokens, 56 heads of 128): quantiser on sampled
  rows and groups, attention on sampled rows.
"""
import numpy as np
import pytest

import oracle
from fp8_layout import vt_key, vt_layout
from video_audio_diffusion_amd import blk, inputs
from video_audio_diffusion_amd.block import device_inputs, host_array

from gpu_util import widen

pytestmark = pytest.mark.gpu
HD = 128
TOL_P = 2.0 ** -4           # softmax weights rounded to e4m3
TOL_E2E = 7.5e-2            # quantised operands and weights against unquantised attention


def _dev(a):
    return device_inputs(None, {"a": a})["a"]


def _n_pad(n):
    return -(-n // 64) * 64


def _quantize(qkv, n, H, n_pad=None):
    """qkv: device bf16 [n][3 H 128] (q | k | v) -> dict of device outputs."""
    import torch
    I = H * HD
    n_pad = n_pad or _n_pad(n)
    r = {"q8": torch.full((n, I), 0x55, dtype=torch.uint8, device="cuda"),
         "k8": torch.full((n, I), 0x55, dtype=torch.uint8, device="cuda"),
         "vt": torch.full((H * HD, n_pad), 0x55, dtype=torch.uint8, device="cuda"),
         "sq": torch.full((H, n), -1.0, dtype=torch.float32, device="cuda"),
         "sk": torch.full((H,), -1.0, dtype=torch.float32, device="cuda"),
         "sv": torch.full((H,), -1.0, dtype=torch.float32, device="cuda"), "n_pad": n_pad}
    ld = qkv.stride(0)
    blk.h3_quantize_qkv_fp8(qkv[:, :I], qkv[:, I:2 * I], qkv[:, 2 * I:], ld, n, H, HD, r["q8"], r["k8"], r["vt"],
                            n_pad, r["sq"], r["sk"], r["sv"], blk.H3_BF16)
    return r


def _attend(r, n, H, scale=HD ** -0.5):
    import torch
    o = torch.full((n, H * HD), float("nan"), dtype=torch.bfloat16, device="cuda")
    blk.h3_attention_fp8(r["q8"], r["k8"], r["vt"], r["n_pad"], r["sq"], r["sk"], r["sv"], o, H * HD, n, H, HD,
                         scale)
    return o


def _host(r):
    return {k: (v.cpu().numpy() if hasattr(v, "cpu") else v) for k, v in r.items()}


def _check_quantiser(h, f, n, H, name):
    I = H * HD
    q8, sq, k8, sk, v8, sv = oracle.quantize_qkv(f[:, :I], f[:, I:2 * I], f[:, 2 * I:], H, HD)
    for key, want in (("sq", sq), ("sk", sk), ("sv", sv)):
        assert np.array_equal(h[key], want), f"{name}: {key} differs"
    for key, want in (("q8", q8), ("k8", k8)):
        bad = np.argwhere(h[key] != want)
        assert bad.size == 0, f"{name}: {key} differs at {bad[:5]}"
    want_vt = vt_layout(v8, H, HD, h["n_pad"]).reshape(H * HD, h["n_pad"])
    bad = np.argwhere(h["vt"] != want_vt)
    assert bad.size == 0, f"{name}: vt differs at {bad[:5]}"
    return q8, sq, k8, sk, v8, sv


def _assert_fp8_attn(name, got, ref, vmax, tol=TOL_P):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    assert np.isfinite(got).all(), f"{name}: non-finite output"
    e_f = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    e_v = np.abs(got - ref).max() / vmax
    print(f"  {name}: e_F={e_f:.3e} e_max/max|v|={e_v:.3e} (tol {tol:g})", flush=True)
    assert e_f <= tol and e_v <= tol, f"{name}: e_F={e_f:.3e} e_v={e_v:.3e} > {tol}"


def _reference(h, n, H, scale=HD ** -0.5, rows=None):
    """fp64 attention of the dequantised operands (q8/k8 as codes, v from
    the oracle's quantisation of the same v, which the quantiser test ties
    to the GPU's V^T)."""
    q, k, v = oracle.dequantize_qkv(h["q8"], h["sq"], h["k8"], h["sk"], h["v8"], h["sv"], H, HD)
    qr = q if rows is None else q[rows]
    return oracle.attention(qr, k, v, H, HD, scale, rows=rows), np.abs(v).max(), v


def _run(qkv_h, n, H, name, n_pad=None):
    import torch
    qkv = _dev(qkv_h)
    r = _quantize(qkv, n, H, n_pad)
    o = _attend(r, n, H)
    torch.cuda.synchronize()
    h = _host(r)
    f = inputs.widen(qkv_h, "bf16")
    h["v8"] = _check_quantiser(h, f, n, H, name)[4]
    return h, f, widen(o, "bf16")


@pytest.mark.parametrize("n", [1, 2, 63, 64, 65, 117, 255, 257, 1000, 4097])
def test_quantise_and_attend_ragged(n):
    H = 3
    qkv_h = inputs.draw_rows(None, (n, 3 * H * HD), 1200 + n, dtype="bf16")
    h, f, got = _run(qkv_h, n, H, f"n={n}")
    ref, vmax, _ = _reference(h, n, H)
    _assert_fp8_attn(f"fp8 attn n={n}", got, ref, vmax)
    I = H * HD
    exact = oracle.attention(f[:, :I], f[:, I:2 * I], f[:, 2 * I:], H, HD, HD ** -0.5)
    _assert_fp8_attn(f"fp8 attn n={n} vs unquantised", got, exact, np.abs(f[:, 2 * I:]).max(), TOL_E2E)


def test_zero_row_zero_head_and_wide_padding():
    """A zero query row and an all-zero head of k and of v (scales 1, codes
    0: uniform weights, zero output there); n_pad two groups past the last
    token (its V^T columns zero; inside the last group, the positions of
    keys past the end)."""
    n, H = 150, 3
    I = H * HD
    qkv_h = inputs.draw_rows(None, (n, 3 * I), 1300, dtype="bf16")
    qkv_h[7, :I] = 0
    qkv_h[:, I + HD:I + 2 * HD] = 0                       # head 1 of k
    qkv_h[:, 2 * I + 2 * HD:2 * I + 3 * HD] = 0           # head 2 of v
    h, f, got = _run(qkv_h, n, H, "zeros", n_pad=_n_pad(n) + 128)
    assert h["sq"][0, 7] == 1.0 and h["sk"][1] == 1.0 and h["sv"][2] == 1.0
    assert np.all(h["vt"][:, _n_pad(n):] == 0)            # whole groups past the last token
    ref, vmax, _ = _reference(h, n, H)
    _assert_fp8_attn("fp8 attn zeros", got, ref, vmax)
    assert np.all(got[:, 2 * HD:] == 0)                   # head 2: v = 0
    v1 = f[:, 2 * I + HD:2 * I + 2 * HD]                  # head 1: all logits 0 -> the mean of v
    np.testing.assert_allclose(got[:, HD:2 * HD], np.broadcast_to(v1.mean(0), (n, HD)), atol=0.05 * np.abs(v1).max())


@pytest.mark.parametrize("n,key", [(65, 64), (4097, 4096), (4100, 63), (4100, 2048), (300, 255)])
def test_dominant_key(n, key):
    """Every query's q lies near one direction u and key `key` is 12 u, so
    its logit exceeds the rest by about 136 (2^-196 of its weight for the
    others): every output row is that key's dequantised v, to the bf16
    rounding of the output.  Keys before it set a reference that its tile
    overtakes by so much that the exponentials overflow and the tile is
    redone; at key 63 the first tile already holds it."""
    H = 2
    I = H * HD
    g = np.random.Generator(np.random.PCG64(1400 + n + key))
    qkv = g.standard_normal((n, 3 * I), dtype=np.float32)
    u = g.standard_normal(I, dtype=np.float32)
    qkv[:, :I] = 0.3 * qkv[:, :I] + u
    qkv[key, I:2 * I] = 12.0 * u
    qkv_h = inputs.f32_to_bf16_bits(qkv)
    h, f, got = _run(qkv_h, n, H, f"dominant n={n} key={key}")
    ref, vmax, vd = _reference(h, n, H)
    _assert_fp8_attn(f"fp8 attn dominant n={n} key={key}", got, ref, vmax)
    vk = vd[key]
    err = np.abs(got - vk[None, :]).max()
    assert err <= 2.0 ** -8 * np.abs(vk).max(), f"dominant key: {err:.3e}"


def test_peaked_logits():
    """Q/K values of std 4: logits of std 16, so nearly every 64-key tile
    raises some query's running reference."""
    n, H = 1500, 3
    I = H * HD
    g = np.random.Generator(np.random.PCG64(1500))
    qkv = g.standard_normal((n, 3 * I), dtype=np.float32)
    qkv[:, :2 * I] *= 4.0
    qkv_h = inputs.f32_to_bf16_bits(qkv)
    h, f, got = _run(qkv_h, n, H, "peaked")
    ref, vmax, _ = _reference(h, n, H)
    _assert_fp8_attn("fp8 attn peaked", got, ref, vmax)


@pytest.mark.parametrize("n", [1, 117, 200])
def test_after_lds_poison(n):
    """A GEMM over all-NaN operands leaves NaN bit patterns in every CU's
    LDS; short sequences then read ring buffers that none of their tiles
    fill."""
    import torch
    H = 3
    poison = torch.full((4096, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    junk = torch.empty(4096, 4096, dtype=torch.bfloat16, device="cuda")
    qkv_h = inputs.draw_rows(None, (n, 3 * H * HD), 1600 + n, dtype="bf16")
    qkv = _dev(qkv_h)
    r = _quantize(qkv, n, H)
    blk.h3_gemm_bf16(poison, 128, poison, 128, junk, 4096, 4096, 4096, 128, blk.H3_BF16)
    o = _attend(r, n, H)
    torch.cuda.synchronize()
    assert bool(torch.isnan(junk[:8, :8]).all())
    h = _host(r)
    h["v8"] = _check_quantiser(h, inputs.widen(qkv_h, "bf16"), n, H, f"poison n={n}")[4]
    ref, vmax, _ = _reference(h, n, H)
    _assert_fp8_attn(f"fp8 attn after poison n={n}", widen(o, "bf16"), ref, vmax)


def test_deterministic():
    import torch
    n, H = 3000, 2
    qkv = _dev(inputs.draw_rows(None, (n, 3 * H * HD), 1700, dtype="bf16"))
    r1 = _quantize(qkv, n, H)
    o1 = _attend(r1, n, H)
    r2 = _quantize(qkv, n, H)
    o2 = _attend(r2, n, H)
    torch.cuda.synchronize()
    for k in ("q8", "k8", "vt", "sq", "sk", "sv"):
        assert torch.equal(r1[k], r2[k]), k
    assert torch.equal(o1, o2)


def test_768p15s_shape_sampled():
    """92840 tokens x 56 heads (the benchmark's attention), bf16 q | k | v
    of N(0, 1) values (the scale after the per-head RMS norm)."""
    import torch
    c3 = inputs.CONFIGS[3]
    n, H = c3.n_tok, c3.heads
    I = H * HD
    print(f"[768p15s] drawing {n} x {3 * I}", flush=True)
    qkv_h = inputs.draw_rows(None, (n, 3 * I), 1800, dtype="bf16")
    qkv = _dev(qkv_h)
    r = _quantize(qkv, n, H)
    o = _attend(r, n, H)
    torch.cuda.synchronize()
    print("[768p15s] checking", flush=True)
    rows = inputs.sample_rows(c3, n_random=24)
    idx = torch.from_numpy(rows).cuda()
    # scales: per-head maxima straight from the bf16 bits (finite values
    # order like their magnitude bits)
    mag = (qkv_h.reshape(n, 3, H, HD) & 0x7FFF).max(axis=(0, 3))           # [3, H] bits
    amax = inputs.widen(mag.astype(np.uint16), "bf16").astype(np.float32)
    want_sk = np.where(amax[1] > 0, amax[1] / np.float32(448), np.float32(1)).astype(np.float32)
    want_sv = np.where(amax[2] > 0, amax[2] / np.float32(448), np.float32(1)).astype(np.float32)
    assert np.array_equal(r["sk"].cpu().numpy(), want_sk) and np.array_equal(r["sv"].cpu().numpy(), want_sv)
    f_rows = inputs.widen(qkv_h[rows], "bf16")
    q8, sq, k8, _, v8, _ = oracle.quantize_qkv(f_rows[:, :I], f_rows[:, I:2 * I], f_rows[:, 2 * I:], H, HD)
    # k and v of the sampled rows quantised with the whole sequence's scales
    k8 = oracle.e4m3_encode((f_rows[:, I:2 * I].reshape(-1, H, HD).astype(np.float32)
                             / want_sk[None, :, None]).reshape(len(rows), I))
    v8 = oracle.e4m3_encode((f_rows[:, 2 * I:].reshape(-1, H, HD).astype(np.float32)
                             / want_sv[None, :, None]).reshape(len(rows), I))
    assert np.array_equal(r["q8"].index_select(0, idx).cpu().numpy(), q8)
    assert np.array_equal(r["sq"][:, idx].cpu().numpy(), sq)
    assert np.array_equal(r["k8"].index_select(0, idx).cpu().numpy(), k8)
    # V^T: each sampled key sits at its permuted position in its group
    pos = (rows // 64) * 64 + np.argsort(vt_key(np.arange(64)))[rows % 64]
    vt_cols = r["vt"][:, torch.from_numpy(pos).cuda()].cpu().numpy()        # [H*128, len(rows)]
    assert np.array_equal(vt_cols.T, v8)
    n_pad = r["n_pad"]
    key_at = (np.arange(n_pad) // 64) * 64 + vt_key(np.arange(n_pad) % 64)
    past = torch.from_numpy(np.nonzero(key_at >= n)[0]).cuda()
    assert bool((r["vt"][:, past] == 0).all())                 # positions of keys past the end
    # attention on sampled rows, head by head, from the GPU's own codes
    arows = rows[:: max(1, len(rows) // 24)]
    got = widen(o.index_select(0, torch.from_numpy(arows).cuda()), "bf16")
    sq_h = r["sq"].cpu().numpy()
    sk_h, sv_h = r["sk"].cpu().numpy(), r["sv"].cpu().numpy()
    ref = np.empty((len(arows), I))
    exact = np.empty((len(arows), I))
    vmax = 0.0
    for hh in range(H):
        sl = slice(hh * HD, (hh + 1) * HD)
        kd = oracle.e4m3_decode(r["k8"][:, sl].cpu().numpy()) * float(sk_h[hh])
        vt_h = r["vt"][hh * HD:(hh + 1) * HD].cpu().numpy()            # [128, n_pad] permuted keys
        src = (np.arange(n_pad) // 64) * 64 + vt_key(np.arange(n_pad) % 64)
        vd = np.empty((n, HD))
        ok = src < n
        vd[src[ok]] = oracle.e4m3_decode(vt_h[:, ok].T) * float(sv_h[hh])
        qd = oracle.e4m3_decode(r["q8"][torch.from_numpy(arows).cuda(), sl].cpu().numpy()) \
            * sq_h[hh, arows][:, None].astype(np.float64)
        ref[:, sl] = oracle.attention(qd, kd, vd, 1, HD, c3.scale)
        vmax = max(vmax, np.abs(vd).max())
        fk = inputs.widen(qkv_h[:, I + hh * HD:I + (hh + 1) * HD], "bf16")
        fv = inputs.widen(qkv_h[:, 2 * I + hh * HD:2 * I + (hh + 1) * HD], "bf16")
        exact[:, sl] = oracle.attention(inputs.widen(qkv_h[arows, hh * HD:(hh + 1) * HD], "bf16"), fk, fv, 1, HD,
                                        c3.scale)
    _assert_fp8_attn("fp8 attn 768p15s sampled", got, ref, vmax)
    _assert_fp8_attn("fp8 attn 768p15s vs unquantised", got, exact, vmax, TOL_E2E)
