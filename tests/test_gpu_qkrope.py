"""GPU parity of h3_gemm_qknorm_rope: the QKV projection with the per-head
RMSNorm and 3-D RoPE of q and k applied in its epilogue.

* q and k against the fp64 oracle (norm and rotation of the exact product,
  positions from the interval table), v bit-equal to h3_gemm_bf16's output
  (v tiles take the plain store);
* q and k against the two-call path (h3_gemm_bf16, then h3_qknorm_rope3d):
  both norm the same product rounded to the storage type and differ only in
  the order of the sum of squares and in how the angle is evaluated, so they
  agree to about a unit in the last place;
* bf16 and fp32 (whose tile takes the epilogue in two passes), head_dim 128
  and 64, ragged M, a padded row stride, 8 v columns (N not a multiple of
  the tile), one interval or text + audio + video grids with position
  offsets up to 5000, with and without gains;
* h3_gemm_fp8_qknorm_rope (the same epilogue after the e4m3 product) against
  h3_gemm_fp8 followed by h3_qknorm_rope3d, and q and k against the oracle's
  norm and rotation of the oracle's product of the same codes.
"""
import numpy as np
import pytest

import oracle
from video_audio_diffusion_amd import blk, inputs
from video_audio_diffusion_amd.block import device_inputs, host_array

from gpu_util import TOL, assert_close, widen

pytestmark = pytest.mark.gpu


def _segments(M, kind):
    """One text interval, or text, audio (t offset 5000), a 3x5 video grid
    (offsets h 2, w 1) and a trailing text interval for the remainder."""
    if kind == "one" or M < 40:
        return [inputs.Segment(start=0, length=M, mod_set=0, T=M, kind="text")]
    n_text, n_audio = M // 8, M // 6
    rest = M - n_text - n_audio
    frames = rest // 15
    segs = [inputs.Segment(start=0, length=n_text, mod_set=0, T=n_text, kind="text"),
            inputs.Segment(start=n_text, length=n_audio, mod_set=2, T=n_audio, t0=5000, kind="audio"),
            inputs.Segment(start=n_text + n_audio, length=frames * 15, mod_set=1, T=frames, H=3, W=5, h0=2, w0=1,
                           kind="video")]
    tail = rest - frames * 15
    if tail:
        segs.append(inputs.Segment(start=M - tail, length=tail, mod_set=0, T=tail, t0=3, kind="text"))
    return segs


def _dev(a):
    return device_inputs(None, {"a": a})["a"]


SPLIT = {128: (64, 32, 32), 64: (16, 24, 24)}


@pytest.mark.parametrize("dtype,M,heads,hd,K,kind,pad,gains,nv", [
    ("bf16", 1, 2, 128, 64, "one", 0, True, None),
    ("bf16", 300, 2, 128, 128, "mixed", 8, True, None),
    ("bf16", 513, 4, 64, 192, "mixed", 0, False, None),
    ("bf16", 1100, 6, 128, 64, "mixed", 0, True, None),
    ("bf16", 300, 2, 128, 64, "mixed", 0, True, 8),
    ("bf16", 257, 2, 128, 8256, "mixed", 8, True, None),     # K past the LDS-DMA loop's limit
    ("f32", 72, 4, 64, 192, "mixed", 0, True, None),
    ("f32", 257, 2, 128, 64, "mixed", 8, False, None),
])
def test_gemm_qknorm_rope(dtype, M, heads, hd, K, kind, pad, gains, nv):
    import torch
    qc = heads * hd
    N = 2 * qc + (qc if nv is None else nv)
    ldc = N + pad
    split, base, eps = SPLIT[hd], 1e4, 1e-6
    a_h = inputs.draw_rows(None, (M, K), 61 + M, dtype=dtype)
    w_h = inputs.draw_rows(None, (N, K), 62 + N, dtype=dtype)
    rng = np.random.Generator(np.random.PCG64(63))
    gq = (1 + 0.1 * rng.standard_normal(hd)).astype(np.float32) if gains else None
    gk = (1 + 0.1 * rng.standard_normal(hd)).astype(np.float32) if gains else None
    segs = _segments(M, kind)
    A, W = _dev(a_h), _dev(w_h)
    gqd = _dev(gq) if gains else None
    gkd = _dev(gk) if gains else None
    dt = blk.H3_BF16 if dtype == "bf16" else blk.H3_F32
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    C = torch.full((M, ldc), float("nan"), dtype=tdt, device="cuda")
    C2 = torch.full((M, ldc), float("nan"), dtype=tdt, device="cuda")
    hs = blk.segments(segs)
    print(f"[qkrope] {dtype} M={M} heads={heads} hd={hd} K={K} N={N} ldc={ldc} segs={len(segs)}", flush=True)
    blk.h3_gemm_qknorm_rope(A, K, W, K, C, ldc, M, N, K, heads, hd, gqd, gkd, eps, *split, base, hs, len(segs), dt)
    blk.h3_gemm_bf16(A, K, W, K, C2, ldc, M, N, K, dt)
    torch.cuda.synchronize()
    plain = host_array(C2, dtype)
    blk.h3_qknorm_rope3d(C2[:, :qc], C2[:, qc:2 * qc], ldc, M, heads, hd, gqd, gkd, eps, *split, base, hs,
                         len(segs), dt)
    torch.cuda.synchronize()
    got_h, two_h = host_array(C, dtype), host_array(C2, dtype)
    got, two = inputs.widen(got_h, dtype), inputs.widen(two_h, dtype)

    # v: the plain store, bit for bit; padding columns untouched
    assert np.array_equal(got_h[:, 2 * qc:N], plain[:, 2 * qc:N]), "v columns differ from h3_gemm_bf16"
    assert np.all(np.isnan(got[:, N:])), "columns beyond N were written"

    # q and k against the oracle
    raw = oracle.linear(inputs.widen(a_h, dtype), inputs.widen(w_h, dtype))
    _, pos = oracle.token_table(segs, M)
    ones = np.ones(hd)
    for name, sl, gam in (("q", slice(0, qc), gq), ("k", slice(qc, 2 * qc), gk)):
        g64 = ones if gam is None else gam.astype(np.float64)
        ref = oracle.rope3d(oracle.qk_rmsnorm(raw[:, sl], heads, hd, g64, eps), pos, heads, hd, split, base)
        assert_close(f"gemm_qknorm_rope {name} {dtype} {M}x{N}x{K}", got[:, sl], ref, TOL[dtype])
        # against the two-call path: one unit in the last place of the larger
        # magnitude (bf16: 8 significant bits), or a few fp32 ulps
        diff = np.abs(got[:, sl] - two[:, sl])
        big = np.maximum(np.abs(got[:, sl]), np.abs(two[:, sl]))
        if dtype == "bf16":
            bound = np.ldexp(1.0, np.frexp(big)[1] - 8) + 1e-5 * np.max(big)
        else:
            bound = 4e-7 * big + 2e-6 * np.max(big)
        excess = diff - bound
        worst = float(np.max(excess))
        r, c = np.unravel_index(int(np.argmax(excess)), excess.shape)
        print(f"  {name} vs two calls: max |diff| {diff.max():.3e}, identical {np.mean(diff == 0):.4f}; "
              f"worst at row {r} col {c}: fused {got[r, sl][c]:.8g} two-call {two[r, sl][c]:.8g} "
              f"oracle {ref[r, c]:.8g} (position {pos[r]})", flush=True)
        assert worst <= 0, f"{name}: fused and two-call results differ by more than an ulp ({worst:.3e})"


def test_gemm_qknorm_rope_no_tokens():
    """M = 0 launches nothing and succeeds."""
    import torch
    A = torch.zeros(1, 64, dtype=torch.bfloat16, device="cuda")
    W = torch.zeros(768, 64, dtype=torch.bfloat16, device="cuda")
    C = torch.zeros(1, 768, dtype=torch.bfloat16, device="cuda")
    blk.h3_gemm_qknorm_rope(A, 64, W, 64, C, 768, 0, 768, 64, 2, 128, None, None, 1e-6, 64, 32, 32, 1e4, None, 0,
                            blk.H3_BF16)
    torch.cuda.synchronize()
    assert torch.count_nonzero(C) == 0


def _ulp_check(name, got, two):
    """Within one bf16 unit in the last place of the larger magnitude."""
    diff = np.abs(got - two)
    big = np.maximum(np.abs(got), np.abs(two))
    bound = np.ldexp(1.0, np.frexp(big)[1] - 8) + 1e-5 * np.max(big)
    print(f"  {name} vs two calls: max |diff| {diff.max():.3e}, identical {np.mean(diff == 0):.4f}", flush=True)
    assert float(np.max(diff - bound)) <= 0, f"{name}: fused and two-call results differ by more than an ulp"


@pytest.mark.parametrize("M,heads,hd,K,gains", [(300, 2, 128, 256, True), (513, 4, 64, 128, False),
                                                 (1100, 6, 128, 384, True)])
def test_gemm_fp8_qknorm_rope(M, heads, hd, K, gains):
    import torch
    qc = heads * hd
    N = 3 * qc
    split, base, eps = SPLIT[hd], 1e4, 1e-6
    a = _dev(inputs.draw_rows(None, (M, K), 71 + M, dtype="bf16"))
    w = _dev(inputs.draw_rows(None, (N, K), 72 + N, dtype="bf16"))
    rng = np.random.Generator(np.random.PCG64(73))
    gq = (1 + 0.1 * rng.standard_normal(hd)).astype(np.float32) if gains else None
    gk = (1 + 0.1 * rng.standard_normal(hd)).astype(np.float32) if gains else None
    gqd = _dev(gq) if gains else None
    gkd = _dev(gk) if gains else None
    qa = torch.empty(M, K, dtype=torch.uint8, device="cuda")
    sa = torch.empty(M, dtype=torch.float32, device="cuda")
    qw = torch.empty(N, K, dtype=torch.uint8, device="cuda")
    sw = torch.empty(N, dtype=torch.float32, device="cuda")
    blk.h3_quantize_fp8(a, K, M, K, qa, K, sa, blk.H3_BF16)
    blk.h3_quantize_fp8(w, K, N, K, qw, K, sw, blk.H3_BF16)
    segs = _segments(M, "mixed")
    hs = blk.segments(segs)
    C = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    C2 = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    print(f"[qkrope fp8] M={M} heads={heads} hd={hd} K={K}", flush=True)
    blk.h3_gemm_fp8_qknorm_rope(qa, K, sa, qw, K, sw, C, N, M, N, K, heads, hd, gqd, gkd, eps, *split, base, hs,
                                len(segs))
    blk.h3_gemm_fp8(qa, K, sa, qw, K, sw, C2, N, M, N, K, blk.H3_BF16)
    torch.cuda.synchronize()
    plain = host_array(C2, "bf16")
    blk.h3_qknorm_rope3d(C2[:, :qc], C2[:, qc:2 * qc], N, M, heads, hd, gqd, gkd, eps, *split, base, hs, len(segs),
                         blk.H3_BF16)
    torch.cuda.synchronize()
    got_h = host_array(C, "bf16")
    got, two = inputs.widen(got_h, "bf16"), inputs.widen(host_array(C2, "bf16"), "bf16")
    assert np.array_equal(got_h[:, 2 * qc:], plain[:, 2 * qc:]), "v columns differ from h3_gemm_fp8"
    raw = oracle.gemm_fp8(qa.cpu().numpy(), sa.cpu().numpy(), qw.cpu().numpy(), sw.cpu().numpy())
    _, pos = oracle.token_table(segs, M)
    for name, sl, gam in (("q", slice(0, qc), gq), ("k", slice(qc, 2 * qc), gk)):
        g64 = np.ones(hd) if gam is None else gam.astype(np.float64)
        ref = oracle.rope3d(oracle.qk_rmsnorm(raw[:, sl], heads, hd, g64, eps), pos, heads, hd, split, base)
        assert_close(f"gemm_fp8_qknorm_rope {name} {M}x{N}x{K}", got[:, sl], ref, TOL["bf16"])
        _ulp_check(name, got[:, sl], two[:, sl])
