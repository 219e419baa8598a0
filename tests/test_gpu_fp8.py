"""GPU parity of the FP8 (OCP e4m3) projections against the oracle.

* h3_quantize_fp8: codes and fp32 scales bit for bit against the oracle's
  quantiser (both divide in fp32 and round by the format's definition),
  with a zero row, a large outlier, values in the subnormal range and
  negative zeros; bf16 and fp32 inputs, strided rows.
* h3_gemm_fp8: against the oracle's fp8 product of the GPU's own codes and
  scales: 4e-3 for a bf16 output (one rounding, 2^-9 per stored element),
  1e-4 for fp32.  The products are exact, but the fp8 MFMA's sums carry a
  relative error near 2^-16 (measured 1.4-1.7e-5 at every K from 128 to
  5376, so per instruction rather than growing with K); ragged M and N.
* End to end (quantise both operands, then multiply) against the
  unquantised fp64 product: the derived quantisation bound 6e-2.
* The 15 s 768p QKV projection (92840 x 21504 x 5376) on sampled rows.
"""
import numpy as np
import pytest

import oracle
from video_audio_diffusion_amd import blk, inputs
from video_audio_diffusion_amd.block import device_inputs, host_array

from gpu_util import assert_close

pytestmark = pytest.mark.gpu


def _dev(a):
    return device_inputs(None, {"a": a})["a"]


def _quantize(x_dev, n, K, dtype, ldq=None):
    import torch
    ldq = ldq or K
    q = torch.full((n, ldq), 0x55, dtype=torch.uint8, device="cuda")
    s = torch.full((n,), -1.0, dtype=torch.float32, device="cuda")
    blk.h3_quantize_fp8(x_dev, x_dev.stride(0), n, K, q, ldq, s, blk.H3_BF16 if dtype == "bf16" else blk.H3_F32)
    return q, s


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("n,K,pad", [(1, 16, 0), (37, 80, 8), (300, 5376, 0)])
def test_quantize_bit_exact(dtype, n, K, pad):
    import torch
    x = inputs.draw_rows(None, (n, K + pad), 900 + n, dtype=dtype)
    w = inputs.widen(x, dtype).astype(np.float32)
    if n > 3:
        x[1] = 0                                            # all-zero row: scale 1, codes 0
        x[2, 3] = inputs.store(np.array([3.0e4], np.float32), dtype)[0]   # one large outlier
        x[2, 5:9] = inputs.store(np.array([1e-4, -2e-4, 3e-6, -0.0], np.float32), dtype)
        w = inputs.widen(x, dtype).astype(np.float32)
    d = _dev(x)
    q, s = _quantize(d[:, :K], n, K, dtype, ldq=K + (16 if pad else 0))
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_rows(w[:, :K])
    got_s = s.cpu().numpy()
    assert np.array_equal(got_s, s_ref), "scales differ"
    got_q = q.cpu().numpy()
    assert np.array_equal(got_q[:, :K], q_ref), f"codes differ at {np.argwhere(got_q[:, :K] != q_ref)[:5]}"
    if pad:
        assert np.all(got_q[:, K:] == 0x55), "wrote past K"


@pytest.mark.parametrize("K", [4096, 7168, 11264, 14336, 20480])
def test_quantize_bit_exact_widths(K):
    """Every row width class of the bf16 quantiser (rows held in registers up
    to 14336 values, the general kernel beyond), and rows holding an
    infinity, which take the general arithmetic: a scale of inf, codes 0
    (0x80 for negative values) and 0x7F for the infinity itself (inf / inf).
    Rows holding a NaN are left out: the oracle's NaN-propagating max and the
    kernel's max differ there, and nothing specifies that case."""
    n = 7
    x = inputs.draw_rows(None, (n, K), 950 + K, dtype="bf16")
    x[1] = 0
    x[2, 7] = inputs.store(np.array([2.5e4], np.float32), "bf16")[0]
    x[3, K // 3] = inputs.store(np.array([np.inf], np.float32), "bf16")[0]
    x[4, K - 1] = inputs.store(np.array([-np.inf], np.float32), "bf16")[0]
    x[5, 5:9] = inputs.store(np.array([1e-4, -2e-4, 3e-6, -0.0], np.float32), "bf16")
    w = inputs.widen(x, "bf16").astype(np.float32)
    q, s = _quantize(_dev(x), n, K, "bf16")
    import torch
    torch.cuda.synchronize()
    with np.errstate(invalid="ignore"):
        q_ref, s_ref = oracle.quantize_rows(w)
    got_s = s.cpu().numpy()
    assert np.array_equal(got_s, s_ref), f"scales differ: {got_s} {s_ref}"
    got_q = q.cpu().numpy()
    assert np.array_equal(got_q, q_ref), f"codes differ at {np.argwhere(got_q != q_ref)[:5]}"


@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("M,N,K", [(1, 8, 128), (255, 200, 384), (513, 1032, 1024), (300, 264, 5376)])
def test_gemm_fp8_against_oracle(out, M, N, K):
    import torch
    a = inputs.draw_rows(None, (M, K), 950 + M, dtype="bf16")
    w = inputs.draw_rows(None, (N, K), 960 + N, dtype="bf16")
    qa, sa = _quantize(_dev(a), M, K, "bf16")
    qw, sw = _quantize(_dev(w), N, K, "bf16")
    tdt = torch.bfloat16 if out == "bf16" else torch.float32
    c = torch.full((M, N), float("nan"), dtype=tdt, device="cuda")
    blk.h3_gemm_fp8(qa, K, sa, qw, K, sw, c, N, M, N, K, blk.H3_BF16 if out == "bf16" else blk.H3_F32)
    torch.cuda.synchronize()
    ref = oracle.gemm_fp8(qa.cpu().numpy(), sa.cpu().numpy(), qw.cpu().numpy(), sw.cpu().numpy())
    got = inputs.widen(host_array(c, out), out)
    assert_close(f"gemm_fp8 {M}x{N}x{K} -> {out}", got, ref, 4e-3 if out == "bf16" else 1e-4)


def test_fp8_quantisation_error_bound():
    """Activations N(0,1), weights N(0, 0.02^2), both bf16: the fp8 product is
    within the derived bound of the unquantised product."""
    import torch
    M, N, K = 512, 768, 5376
    a = inputs.draw_rows(None, (M, K), 970, dtype="bf16")
    w = inputs.store(inputs.widen(inputs.draw_rows(None, (N, K), 971, dtype="f32"), "f32") * 0.02, "bf16")
    qa, sa = _quantize(_dev(a), M, K, "bf16")
    qw, sw = _quantize(_dev(w), N, K, "bf16")
    c = torch.empty((M, N), dtype=torch.float32, device="cuda")
    blk.h3_gemm_fp8(qa, K, sa, qw, K, sw, c, N, M, N, K, blk.H3_F32)
    torch.cuda.synchronize()
    ref = oracle.linear(inputs.widen(a, "bf16"), inputs.widen(w, "bf16"))
    assert_close("fp8 vs unquantised", host_array(c, "f32"), ref, 6e-2)


def test_768p15s_qkv_fp8_sampled():
    import torch
    c3 = inputs.CONFIGS[3]
    M, K, N = c3.n_tok, c3.dim, 3 * c3.inner
    host = inputs.make_inputs(c3, ("x", "w_qkv"))
    x, w = _dev(host["x"]), _dev(host["w_qkv"])
    qa, sa = _quantize(x, M, K, "bf16")
    qw, sw = _quantize(w, N, K, "bf16")
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    blk.h3_gemm_fp8(qa, K, sa, qw, K, sw, out, N, M, N, K, blk.H3_BF16)
    torch.cuda.synchronize()
    rows = inputs.sample_rows(c3, n_random=96)
    idx = torch.from_numpy(rows).cuda()
    ref = oracle.gemm_fp8(qa.index_select(0, idx).cpu().numpy(), sa.index_select(0, idx).cpu().numpy(),
                          qw.cpu().numpy(), sw.cpu().numpy())
    got = inputs.widen(host_array(out.index_select(0, idx), "bf16"), "bf16")
    assert_close("qkv_fp8 sampled", got, ref, 4e-3)
    exact = oracle.linear(inputs.widen(host["x"][rows], "bf16"), inputs.widen(host["w_qkv"], "bf16"))
    assert_close("qkv_fp8 vs unquantised", got, exact, 6e-2)
