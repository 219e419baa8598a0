"""Helpers for the GPU parity tests (device setup, error metrics, running the
block through the C ABI with every intermediate kept)."""
import numpy as np

from video_audio_diffusion_amd import blk, inputs
from video_audio_diffusion_amd.block import device_inputs, host_array

TOL = {"f32": 1e-5, "bf16": 2e-2}


def rel_errors(got, ref):
    """Per-tensor max error relative to the largest reference magnitude, and
    the Frobenius-norm relative error."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = got - ref
    e_max = np.abs(d).max() / max(np.abs(ref).max(), 1e-300)
    e_f = np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300)
    return float(e_max), float(e_f)


def assert_close(name, got, ref, tol):
    e_max, e_f = rel_errors(got, ref)
    print(f"  {name}: e_max={e_max:.3e} e_F={e_f:.3e} (tol {tol:g})", flush=True)
    assert e_max <= tol and e_f <= tol, f"{name}: e_max={e_max:.3e} e_F={e_f:.3e} > {tol}"


def assert_delta_close(name, got_out, ref_out, x, tol, dtype):
    """Parity of the residual-branch contribution out - x.  The output is
    stored in `dtype`, so each element may differ from the exact value by up
    to one spacing of that format at |out| before the branch error counts
    (2^-8 relative for bf16, 2^-23 for fp32)."""
    got_out, ref_out, x = (np.asarray(a, dtype=np.float64) for a in (got_out, ref_out, x))
    unit = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -23
    d = np.abs((got_out - x) - (ref_out - x))
    excess = np.maximum(d - unit * np.abs(ref_out), 0.0)
    ref_d = ref_out - x
    e_max = excess.max() / np.abs(ref_d).max()
    e_f = np.linalg.norm(excess) / np.linalg.norm(ref_d)
    print(f"  {name}: e_max={e_max:.3e} e_F={e_f:.3e} beyond output rounding (tol {tol:g})", flush=True)
    assert e_max <= tol and e_f <= tol, f"{name}: e_max={e_max:.3e} e_F={e_f:.3e} > {tol}"


def widen(t, dtype):
    return inputs.widen(host_array(t, dtype), dtype)


def run_block_steps(cfg, dev, x=None):
    """Run the eleven calls with a separate buffer per intermediate; returns a
    dict of device tensors (a, qkv_raw, qkv, o, y, x1, a2, gu, h, f, out)."""
    import torch
    N, D, H, d, I, F = cfg.n_tok, cfg.dim, cfg.heads, cfg.head_dim, cfg.inner, cfg.ffn
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    dt = blk.H3_BF16 if cfg.dtype == "bf16" else blk.H3_F32
    e = lambda *s: torch.empty(*s, dtype=tdt, device="cuda")
    x = dev["x"] if x is None else x
    mod, segs, ns = dev["mod"], blk.segments(cfg.segments), len(cfg.segments)
    r = {"a": e(N, D), "qkv": e(N, 3 * I), "o": e(N, I), "y": e(N, D), "x1": e(N, D), "a2": e(N, D),
         "gu": e(N, 2 * F), "h": e(N, F), "f": e(N, D), "out": e(N, D)}
    blk.h3_adaln_modulate(x, r["a"], N, D, mod, 3, blk.H3_BRANCH_ATTN, segs, ns, cfg.eps, dt)
    blk.h3_gemm_bf16(r["a"], D, dev["w_qkv"], D, r["qkv"], 3 * I, N, 3 * I, D, dt)
    r["qkv_raw"] = r["qkv"].clone()
    q, k, v = r["qkv"][:, :I], r["qkv"][:, I:2 * I], r["qkv"][:, 2 * I:]
    blk.h3_qknorm_rope3d(q, k, 3 * I, N, H, d, dev["gamma_q"], dev["gamma_k"], cfg.eps, *cfg.rope_split,
                         cfg.rope_base, segs, ns, dt)
    blk.h3_attention_fwd(q, k, v, 3 * I, r["o"], I, N, H, d, cfg.scale, None, dt)
    blk.h3_gemm_bf16(r["o"], I, dev["w_o"], I, r["y"], D, N, D, I, dt)
    blk.h3_gate_residual(x, r["y"], r["x1"], N, D, mod, 3, blk.H3_BRANCH_ATTN, segs, ns, dt)
    blk.h3_adaln_modulate(r["x1"], r["a2"], N, D, mod, 3, blk.H3_BRANCH_FFN, segs, ns, cfg.eps, dt)
    blk.h3_gemm_bf16(r["a2"], D, dev["w_gu"], D, r["gu"], 2 * F, N, 2 * F, D, dt)
    blk.h3_swiglu(r["gu"], r["h"], N, F, dt)
    blk.h3_gemm_bf16(r["h"], F, dev["w_d"], F, r["f"], D, N, D, F, dt)
    blk.h3_gate_residual(r["x1"], r["f"], r["out"], N, D, mod, 3, blk.H3_BRANCH_FFN, segs, ns, dt)
    torch.cuda.synchronize()
    return r


def oracle_inputs(cfg, host):
    """fp64 copies of the host inputs for the oracle."""
    return {k: (inputs.widen(v, cfg.dtype) if k not in ("mod", "gamma_q", "gamma_k") else v.astype(np.float64))
            for k, v in host.items()}


def make_device(cfg, host):
    return device_inputs(cfg, host)

