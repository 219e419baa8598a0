"""ctypes binding of libh3blk: the six block calls under their C names.

Argument marshalling only: every function takes the C arguments in C order
(device tensors may stand in for device pointers), calls the library and
raises H3Error on a non-zero status.  All arithmetic runs in the library's
HIP kernels; there is no fallback of any kind -- if libh3blk.so is missing,
loading fails with an error that says how to build it.
"""
from __future__ import annotations

import ctypes
import os
from typing import Iterable, Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libh3blk.so")

H3_OK, H3_ERR_ARG, H3_ERR_SEGMENTS, H3_ERR_DTYPE, H3_ERR_ALIGN, H3_ERR_SHAPE, H3_ERR_HIP = range(7)
H3_BF16, H3_F32 = 0, 1
H3_BRANCH_ATTN, H3_BRANCH_FFN = 0, 1
H3_MAX_SEGMENTS = 64

EXPORTS = ("h3_status_str", "h3_adaln_modulate", "h3_gemm_bf16", "h3_qknorm_rope3d",
           "h3_attention_fwd", "h3_swiglu", "h3_gate_residual", "h3_euler_update",
           "h3_gemm_gate_residual", "h3_gemm_swiglu", "h3_patchify", "h3_unpatchify", "h3_quantize_fp8",
           "h3_gemm_fp8", "h3_gemm_fp8_gate_residual", "h3_gemm_fp8_swiglu", "h3_quantize_qkv_fp8",
           "h3_attention_fp8", "h3_gemm_qknorm_rope", "h3_gemm_fp8_qknorm_rope", "h3_interleave_gate_up")


class H3Segment(ctypes.Structure):
    _fields_ = [("start", ctypes.c_int64), ("len", ctypes.c_int64), ("mod_set", ctypes.c_int32),
                ("T", ctypes.c_int32), ("H", ctypes.c_int32), ("W", ctypes.c_int32),
                ("t0", ctypes.c_int32), ("h0", ctypes.c_int32), ("w0", ctypes.c_int32)]


class H3Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {status_str(status)} (status {status})")


_lib = None
_P, _I64, _I32, _F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
_SIGS = {
    "h3_adaln_modulate": [_P, _P, _I64, _I32, _P, _I32, _I32, _P, _I32, _F, _I32, _P],
    "h3_gemm_bf16": [_P, _I64, _P, _I64, _P, _I64, _I64, _I32, _I32, _I32, _P],
    "h3_qknorm_rope3d": [_P, _P, _I64, _I64, _I32, _I32, _P, _P, _F, _I32, _I32, _I32, _F, _P, _I32, _I32, _P],
    "h3_attention_fwd": [_P, _P, _P, _I64, _P, _I64, _I64, _I32, _I32, _F, _P, _I32, _P],
    "h3_swiglu": [_P, _P, _I64, _I32, _I32, _P],
    "h3_gate_residual": [_P, _P, _P, _I64, _I32, _P, _I32, _I32, _P, _I32, _I32, _P],
    "h3_euler_update": [_P, _P, _I64, _I32, _P, _P, _I32, _I32, _P],
    "h3_gemm_gate_residual": [_P, _I64, _P, _I64, _P, _P, _I64, _I64, _I32, _I32, _P, _I32, _I32, _P, _I32, _I32,
                              _P],
    "h3_gemm_swiglu": [_P, _I64, _P, _I64, _P, _I64, _I64, _I32, _I32, _I32, _P],
    "h3_interleave_gate_up": [_P, _I64, _P, _I64, _I32, _I32, _I32, _P],
    "h3_gemm_qknorm_rope": [_P, _I64, _P, _I64, _P, _I64, _I64, _I32, _I32, _I32, _I32, _P, _P, _F, _I32, _I32,
                            _I32, _F, _P, _I32, _I32, _P],
    "h3_patchify": [_P, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _P, _I64, _I32, _P],
    "h3_unpatchify": [_P, _I64, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _P, _I32, _P],
    "h3_quantize_fp8": [_P, _I64, _I64, _I32, _P, _I64, _P, _I32, _P],
    "h3_gemm_fp8": [_P, _I64, _P, _P, _I64, _P, _P, _I64, _I64, _I32, _I32, _I32, _P],
    "h3_gemm_fp8_gate_residual": [_P, _I64, _P, _P, _I64, _P, _P, _P, _I64, _I64, _I32, _I32, _P, _I32, _I32, _P,
                                  _I32, _P],
    "h3_gemm_fp8_swiglu": [_P, _I64, _P, _P, _I64, _P, _P, _I64, _I64, _I32, _I32, _P],
    "h3_gemm_fp8_qknorm_rope": [_P, _I64, _P, _P, _I64, _P, _P, _I64, _I64, _I32, _I32, _I32, _I32, _P, _P, _F,
                                _I32, _I32, _I32, _F, _P, _I32, _P],
    "h3_quantize_qkv_fp8": [_P, _P, _P, _I64, _I64, _I32, _I32, _P, _P, _P, _I64, _P, _P, _P, _I32, _P],
    "h3_attention_fp8": [_P, _P, _P, _I64, _P, _P, _P, _P, _I64, _I64, _I32, _I32, _F, _P],
}


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libh3blk.so (once).  Raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise ImportError(f"{path} is not built: run `python -m video_audio_diffusion_amd.build`")
        lib = ctypes.CDLL(path)
        lib.h3_status_str.restype = ctypes.c_char_p
        lib.h3_status_str.argtypes = [ctypes.c_int]
        for name, args in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = ctypes.c_int
            fn.argtypes = args
        _lib = lib
    return _lib


def status_str(s: int) -> str:
    return load().h3_status_str(s).decode()


def ptr(t) -> Optional[int]:
    """Device pointer of a tensor (or an int/None passed through)."""
    if t is None or isinstance(t, int):
        return t
    return t.data_ptr()


def dtype_of(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return H3_BF16
    if t.dtype == torch.float32:
        return H3_F32
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


def current_stream() -> int:
    import torch
    return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else 0


def segments(segs: Iterable) -> "ctypes.Array":
    """Host interval table from objects with start/length/mod_set/T/H/W/t0/h0/w0."""
    segs = list(segs)
    arr = (H3Segment * max(1, len(segs)))()
    for i, s in enumerate(segs):
        arr[i] = H3Segment(s.start, getattr(s, "length", getattr(s, "len", 0)), s.mod_set, s.T, s.H, s.W,
                           s.t0, s.h0, s.w0)
    return arr


def _check(fn: str, status: int) -> None:
    if status != H3_OK:
        raise H3Error(fn, status)


def _stream(stream) -> int:
    return current_stream() if stream is None else stream


def h3_adaln_modulate(x, y, n_tok, dim, mod, n_sets, br, segs, n_segs, eps, dt, stream=None):
    _check("h3_adaln_modulate", load().h3_adaln_modulate(ptr(x), ptr(y), n_tok, dim, ptr(mod), n_sets, br, segs,
                                                         n_segs, eps, dt, _stream(stream)))


def h3_gemm_bf16(A, lda, W, ldw, C, ldc, M, N, K, dt, stream=None):
    _check("h3_gemm_bf16", load().h3_gemm_bf16(ptr(A), lda, ptr(W), ldw, ptr(C), ldc, M, N, K, dt, _stream(stream)))


def h3_gemm_gate_residual(A, lda, W, ldw, x, out, ldo, M, N, K, mod, n_sets, br, segs, n_segs, dt, stream=None):
    _check("h3_gemm_gate_residual",
           load().h3_gemm_gate_residual(ptr(A), lda, ptr(W), ldw, ptr(x), ptr(out), ldo, M, N, K, ptr(mod), n_sets,
                                        br, segs, n_segs, dt, _stream(stream)))


def h3_gemm_swiglu(A, lda, Wgu, ldw, H, ldh, M, F, K, dt, stream=None):
    _check("h3_gemm_swiglu", load().h3_gemm_swiglu(ptr(A), lda, ptr(Wgu), ldw, ptr(H), ldh, M, F, K, dt,
                                                   _stream(stream)))


def h3_gemm_qknorm_rope(A, lda, W, ldw, C, ldc, M, N, K, heads, head_dim, gamma_q, gamma_k, eps, d_t, d_h, d_w,
                        rope_base, segs, n_segs, dt, stream=None):
    _check("h3_gemm_qknorm_rope",
           load().h3_gemm_qknorm_rope(ptr(A), lda, ptr(W), ldw, ptr(C), ldc, M, N, K, heads, head_dim, ptr(gamma_q),
                                      ptr(gamma_k), eps, d_t, d_h, d_w, rope_base, segs, n_segs, dt,
                                      _stream(stream)))


def h3_patchify(latent, T, H, W, C, pt, ph, pw, tokens, ld, dt, stream=None):
    _check("h3_patchify", load().h3_patchify(ptr(latent), T, H, W, C, pt, ph, pw, ptr(tokens), ld, dt,
                                             _stream(stream)))


def h3_unpatchify(tokens, ld, T, H, W, C, pt, ph, pw, latent, dt, stream=None):
    _check("h3_unpatchify", load().h3_unpatchify(ptr(tokens), ld, T, H, W, C, pt, ph, pw, ptr(latent), dt,
                                                 _stream(stream)))


def h3_quantize_fp8(x, ldx, n_rows, K, q, ldq, scales, dt, stream=None):
    _check("h3_quantize_fp8", load().h3_quantize_fp8(ptr(x), ldx, n_rows, K, ptr(q), ldq, ptr(scales), dt,
                                                     _stream(stream)))


def h3_gemm_fp8(A, lda, a_scale, W, ldw, w_scale, C, ldc, M, N, K, out_dt, stream=None):
    _check("h3_gemm_fp8", load().h3_gemm_fp8(ptr(A), lda, ptr(a_scale), ptr(W), ldw, ptr(w_scale), ptr(C), ldc, M, N,
                                             K, out_dt, _stream(stream)))


def h3_gemm_fp8_gate_residual(A, lda, a_scale, W, ldw, w_scale, x, out, ldo, M, N, K, mod, n_sets, br, segs, n_segs,
                              stream=None):
    _check("h3_gemm_fp8_gate_residual",
           load().h3_gemm_fp8_gate_residual(ptr(A), lda, ptr(a_scale), ptr(W), ldw, ptr(w_scale), ptr(x), ptr(out), ldo,
                                            M, N, K, ptr(mod), n_sets, br, segs, n_segs, _stream(stream)))


def h3_gemm_fp8_swiglu(A, lda, a_scale, Wgu, ldw, w_scale, H, ldh, M, F, K, stream=None):
    _check("h3_gemm_fp8_swiglu", load().h3_gemm_fp8_swiglu(ptr(A), lda, ptr(a_scale), ptr(Wgu), ldw, ptr(w_scale),
                                                           ptr(H), ldh, M, F, K, _stream(stream)))


def h3_gemm_fp8_qknorm_rope(A, lda, a_scale, W, ldw, w_scale, C, ldc, M, N, K, heads, head_dim, gamma_q, gamma_k,
                            eps, d_t, d_h, d_w, rope_base, segs, n_segs, stream=None):
    _check("h3_gemm_fp8_qknorm_rope",
           load().h3_gemm_fp8_qknorm_rope(ptr(A), lda, ptr(a_scale), ptr(W), ldw, ptr(w_scale), ptr(C), ldc, M, N, K,
                                          heads, head_dim, ptr(gamma_q), ptr(gamma_k), eps, d_t, d_h, d_w, rope_base,
                                          segs, n_segs, _stream(stream)))


def h3_quantize_qkv_fp8(q, k, v, ld, n_tok, heads, head_dim, q8, k8, vt, n_pad, sq, sk, sv, dt, stream=None):
    _check("h3_quantize_qkv_fp8", load().h3_quantize_qkv_fp8(ptr(q), ptr(k), ptr(v), ld, n_tok, heads, head_dim,
                                                             ptr(q8), ptr(k8), ptr(vt), n_pad, ptr(sq), ptr(sk),
                                                             ptr(sv), dt, _stream(stream)))


def h3_attention_fp8(q8, k8, vt, n_pad, sq, sk, sv, o, ld_o, n_tok, heads, head_dim, scale, stream=None):
    _check("h3_attention_fp8", load().h3_attention_fp8(ptr(q8), ptr(k8), ptr(vt), n_pad, ptr(sq), ptr(sk), ptr(sv),
                                                       ptr(o), ld_o, n_tok, heads, head_dim, scale, _stream(stream)))


def interleave_gate_up_rows(F: int):
    """Row order that turns a [gate | up] weight of 2F rows into the layout
    h3_gemm_swiglu reads: 32 gate rows, then the 32 matching up rows, and so
    on.  Returns the source row of every destination row (a weight-loading
    permutation, applied once)."""
    if F % 32:
        raise ValueError("F must be a multiple of 32")
    out = []
    for u in range(F // 32):
        out.extend(range(32 * u, 32 * u + 32))
        out.extend(range(F + 32 * u, F + 32 * u + 32))
    return out


def h3_interleave_gate_up(w_gu, ld_src, w_il, ld_dst, F, K, dt, stream=None):
    _check("h3_interleave_gate_up", load().h3_interleave_gate_up(ptr(w_gu), ld_src, ptr(w_il), ld_dst, F, K, dt,
                                                                 _stream(stream)))


def h3_qknorm_rope3d(q, k, ld, n_tok, heads, head_dim, gamma_q, gamma_k, eps, d_t, d_h, d_w, rope_base,
                     segs, n_segs, dt, stream=None):
    _check("h3_qknorm_rope3d", load().h3_qknorm_rope3d(ptr(q), ptr(k), ld, n_tok, heads, head_dim, ptr(gamma_q),
                                                       ptr(gamma_k), eps, d_t, d_h, d_w, rope_base, segs, n_segs,
                                                       dt, _stream(stream)))


def h3_attention_fwd(q, k, v, ld_qkv, o, ld_o, n_tok, heads, head_dim, scale, lse, dt, stream=None):
    _check("h3_attention_fwd", load().h3_attention_fwd(ptr(q), ptr(k), ptr(v), ld_qkv, ptr(o), ld_o, n_tok, heads,
                                                       head_dim, scale, ptr(lse), dt, _stream(stream)))


def h3_swiglu(gu, h, n_tok, F, dt, stream=None):
    _check("h3_swiglu", load().h3_swiglu(ptr(gu), ptr(h), n_tok, F, dt, _stream(stream)))


def h3_gate_residual(x, y, out, n_tok, dim, mod, n_sets, br, segs, n_segs, dt, stream=None):
    _check("h3_gate_residual", load().h3_gate_residual(ptr(x), ptr(y), ptr(out), n_tok, dim, ptr(mod), n_sets, br,
                                                       segs, n_segs, dt, _stream(stream)))


def coefficients(values: Iterable[float]) -> "ctypes.Array":
    """Host fp32 array, one value per interval (h3_euler_update)."""
    values = list(values)
    arr = (ctypes.c_float * max(1, len(values)))()
    for i, v in enumerate(values):
        arr[i] = float(v)
    return arr


def h3_euler_update(x, v, n_tok, dim, coef, segs, n_segs, dt, stream=None):
    _check("h3_euler_update", load().h3_euler_update(ptr(x), ptr(v), n_tok, dim, coef, segs, n_segs, dt,
                                                     _stream(stream)))
