"""C-ABI checks that need no GPU: the library loads, exports every call the
header declares, and rejects every kind of bad argument before touching the
device.  Pointers here are fake (never dereferenced): validation fails first,
or, for valid arguments on a machine with no GPU, the launch fails with
H3_ERR_HIP."""
import ctypes
import os
import re

import pytest

from video_audio_diffusion_amd import blk, inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
P = 0x7f0000000000            # fake, 16-byte aligned device addresses
CFG1 = inputs.CONFIGS[1]
CFG2 = inputs.CONFIGS[2]


def _no_gpu():
    import torch
    return torch.cuda.device_count() == 0


@pytest.fixture(scope="module")
def lib():
    return blk.load()


def test_exports_every_header_symbol(lib):
    hdr = open(os.path.join(ROOT, "include", "h3blk.h")).read()
    declared = set(re.findall(r"^\s*(?:h3_status|const char\*)\s+(h3_\w+)\(", hdr, re.M))
    assert declared == set(blk.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for s in range(7):
        assert isinstance(blk.status_str(s), str) and blk.status_str(s)
    assert blk.status_str(99) == "unknown status"


def test_segment_struct_layout():
    assert ctypes.sizeof(blk.H3Segment) == 48
    assert blk.H3Segment.T.offset == 20 and blk.H3Segment.w0.offset == 40


def _adaln(segs=None, n_segs=None, **kw):
    a = dict(x=P, y=P + (1 << 30), n_tok=CFG1.n_tok, dim=CFG1.dim, mod=P + (2 << 30), n_sets=3, br=0,
             eps=1e-6, dt=blk.H3_F32)
    a.update(kw)
    segs = blk.segments(CFG1.segments) if segs is None else segs
    n_segs = len(CFG1.segments) if n_segs is None else n_segs
    return blk.load().h3_adaln_modulate(a["x"], a["y"], a["n_tok"], a["dim"], a["mod"], a["n_sets"], a["br"],
                                        segs, n_segs, a["eps"], a["dt"], 0)


def test_adaln_validation(lib):
    assert _adaln(dt=5) == blk.H3_ERR_DTYPE
    assert _adaln(x=0) == blk.H3_ERR_ARG
    assert _adaln(mod=0) == blk.H3_ERR_ARG
    assert _adaln(br=2) == blk.H3_ERR_ARG
    assert _adaln(eps=-1.0) == blk.H3_ERR_ARG
    assert _adaln(eps=float("nan")) == blk.H3_ERR_ARG
    assert _adaln(x=P + 4) == blk.H3_ERR_ALIGN
    assert _adaln(dim=196) == blk.H3_ERR_SHAPE
    assert _adaln(dim=8192, dt=blk.H3_F32) == blk.H3_ERR_SHAPE     # fp32 rows hold at most 4096
    assert _adaln(y=P + 64) == blk.H3_ERR_ARG                     # y overlaps x
    assert _adaln(n_tok=-1) == blk.H3_ERR_ARG


def _segs(*rows):
    arr = (blk.H3Segment * len(rows))()
    for i, r in enumerate(rows):
        arr[i] = blk.H3Segment(*r)
    return arr


def test_interval_table_validation(lib):
    good = [(0, 16, 0, 16, 1, 1, 0, 0, 0), (16, 8, 2, 8, 1, 1, 0, 0, 0), (24, 48, 1, 2, 4, 6, 0, 0, 0)]
    bad = {
        "gap": [(0, 16, 0, 16, 1, 1, 0, 0, 0), (17, 8, 2, 8, 1, 1, 0, 0, 0), (25, 47, 1, 47, 1, 1, 0, 0, 0)],
        "overlap": [(0, 16, 0, 16, 1, 1, 0, 0, 0), (15, 8, 2, 8, 1, 1, 0, 0, 0), (23, 49, 1, 49, 1, 1, 0, 0, 0)],
        "unsorted": [(16, 8, 2, 8, 1, 1, 0, 0, 0), (0, 16, 0, 16, 1, 1, 0, 0, 0), (24, 48, 1, 2, 4, 6, 0, 0, 0)],
        "len!=THW": [(0, 16, 0, 16, 1, 1, 0, 0, 0), (16, 8, 2, 8, 1, 1, 0, 0, 0), (24, 48, 1, 2, 4, 5, 0, 0, 0)],
        "short": [(0, 16, 0, 16, 1, 1, 0, 0, 0), (16, 8, 2, 8, 1, 1, 0, 0, 0)],
        "long": good + [(72, 1, 0, 1, 1, 1, 0, 0, 0)],
        "mod_set": [(0, 16, 0, 16, 1, 1, 0, 0, 0), (16, 8, 3, 8, 1, 1, 0, 0, 0), (24, 48, 1, 2, 4, 6, 0, 0, 0)],
        "neg_offset": [(0, 16, 0, 16, 1, 1, -1, 0, 0), (16, 8, 2, 8, 1, 1, 0, 0, 0), (24, 48, 1, 2, 4, 6, 0, 0, 0)],
        "zero_grid": [(0, 16, 0, 16, 1, 1, 0, 0, 0), (16, 0, 2, 0, 1, 1, 0, 0, 0), (16, 56, 1, 56, 1, 1, 0, 0, 0)],
    }
    for name, rows in bad.items():
        assert _adaln(segs=_segs(*rows), n_segs=len(rows)) == blk.H3_ERR_SEGMENTS, name
    many = [(i, 1, 0, 1, 1, 1, 0, 0, 0) for i in range(65)]
    assert _adaln(segs=_segs(*many), n_segs=65, n_tok=65) == blk.H3_ERR_SEGMENTS
    assert _adaln(segs=None, n_segs=0) == blk.H3_ERR_SEGMENTS
    assert blk.load().h3_adaln_modulate(P, P + (1 << 30), 72, 192, P, 3, 0, None, 3, 1e-6, 1, 0) == blk.H3_ERR_ARG


def test_empty_sequence_is_a_no_op(lib):
    # nothing is launched for zero tokens, so this succeeds even with no GPU
    assert _adaln(n_tok=0, segs=None, n_segs=0) == blk.H3_OK
    L = blk.load()
    assert L.h3_gemm_bf16(P, 64, P + (1 << 30), 64, P + (2 << 30), 64, 0, 64, 64, 0, 0) == blk.H3_OK
    assert L.h3_swiglu(P, P + (1 << 30), 0, 64, 0, 0) == blk.H3_OK
    assert L.h3_attention_fwd(P, P + 256, P + 512, 384, P + (1 << 30), 128, 0, 1, 128, 0.1, None, 0, 0) == blk.H3_OK
    assert L.h3_qknorm_rope3d(P, P + 256, 384, 0, 1, 128, None, None, 1e-6, 64, 32, 32, 1e4, None, 0, 0, 0) == 0
    assert L.h3_gate_residual(P, P + (1 << 30), P, 0, 64, P + (2 << 30), 3, 0, None, 0, 0, 0) == blk.H3_OK


def test_gemm_validation(lib):
    L = blk.load()
    A, W, C = P, P + (1 << 32), P + (2 << 32)
    g = lambda **k: L.h3_gemm_bf16(k.get("A", A), k.get("lda", 5376), k.get("W", W), k.get("ldw", 5376),
                                   k.get("C", C), k.get("ldc", 21504), k.get("M", 100), k.get("N", 21504),
                                   k.get("K", 5376), k.get("dt", 0), 0)
    assert g(dt=2) == blk.H3_ERR_DTYPE
    assert g(A=0) == blk.H3_ERR_ARG
    assert g(lda=100) == blk.H3_ERR_ARG
    assert g(ldc=100) == blk.H3_ERR_ARG
    assert g(K=5376 - 8, lda=5376 - 8, ldw=5376 - 8) == blk.H3_ERR_SHAPE   # bf16 K % 64
    assert g(N=21500, ldc=21504) == blk.H3_ERR_SHAPE
    assert g(A=A + 2) == blk.H3_ERR_ALIGN
    assert g(lda=5380) == blk.H3_ERR_ALIGN
    assert g(C=A + 1024) == blk.H3_ERR_ARG                                   # C overlaps A
    assert g(M=-1) == blk.H3_ERR_ARG
    assert g(M=1 << 31) == blk.H3_ERR_SHAPE


def test_qknorm_rope_validation(lib):
    L = blk.load()
    segs = blk.segments(CFG2.segments)
    q, k = P, P + 7168 * 2
    def r(**kw):
        a = dict(q=q, k=k, ld=21504, n=CFG2.n_tok, heads=56, hd=128, gq=None, gk=None, eps=1e-6, dt_=64, dh=32,
                 dw=32, base=1e4, segs=segs, ns=len(CFG2.segments), dt=0)
        a.update(kw)
        return L.h3_qknorm_rope3d(a["q"], a["k"], a["ld"], a["n"], a["heads"], a["hd"], a["gq"], a["gk"], a["eps"],
                                  a["dt_"], a["dh"], a["dw"], a["base"], a["segs"], a["ns"], a["dt"], 0)
    assert r(dt=3) == blk.H3_ERR_DTYPE
    assert r(hd=96) == blk.H3_ERR_SHAPE
    assert r(dt_=63, dh=33) == blk.H3_ERR_SHAPE
    assert r(dt_=64, dh=32, dw=30) == blk.H3_ERR_SHAPE
    assert r(base=0.0) == blk.H3_ERR_ARG
    assert r(ld=7000) == blk.H3_ERR_ARG
    assert r(k=q + 128) == blk.H3_ERR_ARG             # k columns overlap q's
    assert r(gq=P + 2) == blk.H3_ERR_ALIGN
    assert r(ns=2) == blk.H3_ERR_SEGMENTS


def test_gemm_qknorm_rope_validation(lib):
    L = blk.load()
    A, W, C = P, P + (1 << 32), P + (2 << 32)
    segs = blk.segments(CFG2.segments)
    def g(**kw):
        a = dict(A=A, lda=5376, W=W, ldw=5376, C=C, ldc=21504, M=CFG2.n_tok, N=21504, K=5376, heads=56, hd=128,
                 gq=None, gk=None, eps=1e-6, dt_=64, dh=32, dw=32, base=1e4, segs=segs, ns=len(CFG2.segments), dt=0)
        a.update(kw)
        return L.h3_gemm_qknorm_rope(a["A"], a["lda"], a["W"], a["ldw"], a["C"], a["ldc"], a["M"], a["N"], a["K"],
                                     a["heads"], a["hd"], a["gq"], a["gk"], a["eps"], a["dt_"], a["dh"], a["dw"],
                                     a["base"], a["segs"], a["ns"], a["dt"], 0)
    assert g(dt=2) == blk.H3_ERR_DTYPE
    assert g(A=0) == blk.H3_ERR_ARG
    assert g(ldc=100) == blk.H3_ERR_ARG
    assert g(K=5376 - 8, lda=5368, ldw=5368) == blk.H3_ERR_SHAPE        # bf16 K % 64
    assert g(C=A + 1024) == blk.H3_ERR_ARG                                # C overlaps A
    assert g(heads=0) == blk.H3_ERR_ARG
    assert g(eps=-1.0) == blk.H3_ERR_ARG
    assert g(base=0.0) == blk.H3_ERR_ARG
    assert g(hd=96) == blk.H3_ERR_SHAPE
    assert g(dt_=63, dh=33) == blk.H3_ERR_SHAPE
    assert g(heads=55) == blk.H3_ERR_SHAPE              # q heads do not fill whole 256-column tiles
    assert g(heads=86) == blk.H3_ERR_SHAPE              # q and k need 22016 > N columns
    assert g(gq=P + 2) == blk.H3_ERR_ALIGN
    assert g(ns=2) == blk.H3_ERR_SEGMENTS
    assert g(M=0, segs=None, ns=0) == blk.H3_OK         # nothing to do, nothing launched


def test_gemm_fp8_qknorm_rope_validation(lib):
    L = blk.load()
    A, sa, W, sw, C = P, P + (1 << 31), P + (1 << 32), P + (3 << 31), P + (2 << 32)
    segs = blk.segments(CFG2.segments)
    def g(**kw):
        a = dict(A=A, lda=5376, sa=sa, W=W, ldw=5376, sw=sw, C=C, ldc=21504, M=CFG2.n_tok, N=21504, K=5376,
                 heads=56, hd=128, gq=None, gk=None, eps=1e-6, dt_=64, dh=32, dw=32, base=1e4, segs=segs,
                 ns=len(CFG2.segments))
        a.update(kw)
        return L.h3_gemm_fp8_qknorm_rope(a["A"], a["lda"], a["sa"], a["W"], a["ldw"], a["sw"], a["C"], a["ldc"],
                                         a["M"], a["N"], a["K"], a["heads"], a["hd"], a["gq"], a["gk"], a["eps"],
                                         a["dt_"], a["dh"], a["dw"], a["base"], a["segs"], a["ns"], 0)
    assert g(sa=0) == blk.H3_ERR_ARG
    assert g(K=5376 - 64, lda=5312, ldw=5312) == blk.H3_ERR_SHAPE      # fp8 K % 128
    assert g(heads=55) == blk.H3_ERR_SHAPE
    assert g(hd=96) == blk.H3_ERR_SHAPE
    assert g(base=-1.0) == blk.H3_ERR_ARG
    assert g(gk=P + 1) == blk.H3_ERR_ALIGN
    assert g(ns=1) == blk.H3_ERR_SEGMENTS
    assert g(M=0, segs=None, ns=0) == blk.H3_OK


def test_attention_validation(lib):
    L = blk.load()
    q, k, v, o = P, P + 14336, P + 28672, P + (4 << 32)
    def a(**kw):
        x = dict(q=q, k=k, v=v, ld=21504, o=o, ldo=7168, n=25616, heads=56, hd=128, scale=0.088, lse=None, dt=0)
        x.update(kw)
        return L.h3_attention_fwd(x["q"], x["k"], x["v"], x["ld"], x["o"], x["ldo"], x["n"], x["heads"], x["hd"],
                                  x["scale"], x["lse"], x["dt"], 0)
    assert a(dt=9) == blk.H3_ERR_DTYPE
    assert a(hd=32) == blk.H3_ERR_SHAPE
    assert a(o=q) == blk.H3_ERR_ARG
    assert a(ldo=100) == blk.H3_ERR_ARG
    assert a(scale=float("inf")) == blk.H3_ERR_ARG
    assert a(scale=0.0) == blk.H3_ERR_ARG       # masked keys are -inf logits: the scale must be > 0
    assert a(scale=-0.088) == blk.H3_ERR_ARG
    assert a(lse=P + 2) == blk.H3_ERR_ALIGN
    assert a(ld=1 << 24) == blk.H3_ERR_SHAPE
    assert a(q=q + 8) == blk.H3_ERR_ALIGN


def test_euler_validation(lib):
    L = blk.load()
    segs = blk.segments(CFG1.segments)
    coef = blk.coefficients([0.0, -0.01, -0.002])
    def e(x=P, v=P + (1 << 30), n=CFG1.n_tok, dim=CFG1.dim, c=coef, sg=segs, ns=3, dt=blk.H3_F32):
        return L.h3_euler_update(x, v, n, dim, c, sg, ns, dt, 0)
    assert e(dt=7) == blk.H3_ERR_DTYPE
    assert e(x=None) == blk.H3_ERR_ARG
    assert e(c=None) == blk.H3_ERR_ARG
    assert e(dim=190) == blk.H3_ERR_SHAPE
    assert e(v=P + 8) == blk.H3_ERR_ALIGN
    assert e(v=P + 64) == blk.H3_ERR_ARG                      # v overlaps x
    assert e(c=blk.coefficients([0.0, float("nan"), 0.0])) == blk.H3_ERR_ARG
    assert e(ns=2) == blk.H3_ERR_SEGMENTS                     # does not cover the tokens
    assert e(n=0, ns=0) == blk.H3_OK                          # nothing to do


def test_swiglu_and_gate_validation(lib):
    L = blk.load()
    assert L.h3_swiglu(P, P + (1 << 32), 10, 12, 0, 0) == blk.H3_ERR_SHAPE
    assert L.h3_swiglu(P, P + 64, 10, 64, 0, 0) == blk.H3_ERR_ARG          # h overlaps gu
    assert L.h3_swiglu(P, P + (1 << 32), 10, 64, 4, 0) == blk.H3_ERR_DTYPE
    segs = blk.segments(CFG1.segments)
    x, y = P, P + (1 << 30)
    assert L.h3_gate_residual(x, y, x + 64, 72, 192, P + (2 << 30), 3, 0, segs, 3, 1, 0) == blk.H3_ERR_ARG
    assert L.h3_gate_residual(x, y, y, 72, 192, P + (2 << 30), 3, 0, segs, 3, 1, 0) == blk.H3_ERR_ARG
    assert L.h3_gate_residual(x, y, x, 72, 191, P + (2 << 30), 3, 0, segs, 3, 1, 0) == blk.H3_ERR_SHAPE
    assert L.h3_gate_residual(x, y, x, 72, 192, P + (2 << 30), 2, 0, segs, 3, 1, 0) == blk.H3_ERR_SEGMENTS


def test_interleave_gate_up_validation(lib):
    L = blk.load()
    src, dst = P, P + (1 << 32)
    g = lambda src=src, ls=5376, dst=dst, ld=5376, F=14336, K=5376, dt=0: L.h3_interleave_gate_up(src, ls, dst, ld, F,
                                                                                                 K, dt, 0)
    assert g(dt=3) == blk.H3_ERR_DTYPE
    assert g(src=0) == blk.H3_ERR_ARG
    assert g(F=-32) == blk.H3_ERR_ARG
    assert g(F=48) == blk.H3_ERR_SHAPE                        # not a multiple of 32
    assert g(K=100, ls=100, ld=100) == blk.H3_ERR_SHAPE       # 200-byte rows
    assert g(ls=5000) == blk.H3_ERR_SHAPE                     # stride below K
    assert g(ld=5380) == blk.H3_ERR_SHAPE                     # rows off 16-byte boundaries
    assert g(dst=dst + 8) == blk.H3_ERR_ALIGN
    assert g(dst=src + 4096) == blk.H3_ERR_ARG                # overlap
    assert g(F=0) == blk.H3_OK                                # nothing to do


@pytest.mark.skipif(not _no_gpu(), reason="needs a machine with no GPU (fake pointers)")
def test_valid_arguments_without_a_device_report_hip_error(lib):
    assert _adaln() == blk.H3_ERR_HIP
    L = blk.load()
    assert L.h3_swiglu(P, P + (1 << 32), 10, 64, 0, 0) == blk.H3_ERR_HIP
    assert L.h3_interleave_gate_up(P, 64, P + (1 << 32), 64, 32, 64, 0, 0) == blk.H3_ERR_HIP


def test_gemm_gate_residual_validation(lib):
    L = blk.load()
    segs = blk.segments(CFG1.segments)
    A, W, x, mod = P, P + (1 << 32), P + (2 << 32), P + (3 << 32)
    M, N, K = CFG1.n_tok, 192, 128

    def g(A=A, lda=K, W=W, ldw=K, x=x, out=x, ldo=N, M=M, N=N, K=K, mod=mod, ns=3, br=0, sg=segs, nsg=3, dt=0):
        return L.h3_gemm_gate_residual(A, lda, W, ldw, x, out, ldo, M, N, K, mod, ns, br, sg, nsg, dt, 0)
    assert g(dt=3) == blk.H3_ERR_DTYPE
    assert g(x=None) == blk.H3_ERR_ARG
    assert g(mod=None) == blk.H3_ERR_ARG
    assert g(br=2) == blk.H3_ERR_ARG
    assert g(ns=0) == blk.H3_ERR_ARG
    assert g(ldo=N - 8) == blk.H3_ERR_ARG
    assert g(K=96, lda=96, ldw=96) == blk.H3_ERR_SHAPE        # bf16 K % 64
    assert g(x=x + 8) == blk.H3_ERR_ALIGN
    assert g(out=x + 64) == blk.H3_ERR_ARG                    # out partly overlaps x
    assert g(out=A) == blk.H3_ERR_ARG                         # out overlaps A
    assert g(ns=2) == blk.H3_ERR_SEGMENTS                     # an interval uses mod set 2
    assert g(nsg=2) == blk.H3_ERR_SEGMENTS                    # intervals do not cover M
    assert g(M=0, sg=None, nsg=0) == blk.H3_OK                # nothing to do


def test_gemm_swiglu_validation(lib):
    L = blk.load()
    A, W, H = P, P + (1 << 32), P + (2 << 32)

    def s(A=A, lda=5376, W=W, ldw=5376, H=H, ldh=14336, M=100, F=14336, K=5376, dt=0):
        return L.h3_gemm_swiglu(A, lda, W, ldw, H, ldh, M, F, K, dt, 0)
    assert s(dt=9) == blk.H3_ERR_DTYPE
    assert s(F=0) == blk.H3_ERR_ARG
    assert s(F=14336 - 16) == blk.H3_ERR_SHAPE                # F % 32
    assert s(ldh=14000) == blk.H3_ERR_ARG
    assert s(H=A + 64) == blk.H3_ERR_ARG                      # H overlaps A
    assert s(ldh=14340) == blk.H3_ERR_ALIGN
    assert s(M=0) == blk.H3_OK


def test_patchify_validation(lib):
    L = blk.load()
    lat, tok = P, P + (1 << 32)

    def pf(lat=lat, T=91, H=48, W=84, C=24, pt=1, ph=2, pw=2, tok=tok, ld=128, dt=0):
        return L.h3_patchify(lat, T, H, W, C, pt, ph, pw, tok, ld, dt, 0)

    def uf(lat=lat, T=91, H=48, W=84, C=24, pt=1, ph=2, pw=2, tok=tok, ld=128, dt=0):
        return L.h3_unpatchify(tok, ld, T, H, W, C, pt, ph, pw, lat, dt, 0)
    for f in (pf, uf):
        assert f(dt=5) == blk.H3_ERR_DTYPE
        assert f(lat=None) == blk.H3_ERR_ARG
        assert f(ph=0) == blk.H3_ERR_ARG
        assert f(H=47) == blk.H3_ERR_SHAPE                    # not a multiple of the patch
        assert f(C=20) == blk.H3_ERR_SHAPE                    # bf16 channels in 16-byte vectors
        assert f(ld=88) == blk.H3_ERR_ARG                     # row narrower than a patch (96)
        assert f(ld=100) == blk.H3_ERR_ALIGN
        assert f(tok=lat + 64) == blk.H3_ERR_ARG              # overlaps the latent
        assert f(T=0) == blk.H3_OK                            # nothing to do
    assert pf(C=20, dt=1, ld=80) != blk.H3_ERR_SHAPE          # fp32: 4-element vectors


def test_fp8_validation(lib):
    L = blk.load()
    x, q, s = P, P + (1 << 32), P + (2 << 32)

    def qz(x=x, ldx=5376, n=100, K=5376, q=q, ldq=5376, s=s, dt=0):
        return L.h3_quantize_fp8(x, ldx, n, K, q, ldq, s, dt, 0)
    assert qz(dt=4) == blk.H3_ERR_DTYPE
    assert qz(s=None) == blk.H3_ERR_ARG
    assert qz(ldq=100) == blk.H3_ERR_ARG
    assert qz(K=5370, ldx=5376) == blk.H3_ERR_SHAPE          # K a multiple of 16
    assert qz(ldq=5380) == blk.H3_ERR_ALIGN
    assert qz(q=x + 64) == blk.H3_ERR_ARG                    # q overlaps x
    assert qz(n=0) == blk.H3_OK
    A, W, C, sa, sw = P, P + (1 << 32), P + (2 << 32), P + (3 << 32), P + (4 << 32)

    def g(A=A, lda=5376, sa=sa, W=W, ldw=5376, sw=sw, C=C, ldc=21504, M=100, N=21504, K=5376, dt=0):
        return L.h3_gemm_fp8(A, lda, sa, W, ldw, sw, C, ldc, M, N, K, dt, 0)
    assert g(dt=3) == blk.H3_ERR_DTYPE
    assert g(sa=None) == blk.H3_ERR_ARG
    assert g(K=5376 - 64, lda=5376, ldw=5376) == blk.H3_ERR_SHAPE   # K a multiple of 128
    assert g(lda=5384) == blk.H3_ERR_ALIGN
    assert g(C=A + 64) == blk.H3_ERR_ARG
    assert g(M=0) == blk.H3_OK


def test_fp8_attention_validation(lib):
    L = blk.load()
    q, k, v = P, P + 256, P + 512
    q8, k8, vt, sq, sk, sv = (P + (i << 32) for i in range(1, 7))
    o = P + (7 << 32)

    def qz(q=q, k=k, v=v, ld=21504, n=1000, H=56, hd=128, q8=q8, k8=k8, vt=vt, n_pad=1024, sq=sq, sk=sk,
           sv=sv, dt=0):
        return L.h3_quantize_qkv_fp8(q, k, v, ld, n, H, hd, q8, k8, vt, n_pad, sq, sk, sv, dt, 0)
    assert qz(dt=1) == blk.H3_ERR_SHAPE                        # bf16 operands only
    assert qz(dt=4) == blk.H3_ERR_DTYPE
    assert qz(sv=None) == blk.H3_ERR_ARG
    assert qz(hd=64) == blk.H3_ERR_SHAPE
    assert qz(n_pad=960) == blk.H3_ERR_ARG                     # fewer columns than tokens
    assert qz(n_pad=1000) == blk.H3_ERR_ARG                    # not a multiple of 64
    assert qz(ld=7000) == blk.H3_ERR_ARG                       # row narrower than the heads
    assert qz(H=70000, ld=70000 * 128) == blk.H3_ERR_SHAPE      # grid limit on heads
    assert qz(q=q + 2) == blk.H3_ERR_ALIGN
    assert qz(k8=q8 + 64) == blk.H3_ERR_ARG                    # outputs overlap
    assert qz(sq=q + 64) == blk.H3_ERR_ARG                     # output overlaps an input
    assert qz(n=0) == blk.H3_OK

    def at(q8=q8, k8=k8, vt=vt, n_pad=1024, sq=sq, sk=sk, sv=sv, o=o, ld_o=7168, n=1000, H=56, hd=128,
           scale=128 ** -0.5):
        return L.h3_attention_fp8(q8, k8, vt, n_pad, sq, sk, sv, o, ld_o, n, H, hd, scale, 0)
    assert at(o=None) == blk.H3_ERR_ARG
    assert at(scale=0.0) == blk.H3_ERR_ARG
    assert at(scale=float("inf")) == blk.H3_ERR_ARG
    assert at(hd=64) == blk.H3_ERR_SHAPE
    assert at(n_pad=999) == blk.H3_ERR_ARG
    assert at(ld_o=7000) == blk.H3_ERR_ARG
    assert at(ld_o=7172) == blk.H3_ERR_ALIGN
    assert at(o=vt + 64) == blk.H3_ERR_ARG                     # output overlaps V^T
    assert at(n=0) == blk.H3_OK


def test_fp8_fused_projection_validation(lib):
    L = blk.load()
    A, W, x, out, sa, sw, mod = (P + (i << 32) for i in range(7))
    seg = blk.segments([inputs.Segment(start=0, length=100, mod_set=0, T=100, kind="audio")])

    def g(A=A, lda=7168, sa=sa, W=W, ldw=7168, sw=sw, x=x, out=out, ldo=5376, M=100, N=5376, K=7168, mod=mod,
          n_sets=1, br=0, segs=seg, n_segs=1):
        return L.h3_gemm_fp8_gate_residual(A, lda, sa, W, ldw, sw, x, out, ldo, M, N, K, mod, n_sets, br, segs, n_segs, 0)
    assert g(sa=None) == blk.H3_ERR_ARG
    assert g(K=7168 - 64) == blk.H3_ERR_SHAPE                  # K a multiple of 128
    assert g(br=5) == blk.H3_ERR_ARG
    assert g(x=A + 64) == blk.H3_ERR_ARG                       # x overlaps A
    assert g(out=x + 64) == blk.H3_ERR_ARG                     # out partially overlaps x
    assert g(x=out) != blk.H3_ERR_ARG                          # in place is allowed
    assert g(n_segs=0) == blk.H3_ERR_SEGMENTS                  # intervals must cover the rows

    def s(A=A, lda=5376, sa=sa, W=W, ldw=5376, sw=sw, H=out, ldh=14336, M=100, F=14336, K=5376):
        return L.h3_gemm_fp8_swiglu(A, lda, sa, W, ldw, sw, H, ldh, M, F, K, 0)
    assert s(sw=None) == blk.H3_ERR_ARG
    assert s(F=14336 + 16) == blk.H3_ERR_SHAPE                 # F a multiple of 32
    assert s(ldh=100) == blk.H3_ERR_ARG
    assert s(H=A + 64) == blk.H3_ERR_ARG                       # H overlaps A
    assert s(M=0) == blk.H3_OK
