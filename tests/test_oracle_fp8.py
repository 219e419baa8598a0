"""Pins of the oracle's OCP e4m3 format, its rounding, the row-wise
quantisation and the fp8 GEMM, plus the error bound the fp8 path is held to.

The pages give no FP8 format or bound (they only mention that the community
quantises to FP8); the format is OCP e4m3, pinned below by its defining
values (1.0 = 0x38, the largest finite 448 = 0x7E, the smallest subnormal
2^-9 = 0x01, the smallest normal 2^-6 = 0x08, NaN = 0x7F), monotonic codes,
exact round trips, ties to even and saturation.

Error bound (derived from the format): inside a binade the e4m3 step is
2^-3 of the binade's base, so rounding leaves a relative error of at most
2^-4 and, spread uniformly, an RMS of 2^-3 / sqrt(12) / 1.44 (the mean
mantissa), about 2.5 %, per quantised operand.  A product of two quantised
operands then carries about sqrt(2) * 2.5 % = 3.5 % per term, and with
random signs that ratio carries over to the sum.  The fp8 GEMM of N(0,1) rows
and N(0, 0.02^2) weights is held to 6e-2 in both metrics against the
unquantised fp64 product (measured 3.9e-2 max, 3.7e-2 Frobenius).
"""
import numpy as np
import pytest

import oracle
from fp8_layout import vt_key, vt_layout


def test_defining_values():
    d = oracle.e4m3_decode
    assert d(0x38) == 1.0 and d(0x40) == 2.0 and d(0x30) == 0.5
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0
    assert d(0x01) == 2.0 ** -9 and d(0x07) == 7 * 2.0 ** -9 and d(0x08) == 2.0 ** -6
    assert d(0x00) == 0.0 and np.signbit(d(0x80))
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    v = d(np.arange(0x7F))
    assert np.all(np.diff(v) > 0)                          # codes 0..0x7E increase
    assert np.isfinite(d(np.arange(256))).sum() == 254


def test_round_trip_of_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    back = oracle.e4m3_encode(oracle.e4m3_decode(codes))
    np.testing.assert_array_equal(back, codes)


def test_nearest_with_ties_to_even():
    v = oracle.e4m3_decode(np.arange(0x7F))
    mid = (v[:-1] + v[1:]) / 2
    want = np.where(np.arange(0x7E) % 2 == 0, np.arange(0x7E), np.arange(1, 0x7F))
    np.testing.assert_array_equal(oracle.e4m3_encode(mid), want)
    eps = 1e-6 * (v[1:] - v[:-1])
    np.testing.assert_array_equal(oracle.e4m3_encode(mid - eps), np.arange(0x7E))
    np.testing.assert_array_equal(oracle.e4m3_encode(mid + eps), np.arange(1, 0x7F))
    assert oracle.e4m3_encode(2.0 ** -10) == 0x00           # tie between 0 and 2^-9 -> even code 0
    assert oracle.e4m3_encode(3 * 2.0 ** -10) == 0x02       # tie between 0x01 and 0x02
    assert oracle.e4m3_encode(-1.0625) == 0xB8              # tie between 1 and 1.125 -> 1.0


def test_saturation_and_nan():
    np.testing.assert_array_equal(oracle.e4m3_encode([448.0, 460.0, 1e9, -500.0, np.inf]),
                                  [0x7E, 0x7E, 0x7E, 0xFE, 0x7E])
    assert oracle.e4m3_encode(np.nan) == 0x7F


def test_quantize_rows_scales_and_extremes():
    g = np.random.Generator(np.random.PCG64(11))
    x = g.standard_normal((5, 64)).astype(np.float32)
    x[3] = 0.0
    q, s = oracle.quantize_rows(x)
    assert s.dtype == np.float32 and s[3] == 1.0 and np.all(q[3] == 0)
    for i in (0, 1, 2, 4):
        k = int(np.argmax(np.abs(x[i])))
        assert q[i, k] & 0x7F == 0x7E                       # the row maximum lands on 448
        assert s[i] == np.float32(np.max(np.abs(x[i]))) / np.float32(448.0)
    rel = np.abs(oracle.e4m3_decode(q) * s[:, None] - x)
    big = np.abs(x) >= 2.0 ** -6 * s[:, None]
    assert np.all(rel[big] <= 2.0 ** -4 * np.abs(x[big]) + 1e-12)
    assert np.all(rel[~big] <= 2.0 ** -10 * np.broadcast_to(s[:, None], x.shape)[~big] + 1e-12)


def test_gemm_fp8_brute_force():
    g = np.random.Generator(np.random.PCG64(12))
    qa = g.integers(0, 256, size=(3, 16)).astype(np.uint8)
    qw = g.integers(0, 256, size=(4, 16)).astype(np.uint8)
    qa[qa & 0x7F == 0x7F] = 0
    qw[qw & 0x7F == 0x7F] = 0
    sa, sw = g.random(3) + 0.5, g.random(4) + 0.5
    c = oracle.gemm_fp8(qa, sa, qw, sw)
    for i in range(3):
        for j in range(4):
            ref = sum(oracle.e4m3_decode(qa[i, k]) * oracle.e4m3_decode(qw[j, k]) for k in range(16)) * sa[i] * sw[j]
            assert c[i, j] == pytest.approx(ref, rel=1e-12, abs=1e-300)


def test_quantisation_error_bound():
    g = np.random.Generator(np.random.PCG64(13))
    a = g.standard_normal((64, 512)).astype(np.float32)
    w = (g.standard_normal((96, 512)) * 0.02).astype(np.float32)
    qa, sa = oracle.quantize_rows(a)
    qw, sw = oracle.quantize_rows(w)
    got = oracle.gemm_fp8(qa, sa, qw, sw)
    ref = oracle.linear(a.astype(np.float64), w.astype(np.float64))
    e_max = np.abs(got - ref).max() / np.abs(ref).max()
    e_f = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert e_f <= 6e-2 and e_max <= 6e-2, (e_max, e_f)
    assert e_f >= 1e-2                                      # the operands really were quantised


# ------------------------------------------------------------------ attention

def test_qkv_quantisation_reduces_to_rows():
    """Per (token, head) q scales are the row quantiser on each head's slice;
    k and v take one scale per head over all tokens."""
    g = np.random.Generator(np.random.PCG64(21))
    n, H, d = 9, 3, 16
    q, k, v = (g.standard_normal((n, H * d)).astype(np.float32) * (1 + i) for i in range(3))
    q8, sq, k8, sk, v8, sv = oracle.quantize_qkv(q, k, v, H, d)
    assert sq.shape == (H, n) and sk.shape == (H,)
    for h in range(H):
        qr, sr = oracle.quantize_rows(q[:, h * d:(h + 1) * d])
        np.testing.assert_array_equal(q8[:, h * d:(h + 1) * d], qr)
        np.testing.assert_array_equal(sq[h], sr)
        assert sk[h] == np.float32(np.abs(k[:, h * d:(h + 1) * d]).max()) / np.float32(448)
        assert np.max(v8[:, h * d:(h + 1) * d] & 0x7F) == 0x7E        # the head maximum lands on 448


def test_vt_key_is_a_permutation_and_layout_inverts():
    keys = vt_key(np.arange(64))
    assert sorted(keys.tolist()) == list(range(64))
    assert keys[:4].tolist() == [0, 1, 2, 3] and keys[4:8].tolist() == [8, 9, 10, 11]
    assert keys[16:20].tolist() == [32, 33, 34, 35] and keys[32:36].tolist() == [4, 5, 6, 7]
    g = np.random.Generator(np.random.PCG64(22))
    n, H, d, n_pad = 100, 2, 8, 128
    v8 = g.integers(0, 0x7F, size=(n, H * d)).astype(np.uint8)
    vt = vt_layout(v8, H, d, n_pad)
    assert vt.shape == (H, d, n_pad)
    for p in (0, 5, 37, 63, 64, 99):
        key = (p // 64) * 64 + int(vt_key(p % 64))
        want = v8[key].reshape(H, d) if key < n else np.zeros((H, d), np.uint8)
        np.testing.assert_array_equal(vt[:, :, p], want)


def test_fp8_attention_reference_on_exact_codes():
    """Operands built to be exact in the quantised form: every slice that
    shares a scale (a token's head for q, a whole head for k and v) holds
    +-448 * 2^e once and otherwise e4m3 values times 2^e, so its scale is
    exactly 2^e and every quotient is an e4m3 value.  The codes then
    dequantise to exactly the operands, with distinct exponents for q, k and
    v (so swapped k and v scales would fail), and the reference attention of
    the dequantised operands is the attention of the operands themselves."""
    g = np.random.Generator(np.random.PCG64(23))
    n, H, d = 40, 2, 8
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    exps = {"q": -3, "k": -1, "v": 2}
    ops = {}
    for name, e in exps.items():
        x = oracle.e4m3_decode(g.choice(finite, size=(n, H * d))).astype(np.float64) * 2.0 ** e
        x = x.reshape(n, H, d)
        if name == "q":
            x[np.arange(n), :, g.integers(0, d, size=n)] = 448 * 2.0 ** e     # every (token, head)
        else:
            for h in range(H):
                x[g.integers(0, n), h, g.integers(0, d)] = -448 * 2.0 ** e    # once per head
        ops[name] = x.reshape(n, H * d).astype(np.float32)
        assert np.array_equal(ops[name].astype(np.float64), x.reshape(n, H * d))   # fp32 holds them
    q8, sq, k8, sk, v8, sv = oracle.quantize_qkv(ops["q"], ops["k"], ops["v"], H, d)
    assert np.all(sq == np.float32(2.0 ** exps["q"]))
    assert np.all(sk == np.float32(2.0 ** exps["k"])) and np.all(sv == np.float32(2.0 ** exps["v"]))
    qd, kd, vd = oracle.dequantize_qkv(q8, sq, k8, sk, v8, sv, H, d)
    for got, want in ((qd, ops["q"]), (kd, ops["k"]), (vd, ops["v"])):
        np.testing.assert_array_equal(got, want.astype(np.float64))
    ref = oracle.attention(*(ops[k].astype(np.float64) for k in "qkv"), H, d, d ** -0.5)
    np.testing.assert_array_equal(oracle.attention(qd, kd, vd, H, d, d ** -0.5), ref)


def test_fp8_attention_quantisation_error_bound():
    """Quantising q, k, v moves the attention output o = sum_j p_j v_j /
    sum_j p_j by two terms of relative size r (the RMS relative rounding of
    one e4m3 value, about 2.5 %): sum_j p_j dv_j / sum p, and from the logit
    error ds_j (RMS sqrt(2) r at logits of RMS 1) sum_j p_j ds_j (v_j - o) /
    sum p.  Both scale like o itself, so |do| / |o| in the Frobenius norm is
    about sqrt(3) r = 4.3 %, held to 6e-2.  The largest single error is
    compared with max |v| (o averages many v and is much smaller): a
    per-element bound of 2^-4 of the range of v."""
    g = np.random.Generator(np.random.PCG64(24))
    n, H, d = 300, 2, 128
    q, k, v = (g.standard_normal((n, H * d)).astype(np.float32) for _ in range(3))
    ref = oracle.attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), H, d, d ** -0.5)
    dq = oracle.dequantize_qkv(*oracle.quantize_qkv(q, k, v, H, d), H, d)
    got = oracle.attention(*dq, H, d, d ** -0.5)
    e_v = np.abs(got - ref).max() / np.abs(v).max()
    e_f = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert e_f <= 6e-2 and e_v <= 2.0 ** -4, (e_f, e_v)
    # a mistake of the kind the GPU layout could make (one 64-key group's
    # values permuted) is far outside that bound
    v_bad = np.array(v)
    v_bad[:64] = v_bad[vt_key(np.arange(64))]
    bad = oracle.attention(*dq[:2], oracle.dequantize_qkv(*oracle.quantize_qkv(q, k, v_bad, H, d), H, d)[2],
                           H, d, d ** -0.5)
    assert np.linalg.norm(bad - ref) / np.linalg.norm(ref) > 0.15
