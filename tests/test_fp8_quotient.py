"""The FP8 quantisers take the quotient x / scale as the fp64 product
x * RN64(1 / scale) rounded to fp32.  For fp32 operands this is the correctly
rounded fp32 quotient (x / s is never an fp32 rounding midpoint and lies at
least 2^-49 from every one, while the fp64 product is within 2^-52 of it), so
the codes equal those of an fp32 division.  Checked here against numpy's fp32
division on random and adversarial operand pairs (CPU only)."""
import numpy as np


def _fast(x, s):
    return (x.astype(np.float64) * (1.0 / s.astype(np.float64))).astype(np.float32)


def _check(x, s):
    x = x.astype(np.float32)
    s = s.astype(np.float32)
    ok = np.isfinite(x) & np.isfinite(s) & (s != 0)
    x, s = x[ok], s[ok]
    with np.errstate(over="ignore", under="ignore"):
        ref = x / s
        got = _fast(x, s)
    same = (ref == got) | (np.isnan(ref) & np.isnan(got))
    assert same.all(), f"{x[~same][:4]} / {s[~same][:4]}: {ref[~same][:4]} != {got[~same][:4]}"
    return x.size


def test_quotient_random_bit_patterns():
    rng = np.random.default_rng(11)
    xb = rng.integers(0, 2**31, 1_000_000, dtype=np.uint64).astype(np.uint32)
    sb = rng.integers(0x30000000, 0x50000000, 1_000_000, dtype=np.uint64).astype(np.uint32)
    assert _check(xb.view(np.float32), sb.view(np.float32)) > 900_000


def test_quotient_quantiser_regime():
    rng = np.random.default_rng(12)
    mx = rng.uniform(1e-3, 1e3, 1_000_000).astype(np.float32)
    s = (mx / np.float32(448)).astype(np.float32)
    x = (rng.uniform(-1, 1, mx.size).astype(np.float32) * mx).astype(np.float32)
    _check(x, s)
    _check(mx, s)                                  # the row max itself: about 448


def test_quotient_adversarial_significands():
    rng = np.random.default_rng(13)
    n = 1_000_000
    e = np.float32(2.0) ** rng.integers(-30, 30, n).astype(np.float32)
    x = (rng.integers(1, 2**24, n).astype(np.float32) * e).astype(np.float32)
    s = ((2**24 - rng.integers(1, 64, n)).astype(np.float32) * e[::-1]).astype(np.float32)   # all bits set
    _check(x, s)
    _check(s, x)
    near1 = (np.float32(1.0) + rng.integers(0, 64, n).astype(np.float32) * np.float32(2.0**-23)).astype(np.float32)
    _check(x, near1)
    small = rng.integers(1, 1000, n).astype(np.float32)
    _check(small, rng.integers(1, 1000, n).astype(np.float32))
