"""The FP8 quantisers take the quotient x / scale as the fp64 product
x * RN64(1 / scale) rounded to fp32.  Where the quotient lies in fp32's
normal range this is the correctly rounded fp32 quotient (x / s is never an
fp32 rounding midpoint and lies at least 2^-49 from every one, while the fp64
product is within 2^-52 of it), so the codes equal those of an fp32 division.
Below 2^-126 the subnormal grid is fixed and the two can differ by one step;
e4m3's smallest step is 2^-9, so both still encode to a signed zero.
Checked here against numpy's fp32 division on random and adversarial operand
pairs (CPU only)."""
import numpy as np

TINY = np.float32(2.0**-126)


def _fast(x, s):
    return (x.astype(np.float64) * (1.0 / s.astype(np.float64))).astype(np.float32)


def _check(x, s):
    """Equal where the quotient is fp32-normal (or overflows); below that,
    both below 2^-126 in magnitude with the same sign."""
    x = x.astype(np.float32)
    s = s.astype(np.float32)
    ok = np.isfinite(x) & np.isfinite(s) & (s != 0)
    x, s = x[ok], s[ok]
    with np.errstate(over="ignore", under="ignore"):
        ref = x / s
        got = _fast(x, s)
    normal = ~(np.abs(ref) < TINY)
    same = (ref == got) | (np.isnan(ref) & np.isnan(got))
    bad = normal & ~same
    assert not bad.any(), f"{x[bad][:4]} / {s[bad][:4]}: {ref[bad][:4]} != {got[bad][:4]}"
    sub = ~normal
    assert (np.abs(got[sub]) < TINY).all() and (np.signbit(got[sub]) == np.signbit(ref[sub])).all()
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


def test_quotient_subnormal_midpoints():
    """Quotients that are exact subnormal midpoints k * 2^-150 (k odd): the
    fast form may round them the other way, so the identity is stated for the
    normal range only; both results stay below 2^-126, under half of e4m3's
    smallest subnormal 2^-9, where every value encodes to a signed zero."""
    ms = np.arange(3, 1024, 2)
    k = np.arange(1, 512, 2)
    m, kk = np.meshgrid(ms, k)
    s = (m * 2.0**20).astype(np.float32).ravel()
    xv = (m * kk).astype(np.float64).ravel() * 2.0**-130
    x = xv.astype(np.float32)
    keep = x.astype(np.float64) == xv                 # representable operands only
    x, s = x[keep], s[keep]
    with np.errstate(under="ignore"):
        ref = x / s
        got = _fast(x, s)
    assert (ref != got).any()                         # the identity does fail here
    _check(x, s)
    _check(-x, s)
    assert float(np.abs(np.concatenate([ref, got])).max()) < 2.0**-10

