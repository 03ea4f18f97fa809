"""Host model of the kernels' fast int8 code decision, checked for exactness.

The kernels decide q = round-half-even(127 x / a) per element without a divide:
with r = RN32(127 / a) computed once per row, t = RN32(x * r) and q0 = rint(t),
q0 is accepted when |t - q0| <= 0.5 - 2^-15; otherwise (a near-tie) the exact
IEEE divide decides. Since |t - 127 x / a| <= 127 * 2^-23 < 2^-16, an accepted
q0 is always the exact rounding. This test emulates that arithmetic with
numpy's IEEE float32 operations for every finite fp16 x against a spread of
fp16 constants a and compares the accepted codes with exact integer rounding.
"""

import numpy as np

NEAR = np.float32(0.5 - 2.0**-15)


def exact_codes(x16, a16):
    X = np.round(x16.astype(np.float64) * 2.0**24).astype(np.int64)
    A = int(round(float(a16) * 2.0**24))
    n = 127 * X
    q = n // A
    r = n - q * A
    return q + ((2 * r > A) | ((2 * r == A) & (q % 2 != 0)))


def test_fast_path_is_exact_when_accepted():
    allv = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16)
    allv = np.concatenate([allv, -allv[1:]])
    rng = np.random.default_rng(17)
    a_bits = np.unique(np.concatenate([
        rng.integers(1, 0x7C00, 800), np.arange(1, 64),
        np.array([np.float16(2.0**e).view(np.uint16) for e in range(-14, 16)]),
        np.array([np.float16(127 * 2.0**e).view(np.uint16) for e in range(-14, 9)]),
        np.array([np.float16(v).view(np.uint16) for v in (12.7, 6.0, 5.99609375, 65504.0)]),
    ]).astype(np.uint16))
    accepted = fallback = 0
    for ab in a_bits:
        a16 = np.uint16(ab).view(np.float16)
        a32 = np.float32(a16)
        v = allv[np.abs(allv.astype(np.float32)) <= a32]
        r = np.float32(127.0) / a32                      # IEEE float32 divide, once per row
        t = v.astype(np.float32) * r                     # IEEE float32 multiply
        q0 = np.rint(t)
        ok = np.abs(t - q0) <= NEAR
        want = exact_codes(v, a16)
        assert np.array_equal(q0[ok].astype(np.int64), want[ok]), f"a={float(a16)!r}"
        assert np.all(np.abs(q0.astype(np.int64) - want) <= 1)
        accepted += int(ok.sum())
        fallback += int((~ok).sum())
    assert accepted > 20_000_000
    # near-ties are rare: the exact fallback runs for a tiny fraction of codes
    assert fallback < accepted * 2e-3


MAGIC = 12582912.0  # fp32 1.5 * 2^23


def fma32(a, b, c):
    """fp32 fused multiply-add: the float64 value of a*b + c is exact for every use
    below (products of at most 24 + 11 bits plus a term of the same scale), so one
    rounding to float32 gives the fused result."""
    return (np.asarray(a, np.float64) * np.asarray(b, np.float64)
            + np.asarray(c, np.float64)).astype(np.float32)


def bracket_model(v16, a16):
    """Emulates quant8_fast and quant8_exact of the kernels: returns the
    lower-bracket codes, a flag per element where the pair disagrees, and the
    exact-path codes for every element."""
    a32 = np.float32(a16)
    r = np.float32(127.0) / a32
    lo = np.nextafter(r, np.float32(0))
    hi = np.nextafter(r, np.float32(np.inf))
    x = v16.astype(np.float32)
    t1 = fma32(x, lo, MAGIC)
    t2 = fma32(x, hi, MAGIC)
    q_lo = (t1.astype(np.float64) - MAGIC).astype(np.int64)
    q_hi = (t2.astype(np.float64) - MAGIC).astype(np.int64)
    # exact path
    w = np.abs(x)
    q1 = (fma32(w, lo, MAGIC) - np.float32(MAGIC)).astype(np.float32)
    d = fma32(np.float32(2.0) * q1 + np.float32(1.0), a32, -np.float32(254.0) * w)
    qi = q1.astype(np.int64)
    q = qi + ((d < 0) | ((d == 0) & (qi % 2 == 1)))
    q_exact = np.where(x < 0, -q, q)
    return q_lo, q_lo != q_hi, q_exact


def test_bracket_and_exact_paths():
    """Where the bracketing pair agrees its code is exact; the division-free exact
    path is exact everywhere (ties included: a = 127 * 2^e puts ties on a lattice)."""
    allv = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16)
    allv = np.concatenate([allv, -allv[1:]])
    rng = np.random.default_rng(23)
    a_bits = np.unique(np.concatenate([
        rng.integers(1, 0x7C00, 300), np.arange(1, 40),
        np.array([np.float16(2.0**e).view(np.uint16) for e in range(-14, 16)]),
        np.array([np.float16(k * 127 * 2.0**e).view(np.uint16)
                  for e in range(-14, 6) for k in (1, 3, 5, 15)]),
        np.array([np.float16(v).view(np.uint16) for v in (3.45703, 3.39648, 6.0, 65504.0)]),
    ]).astype(np.uint16))
    agree = disagree = 0
    for ab in a_bits:
        a16 = np.uint16(ab).view(np.float16)
        if not np.isfinite(a16) or float(a16) == 0.0:
            continue
        v = allv[np.abs(allv.astype(np.float32)) <= np.float32(a16)]
        want = exact_codes(v, a16)
        q_lo, dis, q_exact = bracket_model(v, a16)
        assert np.array_equal(q_lo[~dis], want[~dis]), f"a={float(a16)!r}"
        assert np.array_equal(q_exact, want), f"a={float(a16)!r}"
        agree += int((~dis).sum())
        disagree += int(dis.sum())
    assert agree > 5_000_000 and disagree > 0


def test_bracket_zero_constant():
    """A row whose kept values are all zero has a = 0: both brackets are 0 and every
    code is 0 (the kernels special-case the reciprocal)."""
    x = np.zeros(8, np.float32)
    t = fma32(x, np.float32(0), MAGIC)
    assert np.all(t == np.float32(MAGIC))
    d = fma32(np.float32(1.0), np.float32(0.0), -np.float32(254.0) * x)
    assert np.all(d == 0)
