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
