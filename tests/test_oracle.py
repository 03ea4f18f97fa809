"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test is chosen so that a plausible slip in the oracle (a dropped term, a
wrong sign, a transposed operand, a wrong index, 127 vs 127**2, ">" vs ">=",
absmax over the wrong set, round-half-up) fails at least one of them.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests import _brute

INF = float("inf")


def f16(a):
    return np.asarray(a, dtype=np.float16)


# ---------------------------------------------------------------- Q itself

def test_worked_example_direct(golden_dir):
    """The explainer's scale/round example: 0.73 at scale 0.10 -> 7 -> 0.70."""
    g = json.load(open(os.path.join(golden_dir, "worked_example.json")))
    absmax = g["scale"] * oracle.QMAX          # scale = absmax / 127
    q = oracle.quantize(np.float32(g["original_value"]), np.float32(absmax))
    assert int(q) == g["stored_int8"]
    approx = oracle.dequantize(q, np.float32(absmax))
    assert abs(float(approx) - g["approximation"]) < 1e-6


def test_worked_example_through_row_quant(golden_dir):
    """Same example through the row quantizer: a row whose absmax is 12.7 has step 0.10."""
    g = json.load(open(os.path.join(golden_dir, "worked_example.json")))
    X = f16([[g["original_value"], g["scale"] * 127, 0.0, 0.0]])
    r = oracle.quant_rows(X, INF)
    assert r["count"] == 0
    assert r["Xq"].tolist() == [[g["stored_int8"], 127, 0, 0]]
    assert r["a_x"][0] == np.float32(np.float16(12.7))
    approx = oracle.dequantize(r["Xq"][0, 0], r["a_x"][0])
    assert abs(float(approx) - g["approximation"]) < 1e-3


def test_ties_round_half_even():
    """Reading R3: exact ties go to the even code (half-up would give 3, 4, -3)."""
    a = np.float32(127.0)
    assert oracle.quantize(np.float32(2.5), a) == 2
    assert oracle.quantize(np.float32(3.5), a) == 4
    assert oracle.quantize(np.float32(-2.5), a) == -2
    assert oracle.quantize(np.float32(0.5), a) == 0
    assert oracle.quantize(np.float32(126.5), a) == 126


def test_q_closed_forms():
    rng = np.random.default_rng(7)
    v = f16(rng.standard_normal(4096) * 3).astype(np.float32)
    a = np.float32(np.abs(v).max())
    q = oracle.quantize(v, a)
    # symmetric range, the absmax maps to +-127, odd symmetry
    assert q.min() >= -127 and q.max() <= 127
    assert oracle.quantize(a, a) == 127 and oracle.quantize(-a, a) == -127
    assert np.array_equal(oracle.quantize(-v, a), -q)
    # half-step bound: |v - q a/127| <= a/254
    err = np.abs(v.astype(np.float64) - oracle.dequantize(q, a))
    assert err.max() <= float(a) / 254 * (1 + 1e-12)
    # scale invariance by powers of two
    assert np.array_equal(oracle.quantize(v * 8, a * 8), q)
    assert np.array_equal(oracle.quantize(v / 4, a / 4), q)
    # zero constant gives zero codes
    assert np.all(oracle.quantize(np.zeros(5, np.float32), np.float32(0)) == 0)


def _exact_rne_codes(x16: np.ndarray, a16: np.float16) -> np.ndarray:
    """round-half-even(127 x / a) in exact int64 arithmetic (x, a scaled by 2**24)."""
    X = np.round(x16.astype(np.float64) * 2.0**24).astype(np.int64)
    A = int(round(float(a16) * 2.0**24))
    n = 127 * X
    q = n // A                      # floor
    r = n - q * A                   # 0 <= r < A
    up = (2 * r > A) | ((2 * r == A) & (q % 2 != 0))
    return q + up


def test_q_float32_route_equals_exact_rounding():
    """The fp32 decision equals exact rational rounding for every fp16 |v| <= a.

    All finite fp16 values v against a spread of fp16 constants a: powers of
    two, subnormals, multiples of 127 and random values.
    """
    allv = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16)   # +0 .. max finite
    allv = np.concatenate([allv, -allv[1:]])
    rng = np.random.default_rng(11)
    a_bits = np.unique(np.concatenate([
        rng.integers(1, 0x7C00, 600),                      # random finite positives
        np.arange(1, 40),                                   # subnormals
        np.array([np.float16(2.0**e).view(np.uint16) for e in range(-14, 16)]),
        np.array([np.float16(127 * 2.0**e).view(np.uint16) for e in range(-14, 9)]),
    ]).astype(np.uint16))
    checked = 0
    for ab in a_bits:
        a16 = np.uint16(ab).view(np.float16)
        v = allv[np.abs(allv.astype(np.float32)) <= np.float32(a16)]
        got = oracle.quantize(v.astype(np.float32), np.float32(a16)).astype(np.int64)
        want = _exact_rne_codes(v, a16)
        assert np.array_equal(got, want), f"a={float(a16)!r}"
        checked += v.size
    assert checked > 10_000_000


# ---------------------------------------------------------------- outliers

def test_threshold_tie_is_outlier():
    """Reading R1: |x| == t marks the column (">="); just below does not."""
    X = f16([[6.0, 5.99, -6.0, 1.0], [0.5, -5.99, 0.25, 2.0]])
    mask, idx = oracle.outlier_columns(X, 6.0)
    assert idx.tolist() == [0, 2]
    assert mask.tolist() == [True, False, True, False]


def test_column_exclusion_worked_case():
    """Reading R2: the row constant excludes whole outlier columns.

    Element-wise exclusion would give a_x[1] = 3 (the 3 sits in an outlier
    column but is below t); column exclusion gives 2.
    """
    X = f16([[10.0, 1.0], [3.0, 2.0]])
    r = oracle.quant_rows(X, 6.0)
    assert r["idx"].tolist() == [0]
    assert r["a_x"].tolist() == [1.0, 2.0]
    assert r["Xq"].tolist() == [[0, 127], [0, 127]]


def test_mask_words_bit_order():
    mask = np.zeros(70, dtype=bool)
    mask[[0, 31, 32, 69]] = True
    w = oracle.mask_words(mask)
    assert w.tolist() == [0x80000001, 0x00000001, 0x00000020]


def test_threshold_extremes():
    rng = np.random.default_rng(3)
    X = f16(rng.standard_normal((5, 48)) * 4)
    r = oracle.quant_rows(X, INF)
    assert r["count"] == 0
    assert np.all(np.abs(r["Xq"]).max(axis=1) == 127)      # every nonzero row hits 127
    r0 = oracle.quant_rows(X, 0.0)
    assert r0["count"] == 48 and np.all(r0["Xq"] == 0) and np.all(r0["a_x"] == 0)


def test_zero_and_all_outlier_rows():
    X = f16([[0.0, 0.0, 0.0], [0.0, 9.0, 0.0], [1.0, 7.0, -2.0]])
    r = oracle.quant_rows(X, 6.0)
    assert r["idx"].tolist() == [1]
    assert r["a_x"].tolist() == [0.0, 0.0, 2.0]
    assert r["Xq"].tolist() == [[0, 0, 0], [0, 0, 0], [64, 0, -127]]


# ---------------------------------------------------------------- brute force

def _brute_case(seed, M, K, N, t, adversarial=False):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, K)) * 2
    if adversarial:
        X[:, 0] = 6.0                              # threshold tie
        X[rng.integers(0, M), K - 1] = -20.0       # single-token outlier column
        X[0, :] = 0.0                              # all-zero row
        X[:, 1] = 0.5 * np.sign(X[:, 1] + 1e-9)    # equal magnitudes (ties in absmax)
    W = rng.standard_normal((K, N)) * 0.05
    if adversarial:
        W[:, 0] = 0.0                              # zero weight column
    return f16(X), f16(W), t


@pytest.mark.parametrize("seed,M,K,N,t,adv", [
    (1, 1, 16, 16, 6.0, False), (2, 3, 16, 32, 6.0, True), (3, 5, 32, 16, 6.0, True),
    (4, 4, 32, 32, 3.0, False), (5, 2, 16, 16, INF, False), (6, 3, 16, 16, 0.0, False),
    (7, 5, 32, 16, 2.5, True),
])
def test_oracle_matches_exact_brute_force(seed, M, K, N, t, adv):
    X, W, t = _brute_case(seed, M, K, N, t, adv)
    Wq, a_w = oracle.prepare_weight(W)
    got = oracle.mixed_matmul(X, Wq, a_w, t)
    b = _brute.mixed_matmul(X.astype(np.float64).tolist(), W.astype(np.float64).tolist(),
                            Fraction(float(np.float32(t))) if np.isfinite(t) else Fraction(10**9))
    assert Wq.tolist() == b["Wq"]
    assert [Fraction(float(v)) for v in a_w] == b["a_w"]
    assert got["idx"].tolist() == b["O"]
    assert [Fraction(float(v)) for v in got["a_x"]] == b["a_x"]
    assert got["Xq"].tolist() == b["Xq"]
    assert got["acc"].tolist() == b["acc"]
    # fp16 output: the oracle sums in float64 then rounds; exact rounding of
    # the exact sum may differ by at most one fp16 step (double rounding)
    Yb = np.array([[float(v) for v in row] for row in b["Y16"]], dtype=np.float16)
    ulps = np.abs(got["Y"].view(np.int16).astype(np.int32) - Yb.view(np.int16).astype(np.int32))
    same_sign = np.sign(got["Y"].astype(np.float32)) * np.sign(Yb.astype(np.float32)) >= 0
    assert np.all(same_sign | (np.abs(Yb.astype(np.float32)) < 1e-6))
    assert ulps.max() <= 1
    assert (ulps == 0).mean() > 0.9


# ---------------------------------------------------------------- invariants

def _grid_weight(rng, K, N):
    """W whose columns are exactly q * 2**-e with |q| <= 127 and some |q| == 127.

    Then the int8 conversion is lossless: dequantized Wq equals W exactly.
    """
    q = rng.integers(-127, 128, size=(K, N))
    q[rng.integers(0, K, size=N), np.arange(N)] = 127 * rng.choice([-1, 1], size=N)
    e = rng.integers(5, 9, size=N)
    return f16(q * 2.0 ** (-e[None, :].astype(np.float64)))


def test_zero_outlier_invariant_is_dequantized_int8_product():
    """t = +inf: Y is the int8 product with both operands dequantized (no outlier term)."""
    rng = np.random.default_rng(21)
    X = f16(rng.standard_normal((37, 80)) * 3)
    W = f16(rng.standard_normal((80, 48)) * 0.03)
    Wq, a_w = oracle.prepare_weight(W)
    r = oracle.mixed_matmul(X, Wq, a_w, INF)
    assert r["count"] == 0 and np.all(r["y_out"] == 0)
    Xhat = oracle.dequantize(r["Xq"], r["a_x"][:, None])       # [M, K]
    What = oracle.dequantize(Wq.T, a_w[None, :])               # [K, N]
    Yref = (Xhat @ What).astype(np.float16)
    d = np.abs(r["Y"].view(np.int16).astype(np.int32) - Yref.view(np.int16).astype(np.int32))
    assert d.max() <= 1 and (d == 0).mean() > 0.99


def test_all_outlier_invariant_is_fp16_matmul():
    """t = 0: every column is an outlier, so Y = fp16(X @ W^); with a lossless
    (grid-built) weight that is the textbook product fp16(X @ W)."""
    rng = np.random.default_rng(22)
    X = f16(rng.standard_normal((19, 64)) * 5)
    W = _grid_weight(rng, 64, 40)
    Wq, a_w = oracle.prepare_weight(W)
    assert np.array_equal(oracle.dequantize(Wq.T, a_w[None, :]), W.astype(np.float64))
    r = oracle.mixed_matmul(X, Wq, a_w, 0.0)
    assert r["count"] == 64 and np.all(r["acc"] == 0)
    Yref = (X.astype(np.float64) @ W.astype(np.float64)).astype(np.float16)
    d = np.abs(r["Y"].view(np.int16).astype(np.int32) - Yref.view(np.int16).astype(np.int32))
    assert d.max() <= 1 and (d == 0).mean() > 0.99


def test_decomposition_beats_plain_int8_on_outliers():
    """With planted outlier columns the decomposition is much closer to X @ W than
    plain vector-wise int8 (t = +inf) - the reason the method exists."""
    rng = np.random.default_rng(23)
    X = rng.standard_normal((64, 256))
    X[:, [5, 77]] = 40 * rng.choice([-1, 1], size=(64, 2))
    X = f16(X)
    W = f16(rng.standard_normal((256, 64)) * 0.02)
    Wq, a_w = oracle.prepare_weight(W)
    # against X @ W^ (the weight's own rounding is common to both variants)
    ref = X.astype(np.float64) @ oracle.dequantize(Wq.T, a_w[None, :])
    e_mix = np.abs(oracle.mixed_matmul(X, Wq, a_w, 6.0)["Y"] - ref).max()
    e_int8 = np.abs(oracle.mixed_matmul(X, Wq, a_w, INF)["Y"] - ref).max()
    assert e_mix * 10 < e_int8


def test_error_bound_against_exact_product():
    """|Y - X W| <= sum_{j not in O} (|x^_ij| a_w + |W_jn| a_x) / 254
                  + sum_{j in O} |X_ij| a_w / 254 + half an fp16 step of Y."""
    rng = np.random.default_rng(24)
    X = rng.standard_normal((48, 160)) * 2
    X[:, 9] = 30.0
    X = f16(X)
    W = f16(rng.standard_normal((160, 56)) * 0.02)
    Wq, a_w = oracle.prepare_weight(W)
    r = oracle.mixed_matmul(X, Wq, a_w, 6.0)
    Xd, Wd = X.astype(np.float64), W.astype(np.float64)
    keep = ~r["mask"]
    Xhat = oracle.dequantize(r["Xq"], r["a_x"][:, None])
    aw = a_w.astype(np.float64)[None, :]
    ax = r["a_x"].astype(np.float64)[:, None]
    bound = ((np.abs(Xhat) * keep) @ np.ones_like(Wd) * aw
             + (keep[:, None] * np.abs(Wd)).sum(0)[None, :] * ax
             + (np.abs(Xd) * r["mask"]) @ np.ones_like(Wd) * aw) / 254
    half_ulp = np.abs(r["Y"].astype(np.float64)) * 2.0**-11 + 2.0**-25
    assert np.all(np.abs(r["Y"] - Xd @ Wd) <= bound + half_ulp)


def test_sign_scaling_and_permutation_invariants():
    rng = np.random.default_rng(25)
    X = rng.standard_normal((20, 96)) * 2
    X[:, [3, 50]] = 20.0
    X = f16(X)
    W = f16(rng.standard_normal((96, 32)) * 0.02)
    Wq, a_w = oracle.prepare_weight(W)
    r = oracle.mixed_matmul(X, Wq, a_w, 6.0)
    # X -> -X
    rn = oracle.mixed_matmul(-X, Wq, a_w, 6.0)
    assert np.array_equal(rn["Xq"], -r["Xq"]) and np.array_equal(rn["acc"], -r["acc"])
    assert np.array_equal(rn["Y"], -r["Y"])
    # joint permutation of the K dimension
    p = rng.permutation(96)
    Wqp, a_wp = oracle.prepare_weight(W[p])
    rp = oracle.mixed_matmul(X[:, p], Wqp, a_wp, 6.0)
    assert np.array_equal(rp["acc"], r["acc"])
    assert np.array_equal(rp["Y"], r["Y"]) or np.abs(
        rp["Y"].astype(np.float64) - r["Y"]).max() <= 2.0**-10 * np.abs(r["Y"]).max()
    # power-of-two row scaling without outliers: codes unchanged, Y scales exactly
    r1 = oracle.mixed_matmul(X, Wq, a_w, INF)
    r2 = oracle.mixed_matmul(f16(X.astype(np.float32) / 4), Wq, a_w, INF)
    assert np.array_equal(r1["Xq"], r2["Xq"]) and np.array_equal(r1["acc"], r2["acc"])
    np.testing.assert_array_equal(r2["Y"], f16(r1["Y"].astype(np.float32) / 4))


def test_transposed_shapes_are_distinguished():
    """A non-square case where swapping operand roles would change the result."""
    rng = np.random.default_rng(26)
    X = f16(rng.standard_normal((3, 16)))
    W = f16(rng.standard_normal((16, 32)) * 0.1)
    Wq, a_w = oracle.prepare_weight(W)
    assert Wq.shape == (32, 16) and a_w.shape == (32,)
    b = _brute.mixed_matmul(X.astype(np.float64).tolist(), W.astype(np.float64).tolist(),
                            Fraction(6))
    assert oracle.mixed_matmul(X, Wq, a_w, 6.0)["acc"].tolist() == b["acc"]


def test_weight_memory_halves():
    """\"How much memory can it save?\": int8 storage is half of fp16 (plus N scales)."""
    W = f16(np.ones((64, 48)))
    Wq, a_w = oracle.prepare_weight(W)
    assert Wq.nbytes * 2 == W.nbytes and a_w.nbytes == 4 * 48


# ---------------------------------------------------------------- weight-only variant

@pytest.mark.parametrize("seed,M,K,N", [(11, 1, 16, 16), (12, 3, 32, 16), (13, 4, 16, 32)])
def test_weight_only_matches_exact_brute_force(seed, M, K, N):
    """fp16(X @ dequantized W) against the exact rational product rounded once."""
    X, W, _ = _brute_case(seed, M, K, N, 6.0, adversarial=True)
    Wq, a_w = oracle.prepare_weight(W)
    got = oracle.weight_only_matmul(X, Wq, a_w)
    b = _brute.weight_only_matmul(X.astype(np.float64).tolist(), W.astype(np.float64).tolist())
    Yb = np.array([[float(v) for v in row] for row in b], dtype=np.float16)
    ulps = np.abs(got.view(np.int16).astype(np.int32) - Yb.view(np.int16).astype(np.int32))
    assert ulps.max() <= 1 and (ulps == 0).mean() > 0.9


def test_weight_only_is_the_all_outlier_decomposition_and_differs_from_it_otherwise():
    """Every column an outlier (t = 0) leaves only the 16-bit product over dequantized
    weights, which is the weight-only product; with real outliers they differ."""
    rng = np.random.default_rng(21)
    X = f16(rng.standard_normal((6, 64)))
    X[:, 5] = 40.0
    Wq, a_w = oracle.prepare_weight(f16(rng.standard_normal((64, 48)) * 0.05))
    wo = oracle.weight_only_matmul(X, Wq, a_w)
    assert np.array_equal(wo, oracle.mixed_matmul(X, Wq, a_w, 0.0)["Y"])
    assert not np.array_equal(wo, oracle.mixed_matmul(X, Wq, a_w, 6.0)["Y"])
