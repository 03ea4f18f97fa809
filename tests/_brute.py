"""Exact brute force for tiny shapes: pure Python, rational arithmetic.

A second, independent route to every quantity of the method, used only to pin
the numpy oracle. Every value is an exact ``Fraction``; integer codes come
from exact round-half-to-even of the rational quotient; the fp16 output is the
exact rational result rounded once to the nearest fp16 (ties to even). It uses
loops and ``fractions`` only: no numpy, no float division.
"""

from __future__ import annotations

import math
from fractions import Fraction

QMAX = 127


def rne(x: Fraction) -> int:
    """Round a rational to the nearest integer, ties to even."""
    fl = math.floor(x)
    rem = x - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def q_exact(v: Fraction, a: Fraction) -> int:
    return 0 if a == 0 else rne(QMAX * v / a)


def to_fp16(y: Fraction) -> Fraction:
    """Exact value of the fp16 nearest to y (ties to even; +-inf as None)."""
    if y == 0:
        return Fraction(0)
    s = -1 if y < 0 else 1
    m = abs(y)
    e = m.numerator.bit_length() - m.denominator.bit_length()
    if Fraction(2) ** e > m:
        e -= 1
    while Fraction(2) ** (e + 1) <= m:
        e += 1
    e = max(e, -14)                      # subnormal range shares the 2^-24 step
    ulp = Fraction(2) ** (e - 10)
    r = rne(m / ulp) * ulp
    if r >= 65520:                       # rounds to infinity
        return None
    return s * r


def mixed_matmul(X, W, t):
    """X: list of rows (M x K) of exact values; W: K x N. Returns a dict."""
    M, K, N = len(X), len(W), len(W[0])
    X = [[Fraction(v) for v in row] for row in X]
    W = [[Fraction(v) for v in row] for row in W]
    t = Fraction(t)
    a_w = [max(abs(W[k][n]) for k in range(K)) for n in range(N)]
    Wq = [[q_exact(W[k][n], a_w[n]) for k in range(K)] for n in range(N)]
    O = [j for j in range(K) if any(abs(X[i][j]) >= t for i in range(M))]
    Oset = set(O)
    a_x = [max([abs(X[i][j]) for j in range(K) if j not in Oset], default=Fraction(0))
           for i in range(M)]
    Xq = [[0 if j in Oset else q_exact(X[i][j], a_x[i]) for j in range(K)] for i in range(M)]
    acc = [[sum(Xq[i][k] * Wq[n][k] for k in range(K)) for n in range(N)] for i in range(M)]
    Yex = [[Fraction(acc[i][n]) * a_x[i] * a_w[n] / (QMAX * QMAX)
            + sum(X[i][j] * Wq[n][j] * a_w[n] / QMAX for j in O)
            for n in range(N)] for i in range(M)]
    Y16 = [[to_fp16(y) for y in row] for row in Yex]
    return dict(a_w=a_w, Wq=Wq, O=O, a_x=a_x, Xq=Xq, acc=acc, Yexact=Yex, Y16=Y16)


def weight_only_matmul(X, W):
    """Weight-only int8 product: exact X times the dequantized int8 weight, rounded
    to fp16 once. Returns the list of rows of exact fp16 values."""
    K, N = len(W), len(W[0])
    X = [[Fraction(v) for v in row] for row in X]
    W = [[Fraction(v) for v in row] for row in W]
    a_w = [max(abs(W[k][n]) for k in range(K)) for n in range(N)]
    What = [[Fraction(q_exact(W[k][n], a_w[n])) * a_w[n] / QMAX for n in range(N)]
            for k in range(K)]
    return [[to_fp16(sum(row[k] * What[k][n] for k in range(K))) for n in range(N)] for row in X]


def tensorwise(X, W):
    """One absmax constant for all of X and one for all of W; exact rational result
    and its fp16 rounding: (Yexact, Y16)."""
    M, K, N = len(X), len(W), len(W[0])
    X = [[Fraction(v) for v in row] for row in X]
    W = [[Fraction(v) for v in row] for row in W]
    ax = max(abs(v) for row in X for v in row)
    aw = max(abs(v) for row in W for v in row)
    Xq = [[q_exact(v, ax) for v in row] for row in X]
    Wq = [[q_exact(v, aw) for v in row] for row in W]
    Yex = [[Fraction(sum(Xq[i][k] * Wq[k][n] for k in range(K))) * ax * aw / (QMAX * QMAX)
            for n in range(N)] for i in range(M)]
    return Yex, [[to_fp16(y) for y in row] for row in Yex]


def groupwise(X, W, group):
    """Constants per row of X and per column of W within each group of `group`
    consecutive K entries (the last group may be shorter); exact rational result and
    its fp16 rounding: (Yexact, Y16)."""
    M, K, N = len(X), len(W), len(W[0])
    X = [[Fraction(v) for v in row] for row in X]
    W = [[Fraction(v) for v in row] for row in W]
    Yex = [[Fraction(0)] * N for _ in range(M)]
    for g0 in range(0, K, group):
        ks = range(g0, min(K, g0 + group))
        ax = [max(abs(X[i][k]) for k in ks) for i in range(M)]
        aw = [max(abs(W[k][n]) for k in ks) for n in range(N)]
        for i in range(M):
            for n in range(N):
                acc = sum(q_exact(X[i][k], ax[i]) * q_exact(W[k][n], aw[n]) for k in ks)
                Yex[i][n] += Fraction(acc) * ax[i] * aw[n] / (QMAX * QMAX)
    return Yex, [[to_fp16(y) for y in row] for row in Yex]
