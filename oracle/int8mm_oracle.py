"""CPU oracle for the LLM.int8() mixed-precision decomposed matrix multiply.

TEST INFRASTRUCTURE. Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import or call this module. The product path
(the HIP library and its Python binding) never does, and shares no code with
it: not a kernel, a helper, a constant table or any pre/post-processing.

Plain and slow on purpose: numpy, whole-matrix operations, float64 wherever a
floating-point value is formed (the int8 code decision excepted, see
``quantize``). No blocking, fusion or reordering beyond what the method states.

Sources (web pages on the method; cited by title and section):
  [Abstract]   "LLM.int8(): 8-bit Matrix Multiplication for Transformers at
               Scale" (mlsanity.com paper index), section "Abstract (arXiv)".
  [Summary]    "8-bit Matrix Multiplication for Large Language Models"
               (legiblepapers.com), "Summary & Methodology Analysis".
  [Blog]       "Compress your LLMs" (samsena.com), the bullets
               "Vector-wise quantization" and "Mixed-precision decomposition".
  [Explainer]  "What is 8-bit LLM quantization?" (machinoai.in), section
               "How does INT8 quantization work?".

Notation. X: fp16 activations [M, K] (rows = tokens, columns = feature
dimensions). W: fp16 weights [K, N] (columns = output features). Wq: int8
weights stored [N, K]. a_x: fp32 [M] row absmax. a_w: fp32 [N] column absmax.
O: ascending list of outlier feature columns. t: outlier threshold.

Readings taken where the pages leave a step open (each one has a test):
  R1  outlier rule: column j is an outlier iff some row has |X[i, j]| >= t
      (">=" rather than ">"; per call, over all rows of this X).
  R2  the row constant a_x[i] is the absmax over the non-outlier columns only.
  R3  codes are symmetric in [-127, 127]: Q(v, a) = round-half-even(127 v / a);
      Q = 0 when a = 0. Dequantization is q * a / 127.
  R4  the weight constant a_w[n] is the absmax of column n over all K rows.
  R5  the outlier (16-bit) product uses the weight rows dequantized from int8,
      so only Wq and a_w are kept (halved weight memory).
  R6  int8 products accumulate exactly (int32); the fp16 output is rounded once.
"""

from __future__ import annotations

import numpy as np

QMAX = 127  # largest int8 code of the symmetric range (reading R3)


def _as_f64(a) -> np.ndarray:
    return np.asarray(a).astype(np.float64)


def quantize(v, a) -> np.ndarray:
    """Q(v, a): int8 code of value v under absmax constant a (broadcasting).

    The explainer's scale/round primitive ([Explainer]: a value is stored as
    the rounded quotient by its scale and approximated by code times scale),
    with the scale being a/127 for an absmax constant a (reading R3) and the
    rounding taken half-to-even (the pages print no tie rule).

    The code decision is made in float32: 127*v is exact in float32 for fp16 v
    (11-bit significand times a 7-bit integer), the quotient is the IEEE
    correctly-rounded float32 division, and rint rounds half to even. For
    |v| <= a this equals round-half-even of the exact rational 127 v / a; the
    test suite checks that against exact integer arithmetic.
    """
    v32 = np.asarray(v, dtype=np.float32)
    a32 = np.asarray(a, dtype=np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.rint((np.float32(QMAX) * v32) / a32)
    q = np.where(a32 == 0, np.float32(0), q)
    return q.astype(np.int8)


def dequantize(q, a) -> np.ndarray:
    """q * a / 127 in float64 ([Explainer]: approximation = code times scale)."""
    return _as_f64(q) * _as_f64(a) / QMAX


def prepare_weight(W: np.ndarray):
    """Convert an fp16 weight [K, N] to int8 with one constant per output column.

    [Abstract]: a 16/32-bit checkpoint is converted to Int8 when loaded.
    [Blog] "Vector-wise quantization": each column of the weight matrix gets
    its own scaling constant. Reading R4: the absmax spans all K rows.
    Returns (Wq int8 [N, K], a_w float32 [N]).
    """
    W = np.asarray(W)
    assert W.dtype == np.float16 and W.ndim == 2
    Wd = _as_f64(W)
    assert np.all(np.isfinite(Wd)), "finite inputs only"
    a_w = np.abs(Wd).max(axis=0).astype(np.float32)  # exact: an fp16 magnitude
    Wq = quantize(W.T, a_w[:, None])
    return np.ascontiguousarray(Wq), a_w


def outlier_columns(X: np.ndarray, t: float):
    """Outlier feature dimensions of X (reading R1).

    [Abstract] / [Summary]: the emergent outlier feature dimensions are
    isolated into a 16-bit product. A column is an outlier when any of its
    entries reaches the magnitude threshold t.
    Returns (bool mask [K], ascending int32 index list).
    """
    Xd = _as_f64(X)
    mask = (np.abs(Xd) >= np.float64(np.float32(t))).any(axis=0)
    idx = np.flatnonzero(mask).astype(np.int32)
    return mask, idx


def mask_words(mask: np.ndarray) -> np.ndarray:
    """Pack a bool column mask into uint32 words, bit j%32 of word j//32."""
    K = mask.shape[0]
    nw = (K + 31) // 32
    words = np.zeros(nw, dtype=np.uint64)
    for j in np.flatnonzero(mask):
        words[j // 32] |= np.uint64(1) << np.uint64(j % 32)
    return words.astype(np.uint32)


def quant_rows(X: np.ndarray, t: float):
    """Outlier detection and vector-wise row quantization of the activations.

    [Blog] "Vector-wise quantization": one constant per row of the input.
    [Blog] "Mixed-precision decomposition": the 8-bit product covers the
    non-outlier dimensions, so the row constant is the absmax over those
    columns (reading R2) and outlier columns get code 0 in Xq.
    Returns dict(mask, idx, count, a_x float32 [M], Xq int8 [M, K]).
    """
    X = np.asarray(X)
    assert X.dtype == np.float16 and X.ndim == 2
    Xd = _as_f64(X)
    assert np.all(np.isfinite(Xd)), "finite inputs only"
    mask, idx = outlier_columns(X, t)
    keep = ~mask
    absx = np.abs(Xd) * keep[None, :]
    a_x = (absx.max(axis=1) if X.shape[1] else np.zeros(X.shape[0])).astype(np.float32)
    Xq = quantize(X, a_x[:, None])
    Xq[:, mask] = 0
    return {"mask": mask, "idx": idx, "count": int(idx.size), "a_x": a_x, "Xq": Xq}


def int8_matmul(Xq: np.ndarray, Wq: np.ndarray) -> np.ndarray:
    """acc[i, n] = sum_k Xq[i, k] * Wq[n, k], exactly, as int32.

    [Abstract] / [Blog]: the non-outlier part is an 8-bit matrix
    multiplication (reading R6: exact integer accumulation). A float64 BLAS
    product of integer-valued operands is exact here because every partial
    sum is an integer below K * 127**2 < 2**53.
    """
    K = Xq.shape[1]
    assert Wq.shape[1] == K and K * QMAX * QMAX < 2**31
    acc = _as_f64(Xq) @ _as_f64(Wq).T
    return acc.astype(np.int64).astype(np.int32)


def dequant_outer(acc: np.ndarray, a_x: np.ndarray, a_w: np.ndarray) -> np.ndarray:
    """Dequantize the int8 product by the outer product of row and column constants.

    [Summary]: the 8-bit outputs are dequantized with the outer product of the
    row and column normalization constants. Each constant carries a step of
    a/127, hence the 127**2.
    """
    return _as_f64(acc) * np.outer(_as_f64(a_x), _as_f64(a_w)) / (QMAX * QMAX)


def outlier_matmul(X: np.ndarray, idx: np.ndarray, Wq: np.ndarray, a_w: np.ndarray):
    """The 16-bit product over the outlier columns only.

    [Blog] "Mixed-precision decomposition" / [Abstract]: the outlier feature
    dimensions go through a 16-bit matrix multiplication. Reading R5: their
    weight rows are the int8 weight dequantized, W^[j, n] = Wq[n, j] a_w[n] / 127.
    """
    Xo = _as_f64(X)[:, idx]                                  # [M, |O|]
    What = dequantize(Wq[:, idx].T, a_w[None, :])            # [|O|, N]
    return Xo @ What


def mixed_matmul(X: np.ndarray, Wq: np.ndarray, a_w: np.ndarray, t: float) -> dict:
    """The whole decomposed product, returning Y and every intermediate.

    [Summary]: the results of the regular (8-bit, dequantized) and outlier
    (16-bit) products are accumulated into 16-bit floating-point outputs.
    Reading R6: summed in float64 and rounded to fp16 once.
    """
    q = quant_rows(X, t)
    acc = int8_matmul(q["Xq"], Wq)
    y_int8 = dequant_outer(acc, q["a_x"], a_w)
    y_out = outlier_matmul(X, q["idx"], Wq, a_w)
    Y = (y_int8 + y_out).astype(np.float16)
    return dict(q, acc=acc, Y=Y, y_int8=y_int8, y_out=y_out)


def weight_only_matmul(X: np.ndarray, Wq: np.ndarray, a_w: np.ndarray) -> np.ndarray:
    """Weight-only int8: Y = fp16(X @ W^) with W^[k, n] = Wq[n, k] a_w[n] / 127.

    [Explainer] "What is special about LLM.int8()?": 8-bit weights can be paired
    with activations and arithmetic that stay in 16 bit. Here only the weight is
    quantized; the fp16 activations multiply the dequantized weight in float64 and
    the result is rounded to fp16 once. (No outlier decomposition: the same sum as
    the outlier product of ``outlier_matmul`` taken over every column.)
    """
    What = dequantize(Wq.T, a_w[None, :])                    # [K, N]
    return (_as_f64(X) @ What).astype(np.float16)
