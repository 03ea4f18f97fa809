"""Accuracy ablation of the decomposition, on the CPU (test infrastructure only).

What the mixed-precision decomposition buys, measured against the exact product
X @ W (float64) on synthetic activations with outlier feature columns:

  tensor-wise   one absmax constant for all of X and one for all of W
                ("Compress your LLMs", Vector-wise quantization, contrasts
                per-vector constants with one constant per tensor);
  group-wise    one constant per group of G consecutive K entries, for each row
                of X and each column of W ("What is 8-bit LLM quantization?",
                How does INT8 quantization work?: finer-grained constants, per
                group or per vector, lower the rounding error of one global one);
  vector-wise   one constant per row of X and per column of W, no decomposition
                (the method with threshold +inf);
  decomposed    vector-wise plus the 16-bit product over the outlier columns
                (the method, threshold t; "LLM.int8(): 8-bit Matrix
                Multiplication for Transformers at Scale", Abstract).

All four use the same symmetric round-half-even int8 code as the oracle. Run as a
script to print the table for the benchmark workloads (row x column samples):

    python -m oracle.ablation
"""

from __future__ import annotations

import numpy as np

from .int8mm_oracle import QMAX, mixed_matmul, prepare_weight, quantize


def exact_product(X: np.ndarray, W: np.ndarray) -> np.ndarray:
    """X @ W in float64 from the fp16 inputs (the unquantized reference)."""
    return X.astype(np.float64) @ W.astype(np.float64)


def _q(v: np.ndarray, a: np.ndarray) -> np.ndarray:
    return quantize(v.astype(np.float32), np.broadcast_to(a, v.shape)).astype(np.float64)


def tensorwise_f64(X: np.ndarray, W: np.ndarray) -> np.ndarray:
    """Tensor-wise int8 product before the final rounding: one absmax constant for
    all of X and one for all of W; the integer product is dequantized by their
    product (a / 127 per factor), the same expression as the oracle's outer-product
    dequantization with every row and column constant equal."""
    ax = np.float32(np.abs(X.astype(np.float64)).max())
    aw = np.float32(np.abs(W.astype(np.float64)).max())
    acc = _q(X, ax) @ _q(W, aw)
    return acc * (np.float64(ax) * np.float64(aw)) / (QMAX * QMAX)


def tensorwise(X: np.ndarray, W: np.ndarray) -> np.ndarray:
    return tensorwise_f64(X, W).astype(np.float16)


def groupwise_f64(X: np.ndarray, W: np.ndarray, group: int) -> np.ndarray:
    """Group-wise int8 product before the final rounding: K is cut into consecutive
    groups of `group` entries (the last one possibly shorter); within a group each
    row of X and each column of W has its own absmax constant, and the dequantized
    group products (outer product of the group's constants) are summed."""
    M, K = X.shape
    N = W.shape[1]
    Y = np.zeros((M, N))
    for g0 in range(0, K, group):
        xs = X[:, g0:g0 + group].astype(np.float64)
        ws = W[g0:g0 + group, :].astype(np.float64)
        ax = np.abs(xs).max(axis=1).astype(np.float32)      # per row of X
        aw = np.abs(ws).max(axis=0).astype(np.float32)      # per column of W
        acc = _q(xs, ax[:, None]) @ _q(ws, aw[None, :])
        Y += acc * np.outer(ax.astype(np.float64), aw.astype(np.float64)) / (QMAX * QMAX)
    return Y


def groupwise(X: np.ndarray, W: np.ndarray, group: int) -> np.ndarray:
    return groupwise_f64(X, W, group).astype(np.float16)


def vectorwise(X: np.ndarray, W: np.ndarray) -> np.ndarray:
    Wq, a_w = prepare_weight(W)
    return mixed_matmul(X, Wq, a_w, float("inf"))["Y"]


def decomposed(X: np.ndarray, W: np.ndarray, t: float) -> np.ndarray:
    Wq, a_w = prepare_weight(W)
    return mixed_matmul(X, Wq, a_w, t)["Y"]


def relative_errors(Y: np.ndarray, ref: np.ndarray) -> dict:
    """max |Y - ref| / max |ref| and the relative RMS error."""
    d = Y.astype(np.float64) - ref
    return {"max": float(np.abs(d).max() / np.abs(ref).max()),
            "rms": float(np.sqrt((d * d).mean() / (ref * ref).mean()))}


def ablation(X: np.ndarray, W: np.ndarray, t: float, group: int = 128) -> dict:
    ref = exact_product(X, W)
    return {
        "tensor-wise": relative_errors(tensorwise(X, W), ref),
        f"group-wise ({group})": relative_errors(groupwise(X, W, group), ref),
        "vector-wise": relative_errors(vectorwise(X, W), ref),
        "decomposed": relative_errors(decomposed(X, W, t), ref),
    }


def main() -> None:
    from int8_mixed_precision_col_amd import inputs

    for name, wl in inputs.WORKLOADS.items():
        rows = min(wl.M, 64)
        X, _ = inputs.make_x(wl, rows=rows)
        W = inputs.make_w(wl)[:, :512]
        res = ablation(X, W, wl.threshold)
        cells = "  ".join(f"{k}: {v['rms']:.2e} (max {v['max']:.2e})" for k, v in res.items())
        print(f"{name:18s} rows {rows:3d} x cols {W.shape[1]}:  {cells}", flush=True)


if __name__ == "__main__":
    main()
