"""Seeded synthetic inputs for the mixed-precision int8 matmul.

This module only draws random numbers. It holds none of the method's
arithmetic (no thresholds applied, no scales, no quantization), so both the
HIP path and the CPU oracle can take their inputs from it without sharing any
of the computation under test.

The activation recipe mirrors the structure the pages describe for hidden
states of large transformers: a standard-normal background, plus a handful of
"emergent" feature dimensions (about 0.1% of features) whose magnitudes are
far above the rest and which are large in most sequence positions
("8-bit Matrix Multiplication for Large Language Models", Summary &
Methodology Analysis; "Compress your LLMs", bullets on outlier features and
the 6.7B phase shift). Weights are i.i.d. normal with a small std.

Draw order (fixed, one ``numpy.random.default_rng(seed)`` per workload):
  1. X background: standard_normal((M, K), float32)
  2. outlier dims: choice(K, n_dims, replace=False)
  3. per dim, in that order: tokens = choice(M, round(frac*M), replace=False),
     magnitudes = uniform(lo, hi, len(tokens)), signs = choice([-1, 1], len(tokens));
     X[tokens, dim] = signs * magnitudes
  4. X -> float16
  5. W: standard_normal((K, N), float32) * w_std -> float16, drawn in row chunks
"""

from __future__ import annotations

import dataclasses
import hashlib

import numpy as np

THRESHOLD = 6.0


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    M: int
    K: int
    N: int
    n_dims: int
    lo: float
    hi: float
    frac: float
    w_std: float
    threshold: float = THRESHOLD
    seed: int = 0
    # True when the weight is handed over already converted to int8 with fp32
    # column scales (it is still drawn as fp16 first, then converted).
    prequantized: bool = False

    @property
    def flops(self) -> int:
        return 2 * self.M * self.K * self.N


# The five transformer-shaped workloads.
WORKLOADS = {
    "tiny": Workload("tiny", 16, 1024, 1024, 2, 15.0, 25.0, 0.75, 0.02),
    "opt6.7b_ffn_up": Workload("opt6.7b_ffn_up", 2048, 4096, 16384, 6, 15.0, 60.0, 0.75, 0.02),
    "decode_8x4096": Workload("decode_8x4096", 8, 4096, 4096, 6, 15.0, 60.0, 0.75, 0.02,
                              prequantized=True),
    "13b_ffn_down": Workload("13b_ffn_down", 4096, 20480, 5120, 20, 15.0, 60.0, 0.60, 0.015),
    "175b_layer_share": Workload("175b_layer_share", 4096, 12288, 49152, 12, 20.0, 80.0, 0.75,
                                 0.01, prequantized=True),
}


def make_x(wl: Workload, rows: int | None = None) -> tuple[np.ndarray, np.ndarray]:
    """Return (X float16 [M, K], planted outlier dims int64 [n_dims]).

    ``rows`` keeps only the first rows of the same draw (same outlier dims).
    """
    rng = np.random.default_rng(wl.seed)
    M, K = wl.M, wl.K
    X = rng.standard_normal((M, K), dtype=np.float32)
    dims = rng.choice(K, wl.n_dims, replace=False)
    n_tok = int(round(wl.frac * M))
    for d in dims:
        tokens = rng.choice(M, n_tok, replace=False)
        mags = rng.uniform(wl.lo, wl.hi, n_tok)
        signs = rng.choice(np.array([-1.0, 1.0]), n_tok)
        X[tokens, d] = (signs * mags).astype(np.float32)
    X16 = X.astype(np.float16)
    if rows is not None:
        X16 = np.ascontiguousarray(X16[:rows])
    return X16, np.sort(dims)


def make_w(wl: Workload, chunk_rows: int = 1024) -> np.ndarray:
    """Return W float16 [K, N] (row-major, K = input features)."""
    # A second stream, so that W does not depend on how many numbers X drew.
    rng = np.random.default_rng([wl.seed, 1])
    K, N = wl.K, wl.N
    W = np.empty((K, N), dtype=np.float16)
    for r0 in range(0, K, chunk_rows):
        r1 = min(K, r0 + chunk_rows)
        W[r0:r1] = (rng.standard_normal((r1 - r0, N), dtype=np.float32)
                    * np.float32(wl.w_std)).astype(np.float16)
    return W


def random_case(seed: int, M: int, K: int, N: int, n_dims: int = 3, lo: float = 15.0,
                hi: float = 60.0, frac: float = 0.75, w_std: float = 0.02):
    """Small seeded case of arbitrary shape with the same structure."""
    wl = Workload(f"case{seed}", M, K, N, min(n_dims, K), lo, hi, frac, w_std, seed=seed)
    X, dims = make_x(wl)
    return X, make_w(wl), dims


def digest(*arrays: np.ndarray) -> str:
    """SHA-256 of the raw bytes, so two consumers can show they saw the same input."""
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).view(np.uint8).reshape(-1).data)
    return h.hexdigest()[:16]
