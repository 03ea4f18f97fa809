"""Accuracy ablation: the decomposition against plain int8 schemes, vs exact X @ W.

Pins the claim the method is built on ("LLM.int8(): 8-bit Matrix Multiplication
for Transformers at Scale", Abstract; "8-bit Matrix Multiplication for Large
Language Models", Summary & Methodology Analysis): with outlier feature columns
present, isolating them keeps the int8 product accurate, while per-tensor,
per-vector and (to a lesser degree) per-group constants without the
decomposition lose accuracy to the outliers' magnitude.
"""

import numpy as np
import pytest

from int8_mixed_precision_col_amd import inputs
from oracle import ablation


@pytest.mark.parametrize("name,rows,cols", [("tiny", 16, 256), ("opt6.7b_ffn_up", 32, 256)])
def test_decomposition_is_the_most_accurate(name, rows, cols):
    wl = inputs.WORKLOADS[name]
    X, _ = inputs.make_x(wl, rows=rows)
    W = inputs.make_w(wl)[:, :cols]
    r = ablation.ablation(X, W, wl.threshold)
    dec, vec = r["decomposed"]["rms"], r["vector-wise"]["rms"]
    grp, ten = r["group-wise (128)"]["rms"], r["tensor-wise"]["rms"]
    assert dec < 0.02
    assert dec < grp < vec
    assert vec < ten * 1.05
    assert vec > 3 * dec


def test_without_outliers_the_schemes_agree():
    """No outlier columns: decomposition and plain vector-wise are the same product,
    and both are as accurate as the int8 rounding allows."""
    rng = np.random.default_rng(5)
    X = rng.standard_normal((16, 512)).astype(np.float16)
    W = (rng.standard_normal((512, 128)) * 0.02).astype(np.float16)
    r = ablation.ablation(X, W, 6.0)
    assert r["decomposed"] == r["vector-wise"]
    assert r["vector-wise"]["rms"] < 0.02
