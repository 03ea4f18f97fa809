"""GPU parity of the one-pass activation quantization (one pass over X with provisional
row constants, then the fix-up launch; int8_quantize_activations and int8_mixed_matmul
take it for K <= 32768) against the CPU oracle, bit for bit: the state's Xq, a_x,
outlier column list and count, and Xo.

The inputs drive every branch of the fix-up: rows whose provisional constant sits in a
column that another row makes an outlier (the row is requantized), sub-threshold values
in outlier columns (their codes are zeroed), ties at the row max between an outlier and a
kept column, pass-1 blocks that flag more columns than they list, more outlier columns
than are patched in place, more than max_outliers, thresholds 0 and +inf, zero rows, and
ragged M and K around the pass-1 block geometry (one to several rows per block).
"""

import numpy as np
import pytest
import torch

import oracle
from int8_mixed_precision_col_amd import binding, inputs
from tests.gpu_util import announce, check_y, dev, host

pytestmark = pytest.mark.gpu
INF = float("inf")


def planted(seed, M, K, n_dims=6, lo=15.0, hi=60.0, frac=0.6):
    wl = inputs.Workload(f"f{seed}", M, K, 16, n_dims, lo, hi, frac, 0.02, seed=seed)
    X, _ = inputs.make_x(wl)
    return X


def state_case(X, t, mo):
    """Quantize X once on the GPU and compare every field of the state with the oracle."""
    M = X.shape[0]
    ref = oracle.quant_rows(X, t)
    got = binding.QuantizedActivations(dev(X), t, mo).contents()
    assert got["count"] == ref["count"]
    n = min(ref["count"], mo)
    assert np.array_equal(host(got["idx"])[:n], ref["idx"][:n])
    assert np.array_equal(host(got["a_x"]), ref["a_x"])
    assert np.array_equal(host(got["Xq"]), ref["Xq"])
    o_stride = got["Xo"].shape[1]
    o_pad = min((ref["count"] + 15) // 16 * 16, o_stride)
    k = min(ref["count"], o_pad)
    exp = np.zeros((M, o_pad), np.float16)
    exp[:, :k] = X[:, ref["idx"][:k]]
    assert np.array_equal(host(got["Xo"])[:, :o_pad].view(np.uint16), exp.view(np.uint16))
    return ref


@pytest.mark.parametrize("M,K", [(1, 64), (7, 1040), (512, 1024), (513, 4112), (600, 2048),
                                 (1025, 528), (2048, 4096), (4096, 12288), (4096, 20480),
                                 (33, 32768)])
def test_planted_recipe(M, K):
    announce(f"fused quant planted M={M} K={K}")
    ref = state_case(planted(M + 3 * K, M, K), 6.0, min(256, K))
    assert M < 8 or ref["count"] >= 1


def test_two_launch_fallback_above_32768():
    announce("fused quant fallback K=32784")
    state_case(planted(11, 40, 32784), 6.0, 256)


def argmax_in_outlier_column(seed, M, K):
    """Column 3 is an outlier through row 0 only; in every other row its sub-threshold
    value is the row's largest, so every provisional constant is wrong. Column K - 5 is an
    outlier through the last row only and holds small values elsewhere (zeroed codes)."""
    rng = np.random.default_rng([seed, 3])
    X = (rng.standard_normal((M, K)) * 0.5).astype(np.float32)
    X[:, 3] = 5.5
    X[0, 3] = 10.0
    X[:, K - 5] = 0.75
    X[M - 1, K - 5] = -7.0
    return X.astype(np.float16)


@pytest.mark.parametrize("M,K", [(3, 256), (520, 2048), (1000, 1040)])
def test_provisional_constant_in_outlier_column(M, K):
    announce(f"fused quant requantized rows M={M} K={K}")
    X = argmax_in_outlier_column(M + K, M, K)
    ref = state_case(X, 6.0, 16)
    assert ref["count"] == 2 and ref["a_x"][1] < 5.5


def test_ties_at_the_row_max():
    """Rows whose largest kept magnitude is reached both in an outlier column (flagged
    by another row, in another pass-1 block) and in a kept column, before and after it,
    in the same and in different waves' chunks; and rows reaching it only there."""
    announce("fused quant ties at the row max")
    M, K = 1100, 4096
    rng = np.random.default_rng(9)
    X = (rng.standard_normal((M, K)) * 0.4).astype(np.float32)
    X[M - 1, 100] = 8.0                 # column 100: outlier through the last row
    X[M - 1, 3000] = -8.0               # column 3000: outlier through the last row
    for r in range(0, M - 1, 4):
        X[r, 100] = 4.0                 # outlier column ties with a kept column...
        X[r, 101 if r % 8 == 0 else 2900] = -4.0   # ...next to it, or in another wave
    for r in range(1, M - 1, 4):
        X[r, 3000] = 4.0
        X[r, 50] = 4.0                  # kept column before the outlier one
    for r in range(2, M - 1, 4):
        X[r, :] = 0.0
        X[r, 100] = 3.0                 # only nonzero value sits in an outlier column
    state_case(X.astype(np.float16), 6.0, 16)


def spread_outliers(seed, M, K, ncols, rows_each=1):
    """ncols outlier columns, each reaching the threshold in rows_each rows spread
    over the matrix (so that each pass-1 block sees a few of them)."""
    rng = np.random.default_rng([seed, 5])
    X = (rng.standard_normal((M, K)) * 0.7).astype(np.float32)
    cols = rng.choice(K, size=ncols, replace=False)
    for c in cols:
        rows = rng.choice(M, size=rows_each, replace=False)
        X[rows, c] = rng.choice([-1.0, 1.0], size=rows_each) * rng.uniform(6.0, 30.0, rows_each)
    return X.astype(np.float16)


@pytest.mark.parametrize("M,K,ncols,rows_each,mo", [
    (2048, 1024, 40, 3, 256),    # patched in place, every block flags a few columns
    (700, 2048, 64, 700, 256),   # every row flags 64 columns: the most a block lists
    (700, 2048, 65, 700, 256),   # one more: blocks publish whole masks; rows requantized
    (1500, 1040, 150, 20, 256),  # more than patched in place: every row requantized
    (600, 1024, 20, 30, 16),     # more than max_outliers: status 7, rows requantized
])
def test_many_outlier_columns(M, K, ncols, rows_each, mo):
    announce(f"fused quant {ncols} outlier columns M={M} K={K} max_outliers={mo}")
    X = spread_outliers(M + K + ncols, M, K, ncols, rows_each)
    ref = state_case(X, 6.0, mo)
    assert ref["count"] == ncols


@pytest.mark.parametrize("t", [0.0, INF, 6.0])
def test_threshold_extremes_and_zero_rows(t):
    announce(f"fused quant threshold {t}")
    M, K = 530, 1040
    X = planted(77, M, K)
    X[5] = 0.0
    X[6, ::97] = np.float16(6.0)        # entries exactly at the threshold
    X[7, :] = 0.0
    X[7, 9] = 9.0                       # all of the row's mass in an outlier column
    ref = state_case(X, t, K if t == 0.0 else 256)
    if t == 0.0:
        assert ref["count"] == K and not ref["a_x"].any()
    if t == INF:
        assert ref["count"] == 0


@pytest.mark.parametrize("M,K,N", [(520, 2048, 272), (1025, 4112, 528)])
def test_mixed_matmul_requantized_rows(M, K, N):
    """The one-call product over inputs whose rows are requantized by the fix-up: the
    int32 sums bit for bit, the fp16 output within tolerance."""
    announce(f"fused quant through int8_mixed_matmul M={M} K={K} N={N}")
    X = argmax_in_outlier_column(M * 3 + K, M, K)
    rng = np.random.default_rng([M, N])
    W = (rng.standard_normal((K, N)) * 0.02).astype(np.float16)
    Wq_ref, aw_ref = oracle.prepare_weight(W)
    ref = oracle.mixed_matmul(X, Wq_ref, aw_ref, 6.0)
    Wq, aw = binding.prepare_weight(dev(W))
    acc = torch.empty((M, N), dtype=torch.int32, device="cuda")
    Y = binding.mixed_matmul(dev(X), Wq, aw, 6.0, 256, acc_out=acc)
    assert np.array_equal(host(acc), ref["acc"])
    check_y(host(Y), ref["Y"])
