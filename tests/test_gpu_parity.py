"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bit-exact: Wq, a_w, outlier mask / index list / count, a_x, Xq and the int32
accumulators. Within TOL of max|Y_oracle|: the fp16 output. Shapes span several
tiles with ragged tails on both dispatch paths (decode kernel for M <= 16, and
mask -> quant -> MFMA GEMM otherwise, in its small- and large-tile configurations).
"""

import numpy as np
import pytest
import torch

import oracle
from int8_mixed_precision_col_amd import binding, inputs
from tests.gpu_util import TOL, announce, check_y, dev, grid_weight, host

pytestmark = pytest.mark.gpu
INF = float("inf")


def planted(seed, M, K, n_dims=4, lo=15.0, hi=60.0, frac=0.75):
    wl = inputs.Workload(f"p{seed}", M, K, 16, n_dims, lo, hi, frac, 0.02, seed=seed)
    X, _ = inputs.make_x(wl)
    return X


def weight(seed, K, N, std=0.02):
    rng = np.random.default_rng([seed, 7])
    return (rng.standard_normal((K, N), dtype=np.float32) * np.float32(std)).astype(np.float16)


# ------------------------------------------------------------------ prepare

@pytest.mark.parametrize("K,N,layout", [(1024, 1024, 0), (1040, 528, 0), (1040, 528, 1),
                                        (16, 16, 0), (4112, 80, 1), (48, 32, 0), (48, 32, 1),
                                        # wide [K, N] weights, ragged in K and N
                                        (1040, 49216, 0), (2064, 24528, 0)])
def test_prepare_weight_bit_exact(K, N, layout):
    announce(f"prepare_weight K={K} N={N} layout={layout}")
    W = weight(K + N, K, N)
    W[:, 3] = 0                         # all-zero column: constant 0, codes 0
    Wq_ref, aw_ref = oracle.prepare_weight(W)
    src = W if layout == 0 else np.ascontiguousarray(W.T)
    Wq, aw = binding.prepare_weight(dev(src), layout)
    assert np.array_equal(host(aw), aw_ref)
    assert np.array_equal(host(binding.untile_weight(Wq, K)), Wq_ref)
    # the K padding of the last unit holds zero codes
    pad = host(Wq).reshape(N // 16, -1, 16, 64)[:, -1, :, K % 64:] if K % 64 else None
    assert pad is None or not pad.any()


@pytest.mark.parametrize("K,N", [(1024, 1024), (1040, 528), (16, 16), (4112, 80), (48, 32)])
def test_tile_weight_round_trip(K, N):
    """int8_tile_weight is layout only: the [N, K] view of a prepared weight, tiled again,
    is the prepared weight byte for byte (K padding zero)."""
    announce(f"tile_weight round trip K={K} N={N}")
    Wq, _ = binding.prepare_weight(dev(weight(K + N + 5, K, N)))
    again = binding.tile_weight(binding.untile_weight(Wq, K))
    assert torch.equal(again, Wq)


@pytest.mark.parametrize("M,K,N", [(8, 4096, 1024), (300, 1040, 528), (24, 4096, 1040)])
def test_imported_int8_weight(M, K, N):
    """A weight handed over already in int8 ([N, K] codes with fp32 column constants, the
    form a pre-quantized checkpoint takes): the oracle's own conversion, placed by
    int8_tile_weight, gives the oracle's product (decode kernel, tiled GEMM and
    weight-stream GEMM)."""
    path = "decode" if binding.is_decode(M, K) else "prefill"
    announce(f"imported int8 weight {path} M={M} K={K} N={N}")
    X = planted(M + K + 7, M, K, n_dims=3)
    W = weight(M + N + 7, K, N)
    Wq_ref, aw_ref = oracle.prepare_weight(W)
    ref = oracle.mixed_matmul(X, Wq_ref, aw_ref, 6.0)
    Wq = binding.tile_weight(dev(Wq_ref))
    acc = torch.empty((M, N), dtype=torch.int32, device="cuda")
    Y = binding.mixed_matmul(dev(X), Wq, dev(aw_ref), 6.0, 256, acc_out=acc)
    assert np.array_equal(host(acc), ref["acc"])
    check_y(host(Y), ref["Y"])


# ------------------------------------------------------------------ quant rows

def _quant_case(X, t, mo):
    ref = oracle.quant_rows(X, t)
    got = binding.quant_rows(dev(X), t, mo)
    count = int(host(got["count"])[0])
    assert count == ref["count"]
    assert np.array_equal(host(got["mask"]).view(np.uint32), oracle.mask_words(ref["mask"]))
    n = min(count, mo)
    assert np.array_equal(host(got["idx"])[:n], ref["idx"][:n])
    assert np.array_equal(host(got["a_x"]), ref["a_x"])
    assert np.array_equal(host(got["Xq"]), ref["Xq"])
    return ref


@pytest.mark.parametrize("M,K,t,mo", [
    (16, 1024, 6.0, 256), (300, 1040, 6.0, 256), (7, 20480, 6.0, 256),
    (3, 33024, 6.0, 64), (129, 4096, INF, 16), (33, 528, 0.0, 528), (65, 1024, 6.0, 2),
])
def test_quant_rows_bit_exact(M, K, t, mo):
    announce(f"quant_rows M={M} K={K} t={t} max_outliers={mo}")
    X = planted(M * 31 + K, M, K, n_dims=5)
    _quant_case(X, t, mo)


def test_quant_rows_adversarial():
    announce("quant_rows adversarial ties / zero rows / all-outlier rows")
    rng = np.random.default_rng(5)
    X = rng.standard_normal((37, 96)).astype(np.float32)
    X[:, 10] = 6.0                       # exactly the threshold: outlier
    X[:, 11] = np.float16(5.99609375)    # largest fp16 below 6: not an outlier
    X[2, :] = 0.0                        # zero row
    X[3, :] = 0.0
    X[3, 40] = 9.0                       # row whose only nonzero is in an outlier column
    X[4, :] = 2.5                        # constant row: every code 127
    X[5, 50] = -6.0
    ref = _quant_case(X.astype(np.float16), 6.0, 16)
    assert 10 in ref["idx"] and 11 not in ref["idx"] and ref["a_x"][3] == 0


def tie_rows(seed, M, K):
    """Rows whose codes are exact half-integers in bulk. With row absmax a = 127 / 2^p,
    127 x / a = 2^p x, so every x = (k + 1/2) / 2^p (exact in fp16) is a tie that
    round-half-to-even must settle; the bracketing pair disagrees on all of them. Row 0
    is ties only (max 127/64), row 1 half ties, row 2 ties under a = 127/32, row 3 also
    holds an outlier column; the other rows are ordinary."""
    rng = np.random.default_rng([seed, 11])
    X = (rng.standard_normal((M, K)) * 0.5).astype(np.float32)
    sgn = rng.choice([-1.0, 1.0], size=(M, K))
    ties64 = (rng.integers(0, 127, size=(M, K)) + 0.5) / 64.0 * sgn
    ties32 = (rng.integers(0, 127, size=(M, K)) + 0.5) / 32.0 * sgn
    X[0] = ties64[0]
    X[0, 5] = 127.0 / 64.0
    if M > 1:
        half = rng.random(K) < 0.5
        X[1] = np.where(half, ties64[1], np.clip(X[1], -1.9, 1.9))
        X[1, 9] = -127.0 / 64.0
    if M > 2:
        X[2] = ties32[2]
        X[2, 3] = 127.0 / 32.0
    if M > 3:
        X[3] = ties64[3]
        X[3, 1] = 127.0 / 64.0
        X[3, 7] = 6.0                      # outlier column: excluded from the row max
    return X.astype(np.float16)


@pytest.mark.parametrize("M,K", [(8, 1024), (8, 4096), (3, 8192), (40, 1040)])
def test_ties_in_bulk(M, K):
    """Codes at exact half-integers, many per 8-column chunk, on both paths: the int32
    sums (and, on the multi-kernel path, Xq itself) must match the oracle bit for bit."""
    path = "decode" if binding.is_decode(M, K) else "prefill"
    announce(f"ties in bulk {path} M={M} K={K}")
    X = tie_rows(M + K, M, K)
    if path == "prefill":
        _quant_case(X, 6.0, 16)
    W = weight(M + 2 * K, K, 272)
    ref, Y, acc = _mixed(X, W, 6.0, mo=16)
    assert ref["a_x"][0] == np.float32(127.0 / 64.0) and (M <= 3 or ref["count"] >= 1)
    assert np.array_equal(acc, ref["acc"])
    check_y(Y, ref["Y"])


# ------------------------------------------------------------------ mixed matmul

def _mixed(X, W, t, mo=256, workspace=None):
    Wq_ref, aw_ref = oracle.prepare_weight(W)
    ref = oracle.mixed_matmul(X, Wq_ref, aw_ref, t)
    Wq, aw = binding.prepare_weight(dev(W))
    M, N = X.shape[0], W.shape[1]
    acc = torch.empty((M, N), dtype=torch.int32, device="cuda")
    Y = binding.mixed_matmul(dev(X), Wq, aw, t, mo, workspace=workspace, acc_out=acc)
    return ref, host(Y), host(acc)


CASES = [
    # (M, K, N): decode kernel
    (16, 1024, 1024), (5, 1040, 528), (8, 4096, 4096), (1, 32, 16), (16, 2048, 80),
    (4, 8192, 256), (3, 8176, 48), (9, 3600, 144),
    # prefill, small tiles
    (300, 1040, 528), (17, 256, 4112), (64, 8192, 256), (1, 12288, 64),
    # prefill, tile shapes the launcher picks: 128 x 128 (many tiles), 256 x 256,
    # 128 x 256
    (1040, 1040, 16400), (385, 1040, 16608), (129, 1040, 16608),
    # prefill, weight-stream GEMM for a few tokens (token groups x feature groups per
    # block: 1x1, 2x1, 3x1, 4x1, 2x2)
    (9, 8208, 272), (24, 4096, 1040), (40, 2064, 1040), (64, 1024, 2064), (20, 1040, 32784),
    # prefill, two launches: the features that fill whole waves of 256 x 256 tiles, then
    # the remaining features on 128 x 128 tiles writing into the same output rows
    (4096, 1024, 4352), (4000, 1040, 4400),
]


@pytest.mark.parametrize("M,K,N", CASES)
def test_mixed_matmul_parity(M, K, N):
    path = "decode" if binding.is_decode(M, K) else "prefill"
    announce(f"mixed_matmul {path} M={M} K={K} N={N}")
    X = planted(M + 3 * K + N, M, K, n_dims=3)
    W = weight(M + K, K, N)
    ref, Y, acc = _mixed(X, W, 6.0, mo=min(256, K))
    assert np.array_equal(acc, ref["acc"])
    check_y(Y, ref["Y"])


def test_largest_k_extreme_accumulators():
    """K at the library's int32 guard (127^2 K < 2^31): a row of +1.0 and a row of -1.0
    (every code +-127) against a weight column of 0.25 (every code 127) give the
    largest sums the library admits, +-2 147 350 544, next to ordinary rows."""
    M, K, N = 4, 133136, 32
    announce(f"largest K M={M} K={K} N={N}")
    rng = np.random.default_rng(11)
    X = rng.standard_normal((M, K), dtype=np.float32).astype(np.float16)
    X[0, :] = 1.0
    X[1, :] = -1.0
    W = weight(K + N, K, N)
    W[:, 0] = 0.25
    ref, Y, acc = _mixed(X, W, 6.0, mo=16)
    assert ref["acc"][0, 0] == 127 * 127 * K and ref["acc"][1, 0] == -127 * 127 * K
    assert np.array_equal(acc, ref["acc"])
    check_y(Y, ref["Y"])
    check_y(Y[2:], ref["Y"][2:])


# one shape per decode instantiation (rows held 2/4/8/16 x k-steps per wave 2/4/8/16,
# masked X staged in LDS), then the two without the staged copy (M = 16 from K = 2880,
# M = 5..8 from K = 5536), at their largest shapes too
DECODE_SHAPES = [(2, 528), (1, 2000), (2, 4000), (1, 8000), (3, 1008), (4, 1552), (3, 4080),
                 (4, 8192), (6, 992), (7, 2032), (5, 4096), (6, 5456), (12, 720), (11, 1792),
                 (10, 3264),
                 (7, 7008), (8, 8192), (13, 3600), (16, 4096),
                 # one or two rows at 513-2048 columns (8 pairs of waves there; from 3 rows
                 # on, 2 or 4 pairs: (3, 1008), (6, 992), (12, 720), (4, 1552), (7, 2032),
                 # (11, 1792) above)
                 (1, 1008), (2, 1104)]


@pytest.mark.parametrize("M,K", DECODE_SHAPES)
def test_decode_every_instantiation(M, K):
    assert binding.is_decode(M, K)
    announce(f"decode instantiation M={M} K={K}")
    X = planted(5 * M + K, M, K, n_dims=4)
    W = weight(K + 1, K, 80)
    ref, Y, acc = _mixed(X, W, 6.0, mo=min(256, K))
    assert np.array_equal(acc, ref["acc"])
    check_y(Y, ref["Y"])


@pytest.mark.parametrize("M,K", [(1, 1024), (2, 4000), (3, 2048), (8, 4096), (16, 1040),
                                 # two pairs of waves: later outlier passes of 16 columns
                                 (4, 1024), (16, 960)])
def test_decode_many_outlier_columns(M, K):
    """More outlier columns than the decode kernel stages while it makes the codes (16),
    spread over every pair of waves: the first 16 come from the staged values (copied
    from registers at one or two tokens, gathered from X and Wq from three on), the rest
    from the epilogue's later passes (32 columns a pass, 16 with two pairs of waves); the
    ascending order of the outlier sum is kept."""
    assert binding.is_decode(M, K)
    announce(f"decode many outliers M={M} K={K}")
    X = planted(11 * M + K, M, K, n_dims=40, frac=1.0)
    W = weight(K + 3, K, 48)
    ref, Y, acc = _mixed(X, W, 6.0, mo=256)
    assert ref["count"] == 40
    assert np.array_equal(acc, ref["acc"])
    check_y(Y, ref["Y"])


@pytest.mark.parametrize("M,K,N,dims", [(8, 4096, 4112, 4), (2, 2048, 8192, 4), (1, 512, 4128, 4),
                                         (5, 2992, 4624, 4), (6, 2560, 8208, 40)])
def test_decode_two_row_groups(M, K, N, dims):
    """More 16-row groups of Wq than CUs: with 5-8 token rows each decode block takes two
    row groups (32 output features) for one activation pass; odd counts leave the last
    block one real row group (its second clamped, its outputs past N not stored); with 40
    outlier columns the epilogue's later passes stage 32 features per rank. With one or
    two rows the blocks keep one row group and run in several rounds."""
    announce(f"decode two row groups M={M} K={K} N={N} dims={dims}")
    assert binding.is_decode(M, K)
    X = planted(7 * M + K + N, M, K, n_dims=dims, frac=1.0)
    W = weight(K + N, K, N)
    ref, Y, acc = _mixed(X, W, 6.0, mo=256)
    assert ref["count"] == dims
    assert np.array_equal(acc, ref["acc"])
    check_y(Y, ref["Y"])


@pytest.mark.parametrize("M,K,N", [(2048, 1024, 64), (600, 2000, 48)])
def test_lone_outlier_rows_in_every_row_chunk(M, K, N):
    """Each outlier column holds one large value in a single row (first, middle and last
    row chunks of the outlier-mask launch: 64 chunks of 32 rows at 2048 x 1024, 19 at
    600 x 2000): the column mask is the OR over all chunks, so a chunk left out of it
    would quantize that column instead of carrying it in fp16, and the int32
    accumulators would differ."""
    announce(f"lone outlier rows M={M} K={K} N={N}")
    rng = np.random.default_rng([M, K, 3])
    X = (rng.standard_normal((M, K)) * 0.5).astype(np.float32)
    lone = {0: 3, 31: 517 % K, M // 2: 700 % K, M - 33: 901 % K, M - 1: K - 1}
    for r, c in lone.items():
        X[r, c] = 20.0 if r % 2 else -20.0
    X = X.astype(np.float16)
    W = weight(M + K, K, N)
    ws = binding.make_workspace(M, K, N, 256)
    ref, Y, acc = _mixed(X, W, 6.0, workspace=ws)
    assert ref["count"] == len(set(lone.values()))
    assert binding.read_status(ws) == (0, ref["count"])
    assert np.array_equal(acc, ref["acc"])
    check_y(Y, ref["Y"])


@pytest.mark.parametrize("M,K,N", [(16, 1024, 256), (200, 1040, 528), (40, 1040, 528)])
def test_zero_outlier_invariant(M, K, N):
    """t = +inf: no outlier columns; Y is the dequantized int8 product."""
    announce(f"zero-outlier invariant M={M} K={K} N={N}")
    X = planted(11 + M, M, K, n_dims=2)
    W = weight(12 + M, K, N)
    ref, Y, acc = _mixed(X, W, INF)
    assert ref["count"] == 0
    assert np.array_equal(acc, ref["acc"])
    check_y(Y, ref["y_int8"].astype(np.float16))


@pytest.mark.parametrize("M,K,N", [(16, 512, 128), (96, 528, 272), (40, 1024, 272),
                                   # decode kernel with two and four pairs of waves
                                   (16, 1024, 64), (8, 2048, 64)])
def test_all_outlier_invariant(M, K, N):
    """t = 0: every column is an outlier; with a lossless int8 weight, Y = fp16(X @ W)."""
    announce(f"all-outlier invariant M={M} K={K} N={N}")
    rng = np.random.default_rng(M + K)
    X = (rng.standard_normal((M, K)) * 3).astype(np.float16)
    W = grid_weight(rng, K, N)
    ref, Y, acc = _mixed(X, W, 0.0, mo=K)
    assert ref["count"] == K and np.all(acc == 0)
    textbook = (X.astype(np.float64) @ W.astype(np.float64)).astype(np.float16)
    check_y(Y, textbook)


@pytest.mark.parametrize("M,K,N", [(8, 1024, 256), (100, 1024, 256), (40, 1040, 256)])
def test_outlier_overflow_sets_status_and_nan(M, K, N):
    announce(f"outlier overflow M={M} K={K} N={N}")
    X = planted(21 + M, M, K, n_dims=5)
    W = weight(22, K, N)
    Wq, aw = binding.prepare_weight(dev(W))
    ws = binding.make_workspace(M, K, N, 2)
    Y = binding.mixed_matmul(dev(X), Wq, aw, 6.0, 2, workspace=ws)
    status, count = binding.read_status(ws)
    assert status == 7 and count >= 5
    assert torch.isnan(Y).all().item()
    # the same workspace, enough capacity: status clears
    ws2 = binding.make_workspace(M, K, N, 16)
    binding.mixed_matmul(dev(X), Wq, aw, 6.0, 16, workspace=ws2)
    assert binding.read_status(ws2) == (0, count)


@pytest.mark.parametrize("M,K,N", [(100, 1024, 256), (40, 1040, 256)])
def test_quantize_once_overflow_sets_status_and_nan(M, K, N):
    """Too many outlier columns for the state's capacity: the state's status word says
    so and every weight's Y is NaN (tiled and weight-stream GEMMs, whose epilogues
    dequantize the outlier weights from the column list and must not read past it)."""
    announce(f"quantize-once overflow M={M} K={K} N={N}")
    X = planted(41 + M, M, K, n_dims=5)
    Wq, aw = binding.prepare_weight(dev(weight(42, K, N)))
    qa = binding.QuantizedActivations(dev(X), 6.0, 2)
    status, count = binding.read_status(qa.state)
    assert status == 7 and count >= 5
    assert torch.isnan(qa.matmul(Wq, aw)).all().item()
    assert all(torch.isnan(y).all().item() for y in qa.matmul_grouped([(Wq, aw), (Wq, aw)]))


@pytest.mark.parametrize("M,K,N", [(8, 4096, 4096), (700, 2064, 1040), (40, 2064, 1040)])
def test_deterministic(M, K, N):
    announce(f"determinism M={M} K={K} N={N}")
    X = dev(planted(31, M, K))
    Wq, aw = binding.prepare_weight(dev(weight(32, K, N)))
    a = binding.mixed_matmul(X, Wq, aw, 6.0)
    b = binding.mixed_matmul(X, Wq, aw, 6.0)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_workspace_reuse_across_shapes():
    """One workspace sized for the larger call serves a smaller one afterwards."""
    announce("workspace reuse")
    big = binding.make_workspace(512, 2048, 1024, 256)
    for (M, K, N) in [(512, 2048, 1024), (40, 1040, 528)]:
        X = planted(M, M, K)
        W = weight(M, K, N)
        ref, Y, acc = _mixed(X, W, 6.0, workspace=big)
        assert np.array_equal(acc, ref["acc"])
        check_y(Y, ref["Y"])


def test_timing_hook_counts_main_kernel():
    announce("timing hook")
    X = dev(planted(41, 64, 1024))
    Wq, aw = binding.prepare_weight(dev(weight(42, 1024, 512)))
    binding.timing_read()
    binding.timing_enable(True)
    try:
        for _ in range(3):
            binding.mixed_matmul(X, Wq, aw, 6.0)
        ms, n = binding.timing_read()
    finally:
        binding.timing_enable(False)
    assert n == 3 and ms > 0


@pytest.mark.parametrize("M,K,N", [(8, 4096, 1024), (96, 1040, 528)])
def test_graph_replay_matches_eager(M, K, N):
    """A call captured in a HIP graph gives the eager result on every replay, with
    eager work and synchronizations between the replays (the path issues no memset)."""
    path = "decode" if binding.is_decode(M, K) else "prefill"
    announce(f"graph replay {path} M={M} K={K} N={N}")
    X = dev(planted(51, M, K))
    Wq, aw = binding.prepare_weight(dev(weight(52, K, N)))
    ws = binding.make_workspace(M, K, N, 256)
    want = binding.mixed_matmul(X, Wq, aw, 6.0, 256, workspace=ws).clone()
    Y = torch.empty_like(want)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        binding.mixed_matmul(X, Wq, aw, 6.0, 256, workspace=ws, out=Y)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        binding.mixed_matmul(X, Wq, aw, 6.0, 256, workspace=ws, out=Y)
    other = binding.make_workspace(M, K, N, 256)
    for i in range(4):
        Y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.int16), want.view(torch.int16)), f"replay {i}"
        # eager work between replays, on another workspace
        binding.mixed_matmul(X, Wq, aw, 6.0, 256, workspace=other)
        torch.cuda.synchronize()
    assert binding.read_status(ws)[0] == 0


@pytest.mark.parametrize("M,K,N", [(8, 4096, 4096), (1, 32, 16), (16, 1040, 528),
                                   (5, 12288, 64), (3, 16, 48), (16, 12288, 272),
                                   (7, 20480, 48), (12, 5136, 16),
                                   # 32 features per block, odd count of 16-feature groups
                                   (3, 1040, 32784), (16, 528, 34816), (4, 8192, 8192),
                                   # X staged in LDS (M >= 12, K a multiple of 512)
                                   (16, 2048, 4096), (12, 512, 80), (13, 2560, 528)])
def test_weight_only_parity(M, K, N):
    """Weight-only int8 (no activation quantization) against the oracle's fp16(X @ W^)."""
    announce(f"weight-only M={M} K={K} N={N}")
    X = planted(M + K, M, K, n_dims=3)
    W = weight(M + N, K, N)
    Wq_ref, aw_ref = oracle.prepare_weight(W)
    want = oracle.weight_only_matmul(X, Wq_ref, aw_ref)
    Wq, aw = binding.prepare_weight(dev(W))
    Y = binding.weight_only_matmul(dev(X), Wq, aw)
    check_y(host(Y), want)


@pytest.mark.parametrize("M,K,Ns", [(300, 1040, (528, 272, 1040)), (8, 4096, (1024, 512)),
                                    (64, 8192, (256,)), (5, 1024, (32784, 65552)),
                                    (129, 1040, (16608,)), (4000, 528, (4400,))])
def test_quantize_once_feeds_several_weights(M, K, Ns):
    """One activation quantization, several weights: each product equals the oracle
    (acc bit-exact, Y within tolerance) and, on the multi-kernel path, the one-call
    int8_mixed_matmul bit for bit."""
    announce(f"quantize once M={M} K={K} N={Ns}")
    X = planted(M + K, M, K, n_dims=4)
    Xd = dev(X)
    qa = binding.QuantizedActivations(Xd, 6.0, 256)
    q_ref = oracle.quant_rows(X, 6.0)
    assert binding.read_status(qa.state) == (0, q_ref["count"])
    for i, N in enumerate(Ns):
        W = weight(M + N + i, K, N)
        Wq_ref, aw_ref = oracle.prepare_weight(W)
        ref = oracle.mixed_matmul(X, Wq_ref, aw_ref, 6.0)
        Wq, aw = binding.prepare_weight(dev(W))
        acc = torch.empty((M, N), dtype=torch.int32, device="cuda")
        Y = qa.matmul(Wq, aw, acc_out=acc)
        assert np.array_equal(host(acc), ref["acc"])
        check_y(host(Y), ref["Y"])
        if not binding.is_decode(M, K):
            Y1 = binding.mixed_matmul(Xd, Wq, aw, 6.0, 256)
            assert torch.equal(Y.view(torch.int16), Y1.view(torch.int16))


@pytest.mark.parametrize("M,K,Ns", [(300, 1040, (528, 272, 1040)), (8, 4096, (1024, 512)),
                                    (2048, 1024, (4096, 4096, 4096)),
                                    (257, 528, (16, 48, 80, 272, 528, 16, 32, 64)),
                                    (40, 1040, (528, 65536)), (129, 1040, (8304, 8304))])
def test_grouped_launch_equals_per_weight_calls(M, K, Ns):
    """One grouped GEMM launch over several weights: every output equals the
    one-weight int8_mixed_matmul_q call bit for bit (small- and large-tile grids, and
    the weight-stream kernel). In the last case the 68 MB weight sends the grouped call
    to the 128 x 128 tiles while the one-weight call of the small weight takes the
    weight-stream kernel: the two kernels' outputs are compared bit for bit."""
    announce(f"grouped launch M={M} K={K} Ns={Ns}")
    X = planted(M + K + len(Ns), M, K, n_dims=3)
    state = binding.QuantizedActivations(dev(X), 6.0, 64)
    Ws = [weight(M + q, K, n) for q, n in enumerate(Ns)]
    weights = [binding.prepare_weight(dev(W)) for W in Ws]
    got = state.matmul_grouped(weights)
    q_ref = oracle.quant_rows(X, 6.0)
    for (Wq, aw), Yg, W in zip(weights, got, Ws):
        Y1 = state.matmul(Wq, aw)
        assert np.array_equal(host(Yg).view(np.uint16), host(Y1).view(np.uint16))
        # every group against the oracle, element by element
        Wq_ref, aw_ref = oracle.prepare_weight(W)
        assert np.array_equal(host(binding.untile_weight(Wq, K)), Wq_ref)
        ref = oracle.mixed_matmul(X, Wq_ref, aw_ref, 6.0)
        assert np.array_equal(ref["Xq"], q_ref["Xq"])
        check_y(host(Yg), ref["Y"])
