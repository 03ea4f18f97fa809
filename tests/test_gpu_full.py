"""GPU parity at the five transformer-shaped workloads' full sizes, in the same
launch configuration the benchmark times (default max_outliers, threshold 6.0).

The activation quantization (mask, ranked outlier columns, count, a_x, Xq) is
compared in full, bit for bit. For the product, the oracle computes a sample of
rows x columns from its own full-size quantization: those int32 accumulators
must match bit for bit and those fp16 outputs within TOL of their absmax.
"""

import numpy as np
import pytest
import torch

import oracle
from int8_mixed_precision_col_amd import binding, inputs
from tests.gpu_util import announce, check_y, dev, host

pytestmark = pytest.mark.gpu

MAX_OUTLIERS = 256


@pytest.mark.parametrize("name", list(inputs.WORKLOADS))
def test_full_size_workload(name):
    wl = inputs.WORKLOADS[name]
    announce(f"full-size {name}: M={wl.M} K={wl.K} N={wl.N} "
             f"({'decode' if binding.is_decode(wl.M, wl.K) else 'prefill'} path)")
    X, dims = inputs.make_x(wl)
    W = inputs.make_w(wl)
    rng = np.random.default_rng(123)
    cols = np.sort(rng.choice(wl.N, min(wl.N, 192), replace=False))
    rows = np.sort(rng.choice(wl.M, min(wl.M, 48), replace=False))

    # weight conversion: sampled columns, bit-exact
    Xd = dev(X)
    Wd = dev(W)
    Wq, aw = binding.prepare_weight(Wd)
    del Wd
    Wq_s_ref, aw_s_ref = oracle.prepare_weight(np.ascontiguousarray(W[:, cols]))
    del W
    cols_t = torch.from_numpy(cols).cuda()
    assert np.array_equal(host(aw[cols_t]), aw_s_ref)
    assert np.array_equal(host(binding.untile_weight(Wq, wl.K)[cols_t]), Wq_s_ref)

    # activation quantization: complete, bit-exact
    q_ref = oracle.quant_rows(X, wl.threshold)
    assert set(dims.tolist()) <= set(q_ref["idx"].tolist())
    q = binding.quant_rows(Xd, wl.threshold, MAX_OUTLIERS)
    assert int(host(q["count"])[0]) == q_ref["count"]
    assert np.array_equal(host(q["idx"])[:q_ref["count"]], q_ref["idx"])
    assert np.array_equal(host(q["mask"]).view(np.uint32), oracle.mask_words(q_ref["mask"]))
    assert np.array_equal(host(q["a_x"]), q_ref["a_x"])
    assert np.array_equal(host(q["Xq"]), q_ref["Xq"])
    del q

    # the product, in the benchmark's configuration
    acc = torch.empty((wl.M, wl.N), dtype=torch.int32, device="cuda")
    ws = binding.make_workspace(wl.M, wl.K, wl.N, MAX_OUTLIERS)
    Y = binding.mixed_matmul(Xd, Wq, aw, wl.threshold, MAX_OUTLIERS, workspace=ws, acc_out=acc)
    assert binding.read_status(ws) == (0, q_ref["count"])
    rows_t = torch.from_numpy(rows).cuda()
    acc_s = host(acc[rows_t][:, cols_t])
    y_s = host(Y[rows_t][:, cols_t])
    assert torch.isfinite(Y).all().item()

    # oracle on the sample, from its full-size quantization
    acc_ref = oracle.int8_matmul(q_ref["Xq"][rows], Wq_s_ref)
    y_ref = (oracle.dequant_outer(acc_ref, q_ref["a_x"][rows], aw_s_ref)
             + oracle.outlier_matmul(X[rows], q_ref["idx"], Wq_s_ref, aw_s_ref)).astype(np.float16)
    assert np.array_equal(acc_s, acc_ref)
    rel = check_y(y_s, y_ref)
    print(f"[gpu case] {name}: sampled rel err {rel:.2e}, outliers {q_ref['count']}", flush=True)
