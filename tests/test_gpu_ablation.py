"""The accuracy ablation on the GPU path. Element by element, the library's decomposed
product (t = 6), the same kernels without the decomposition (t = +inf) and the
weight-only product each match the oracle's version of that scheme within the fp16
tolerance; and, as error against exact X @ W, the decomposed product is as close as
the oracle's and several times closer than plain vector-wise int8."""

import numpy as np
import pytest
import torch

import oracle
from int8_mixed_precision_col_amd import binding, inputs
from oracle import ablation
from tests.gpu_util import announce, check_y, dev, host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,rows,cols", [("opt6.7b_ffn_up", 64, 1024), ("decode_8x4096", 8, 1024)])
def test_gpu_decomposition_accuracy(name, rows, cols):
    announce(f"ablation on the GPU path: {name} rows {rows} cols {cols}")
    wl = inputs.WORKLOADS[name]
    X, _ = inputs.make_x(wl, rows=rows)
    W = np.ascontiguousarray(inputs.make_w(wl)[:, :cols])
    ref = ablation.exact_product(X, W)
    Xd = dev(X)
    Wq, aw = binding.prepare_weight(dev(W))
    y_dec = host(binding.mixed_matmul(Xd, Wq, aw, wl.threshold, 256))
    y_vec = host(binding.mixed_matmul(Xd, Wq, aw, float("inf"), 256))
    # element by element: both GPU products against the oracle's same scheme
    check_y(y_dec, ablation.decomposed(X, W, wl.threshold))
    check_y(y_vec, ablation.vectorwise(X, W))
    e_dec = ablation.relative_errors(y_dec, ref)["rms"]
    e_vec = ablation.relative_errors(y_vec, ref)["rms"]
    o_dec = ablation.relative_errors(ablation.decomposed(X, W, wl.threshold), ref)["rms"]
    assert abs(e_dec - o_dec) < 0.1 * o_dec
    assert e_vec > 3 * e_dec
    if binding.is_decode(rows, wl.K):
        y_wo = host(binding.weight_only_matmul(Xd, Wq, aw))
        Wq_ref, aw_ref = oracle.prepare_weight(W)
        check_y(y_wo, oracle.weight_only_matmul(X, Wq_ref, aw_ref))
        e_wo = ablation.relative_errors(y_wo, ref)["rms"]
        assert e_wo < e_dec
    print(f"[gpu case] {name}: rms error decomposed {e_dec:.2e}, vector-wise only {e_vec:.2e}",
          flush=True)
