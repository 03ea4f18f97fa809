"""Benchmark of the mixed-precision int8 matmul on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one int8_mixed_matmul call (outlier mask, row quantization + outlier
gathers, int8 MFMA GEMM with the fp16 outlier product and dequant epilogue)
over the workload's synthetic inputs, which are resident in HBM; the weight is
converted to int8 once beforehand, as at checkpoint load. Prints ONE JSON line:
`value` is the prefill effective TOPS (2 M K N / time per call). The `roofline`
object is the GEMM kernel's own rate from HIP events recorded around its
launches during the timed steps. The decode shape (8 tokens) is measured in
the same run as `decode` (GB/s of algorithmic bytes over 32 rotated weights).
`cpu_baseline` times the CPU oracle on a bounded row x column sample.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "mixed int8 matmul effective TOPS (prefill) and HBM GB/s (decode), 1 MI355X"
PEAK_INT8_TOPS = 5000.0      # MI355X dense int8 MFMA, 5.0 POP/s
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, 8 TB/s
MAX_OUTLIERS = 256
MALL_BYTES = 256 << 20       # last-level cache to defeat when re-reading weights


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_digest(*names: str) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "int8_mixed_precision_col_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, kernel_src: str) -> float | None:
    """HBM bytes per launch from committed rocprofv3 counter runs, if still current."""
    path = os.path.join(ROOT, "profiles", f"gemm_hbm_traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256_16") != source_digest(kernel_src):
        return None
    return rec.get("hbm_bytes_per_launch")


def prepare(binding, torch, wl, inputs, copies: int):
    """Draw the workload, move it to the GPU, convert `copies` weights (untimed)."""
    X, _ = inputs.make_x(wl)
    W = inputs.make_w(wl)
    Xd = torch.from_numpy(X).cuda()
    Wd = torch.from_numpy(W).cuda()
    weights = [binding.prepare_weight(Wd)]
    for _ in range(copies - 1):
        Wq, aw = weights[0]
        weights.append((Wq.clone(), aw.clone()))
    del Wd
    torch.cuda.synchronize()
    return X, W, Xd, weights


def time_calls(binding, torch, Xd, weights, wl, n_calls: int, ws, Y):
    binding.timing_read()
    binding.timing_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n_calls):
        Wq, aw = weights[i % len(weights)]
        binding.mixed_matmul(Xd, Wq, aw, wl.threshold, MAX_OUTLIERS, workspace=ws, out=Y)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    binding.timing_enable(False)
    kern_ms, launches = binding.timing_read()
    return (t1 - t0) * 1e3, kern_ms, launches


def cpu_baseline(oracle, X, W, wl, budget_s: float = 15.0) -> dict:
    """The oracle as it stands, on a row x column sample of the workload (full K)."""
    from threadpoolctl import threadpool_info

    def run(ms, ns):
        Wq, aw = oracle.prepare_weight(np.ascontiguousarray(W[:, :ns]))   # load time, untimed
        t0 = time.perf_counter()
        oracle.mixed_matmul(X[:ms], Wq, aw, wl.threshold)
        return time.perf_counter() - t0

    ms = min(wl.M, 256)
    ns = min(wl.N, 512)
    t = run(ms, ns)
    scale = budget_s / max(t, 1e-3)
    ns2 = int(min(wl.N, max(ns, ns * scale)) // 16 * 16)
    rows_scale = max(1.0, ns * scale / ns2)
    ms2 = int(min(wl.M, ms * rows_scale))
    t2 = run(ms2, ns2)
    ops = 2.0 * ms2 * wl.K * ns2
    threads = [d.get("num_threads", 1) for d in threadpool_info()
               if d.get("internal_api") in ("openblas", "mkl", "blis")]
    return {"value": ops / t2 / 1e12, "unit": "TOPS", "cores": max(threads) if threads else 1,
            "kind": "oracle",
            "sample": f"rows 0..{ms2 - 1} x output columns 0..{ns2 - 1} of {wl.name} "
                      f"(M={ms2}, K={wl.K}, N={ns2}; outlier mask from the sampled rows), "
                      f"{t2:.1f} s, numpy float64 BLAS"}


def bench_decode(binding, torch, inputs, steps: int) -> dict:
    wl = inputs.WORKLOADS["decode_8x4096"]
    wq_bytes = wl.N * wl.K
    copies = max(1, -(-2 * MALL_BYTES // wq_bytes))          # 32 for 16.8 MB weights
    _, _, Xd, weights = prepare(binding, torch, wl, inputs, copies)
    ws = binding.make_workspace(wl.M, wl.K, wl.N, MAX_OUTLIERS)
    Y = torch.empty((wl.M, wl.N), dtype=torch.float16, device="cuda")
    time_calls(binding, torch, Xd, weights, wl, copies * 2, ws, Y)       # warmup
    n = copies * max(4, steps)
    wall_ms, kern_ms, launches = time_calls(binding, torch, Xd, weights, wl, n, ws, Y)
    status, count = binding.read_status(ws)
    assert status == 0, f"decode status {status}"
    alg_bytes = wl.M * wl.K * 2 + wq_bytes + wl.N * 4 + wl.M * wl.N * 2
    per_call_ms = wall_ms / n
    kern_avg_ms = kern_ms / launches
    return {
        "workload": wl.name, "M": wl.M, "K": wl.K, "N": wl.N, "outlier_cols": count,
        "value": alg_bytes / (per_call_ms * 1e-3) / 1e9, "unit": "GB/s",
        "us_per_call": per_call_ms * 1e3, "weights_rotated": copies,
        "algorithmic_bytes_per_call": alg_bytes,
        "roofline": {"bound": "hbm", "achieved": alg_bytes / (kern_avg_ms * 1e-3) / 1e9,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": alg_bytes / (kern_avg_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                     "kernel": "k_decode", "kernel_avg_us": kern_avg_ms * 1e3},
    }


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="175b_layer_share")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path is single-GPU; see the sharding notes in DESIGN.md)", file=sys.stderr)
        return 2

    import torch

    from int8_mixed_precision_col_amd import binding, inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    binding.lib()
    wl = inputs.WORKLOADS[args.workload]
    if binding.is_decode(wl.M, wl.K):
        raise SystemExit(f"{wl.name} is a decode shape; the headline workload is a prefill one")
    log(f"workload {wl.name} M={wl.M} K={wl.K} N={wl.N}: drawing inputs")
    copies = max(1, -(-MALL_BYTES // (wl.N * wl.K)))
    X, W, Xd, weights = prepare(binding, torch, wl, inputs, copies)
    ws = binding.make_workspace(wl.M, wl.K, wl.N, MAX_OUTLIERS)
    Y = torch.empty((wl.M, wl.N), dtype=torch.float16, device="cuda")

    log(f"warmup {args.warmup}")
    time_calls(binding, torch, Xd, weights, wl, args.warmup, ws, Y)
    log(f"timing {args.steps} steps")
    wall_ms, kern_ms, launches = time_calls(binding, torch, Xd, weights, wl, args.steps, ws, Y)
    status, count = binding.read_status(ws)
    if status != 0 or not torch.isfinite(Y).all().item():
        raise SystemExit(f"bad result: status {status}")
    ms_per_step = wall_ms / args.steps
    ops = float(wl.flops)
    gemm_avg_ms = kern_ms / launches
    achieved = ops / (gemm_avg_ms * 1e-3) / 1e12
    log(f"{ms_per_step:.3f} ms/step, GEMM {gemm_avg_ms:.3f} ms avg over {launches} launches")

    result = {
        "metric": METRIC,
        "value": ops / (ms_per_step * 1e-3) / 1e12,
        "unit": "TOPS",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": wl.name, "M": wl.M, "K": wl.K, "N": wl.N,
                   "threshold": wl.threshold, "max_outliers": MAX_OUTLIERS,
                   "outlier_cols": count, "weights_rotated": copies,
                   "ops_per_step": ops},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_INT8_TOPS,
                     "unit": "TOP/s", "frac": achieved / PEAK_INT8_TOPS,
                     "traffic": load_traffic(wl.name, "gemm.hip"),
                     "kernel": "k_gemm", "kernel_avg_ms": gemm_avg_ms},
    }
    del Xd, weights, ws, Y
    torch.cuda.empty_cache()
    if not args.no_decode:
        log("decode workload")
        result["decode"] = bench_decode(binding, torch, inputs, 8)
    if not args.no_cpu_baseline:
        import oracle

        log("cpu baseline (oracle on a sample)")
        result["cpu_baseline"] = cpu_baseline(oracle, X, W, wl)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
