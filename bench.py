"""Benchmark of the mixed-precision int8 matmul on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one int8_mixed_matmul call (activation quantization: one pass over X for
the outlier columns, row constants and codes, then a fix-up with the outlier
gathers; int8 MFMA GEMM with the fp16 outlier product and dequant epilogue)
over the workload's synthetic inputs, which are resident in HBM; the weight is
converted to int8 once beforehand, as at checkpoint load. Prints ONE JSON line:
`value` is the prefill effective TOPS (2 M K N / time per call). The `roofline`
object is the GEMM kernel's own rate from HIP events recorded around its
launches during the timed steps; `kernels` splits a step into its kernels (a
separate pass with every kernel bracketed by events). The decode shape (8 tokens)
is measured in the same run as `decode` (GB/s of algorithmic bytes; 32 calls over
32 rotated weights captured in one HIP graph, per-call time from events around the
replays), next to a plain copy kernel of the same size. `configs` measures the
other workloads (16 x 1024 x 1024, the 6.7B-like and 13B-like FFN shapes) the same
way as the headline, and `vendor_int8_gemm` the vendor int8 GEMM on the headline
shape. `cpu_baseline` times the CPU oracle on a bounded row x column sample.
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
    print(f"[bench {time.time():.3f}] {msg}", file=sys.stderr, flush=True)


def source_digest(*names: str) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "int8_mixed_precision_col_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def array_digest(a: np.ndarray) -> str:
    """First 16 hex digits of the SHA-256 of an array's bytes (C order)."""
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()[:16]


KERNEL_SOURCES = {
    "k_gemm": ("gemm.hip", "gemm_kernel.hpp", "epilogue.hpp", "launch.hpp", "common.hpp"),
    "k_decode": ("decode.hip", "common.hpp"),
}
COPY_PROBE_BYTES = 1 << 30   # plain copy kernel of known size for counter scaling


def traffic_path(kernel: str, workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"{kernel}_hbm_traffic_{workload}.json")


def load_traffic(kernel: str, workload: str) -> float | None:
    """HBM bytes per launch from committed rocprofv3 counter runs, if the kernel's
    sources are unchanged since; else None."""
    path = traffic_path(kernel, workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256_16") != source_digest(*KERNEL_SOURCES[kernel]):
        return None
    return rec.get("hbm_bytes_per_launch")


def copy_probe(torch) -> None:
    """A plain elementwise kernel that reads and writes COPY_PROBE_BYTES once each
    (bitwise NOT of uint8): the reference for scaling FETCH_SIZE / WRITE_SIZE."""
    src = torch.zeros(COPY_PROBE_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.bitwise_not(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def _counter_rows(directory: str, counter: str):
    import csv
    import glob

    files = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {directory}")
    for fn in files:
        with open(fn) as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] == counter:
                    yield row["Kernel_Name"], float(row["Counter_Value"])


def summarize_traffic(fetch_dir: str, write_dir: str, workload: str, command: str) -> None:
    """Turn the FETCH_SIZE and WRITE_SIZE passes of a --traffic-probe run into
    profiles/<kernel>_hbm_traffic_<workload>.json for k_gemm (and k_decode, if seen)."""
    from int8_mixed_precision_col_amd import inputs

    def per_kernel(directory, counter):
        vals = {}
        for name, v in _counter_rows(directory, counter):
            vals.setdefault(name, []).append(v)
        return vals

    fetch = per_kernel(fetch_dir, "FETCH_SIZE")
    write = per_kernel(write_dir, "WRITE_SIZE")
    copy_name = next((n for n in fetch if "bitwise_not" in n), None)
    if copy_name is None:
        raise SystemExit("copy probe kernel not found; kernels seen: " + "; ".join(fetch))
    copy_kib = COPY_PROBE_BYTES / 1024.0

    def probe_mean(vals):
        # the probe's launches are the 1 GiB ones; the same elementwise kernel also runs on
        # small buffers elsewhere in the run (the decode leg's copy floor)
        big = [v for v in vals if v >= 0.5 * max(vals)]
        return sum(big) / len(big)

    f_scale = copy_kib / probe_mean(fetch[copy_name])
    w_scale = copy_kib / probe_mean(write[copy_name])
    plans = {"k_gemm": (workload, None), "k_decode": ("decode_8x4096", None)}
    for kernel, (wl_name, _) in plans.items():
        names = [n for n in fetch if f"i8mm::{kernel}<" in n]
        if not names:
            continue
        fv = [v for n in names for v in fetch[n]]
        wv = [v for n in names for v in write.get(n, [])]
        f_kib, w_kib = sum(fv) / len(fv), sum(wv) / len(wv)
        wl = inputs.WORKLOADS[wl_name]
        rec = {
            "kernel": kernel, "kernel_names": names, "workload": wl_name,
            "kernel_source_sha256_16": source_digest(*KERNEL_SOURCES[kernel]),
            "launches": len(fv),
            "fetch_kib_per_launch_raw": f_kib, "write_kib_per_launch_raw": w_kib,
            "copy_probe_bytes": COPY_PROBE_BYTES, "copy_probe_kernel": copy_name,
            "fetch_scale": f_scale, "write_scale": w_scale,
            "hbm_bytes_per_launch": (f_kib * f_scale + w_kib * w_scale) * 1024.0,
            "algorithmic_bytes_per_launch": wl.M * wl.K + wl.N * wl.K + wl.M * wl.N * 2
            if kernel == "k_gemm" else wl.M * wl.K * 2 + wl.N * wl.K + wl.N * 4 + wl.M * wl.N * 2,
            "command": command,
        }
        with open(traffic_path(kernel, wl_name), "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        print(json.dumps(rec))


def prepare(binding, torch, wl, inputs, copies: int, time_prepare: bool = False):
    """Draw the workload, move it to the GPU, convert `copies` weights (untimed by the
    step clock). With time_prepare, the conversion is also run 3 more times between
    events and its rate returned (checkpoint-load path)."""
    X, _ = inputs.make_x(wl)
    W = inputs.make_w(wl)
    Xd = torch.from_numpy(X).cuda()
    Wd = torch.from_numpy(W).cuda()
    weights = [binding.prepare_weight(Wd)]
    prep = None
    if time_prepare:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(3):
            binding.prepare_weight(Wd)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 3
        nbytes = wl.K * wl.N * 2 + wl.K * wl.N + wl.N * 4   # read W once, write Wq and a_w
        gbs = nbytes / (ms * 1e-3) / 1e9
        prep = {"ms": ms, "algorithmic_bytes": nbytes, "GB/s": gbs,
                "frac_of_hbm_peak": gbs / PEAK_HBM_GBS,
                "note": "two passes over W (column absmax, then quantize + transpose)"}
    for _ in range(copies - 1):
        Wq, aw = weights[0]
        weights.append((Wq.clone(), aw.clone()))
    del Wd
    torch.cuda.synchronize()
    return X, W, Xd, weights, prep


def time_calls(binding, torch, Xd, weights, wl, n_calls: int, ws, Y, mode: int = 1):
    """n_calls int8_mixed_matmul calls over the rotated weights, bracketed by device
    synchronisations. mode 1: the library's events bracket each call's main kernels; mode
    2: also the two activation quantization phases. Returns (wall ms, {phase: (ms,
    bracketed calls)})."""
    binding.timing_read_phases()
    binding.timing_enable(mode)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n_calls):
        Wq, aw = weights[i % len(weights)]
        binding.mixed_matmul(Xd, Wq, aw, wl.threshold, MAX_OUTLIERS, workspace=ws, out=Y)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    binding.timing_enable(0)
    return (t1 - t0) * 1e3, binding.timing_read_phases()


def phase_breakdown(phases: dict, n_calls: int, wall_ms: float) -> dict:
    """Per-phase time per call (us) and its share of the call, from a mode-2 timing pass
    (every phase bracketed by events) whose own wall time is wall_ms. Phases: the pass
    over X (one kernel), the fix-up (two kernels), the main kernels (the GEMM, two
    launches when a partial last wave of tiles is split off)."""
    out = {"pass_ms_per_call": wall_ms / n_calls}
    for name, (ms, n) in phases.items():
        if n:
            us = ms / n_calls * 1e3
            out[name] = {"us_per_call": us, "share_of_call": ms / wall_ms}
    return out


def cpu_baseline(oracle, X, W, wl, budget_s: float = 15.0) -> dict:
    """The oracle as it stands, on all rows of the workload x a sample of output columns.

    Two short calls (256 and 1024 columns) fit time = fixed + per-column cost; the
    reported call takes about 80% of the budget. Its weight columns are converted
    untimed, as at load time (the conversion is per column, so the slice of one
    conversion is the conversion of the slice).
    """
    from threadpoolctl import threadpool_info

    ms = wl.M

    def run(Wq, aw, ns):
        t0 = time.perf_counter()
        oracle.mixed_matmul(X[:ms], np.ascontiguousarray(Wq[:ns]), aw[:ns], wl.threshold)
        return time.perf_counter() - t0

    n1, n2 = min(wl.N, 256), min(wl.N, 1024)
    Wq, aw = oracle.prepare_weight(np.ascontiguousarray(W[:, :n2]))
    t1, t2 = run(Wq, aw, n1), run(Wq, aw, n2)
    per_col = max((t2 - t1) / max(n2 - n1, 1), 1e-9)
    ns = int(min(wl.N, max(n2, (0.8 * budget_s - max(t1 - per_col * n1, 0.0)) / per_col)))
    ns = max(16, ns // 16 * 16)
    if ns > n2:
        Wq, aw = oracle.prepare_weight(np.ascontiguousarray(W[:, :ns]))
    t = run(Wq, aw, ns)
    ops = 2.0 * ms * wl.K * ns
    threads = [d.get("num_threads", 1) for d in threadpool_info()
               if d.get("internal_api") in ("openblas", "mkl", "blis")]
    blas = max(threads) if threads else 1
    cores = len(os.sched_getaffinity(0))
    return {"value": ops / t / 1e12, "unit": "TOPS", "cores": cores, "blas_threads": blas,
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"all {ms} rows x output columns 0..{ns - 1} of {wl.name} "
                      f"(M={ms}, K={wl.K}, N={ns}), {t:.1f} s for one oracle call "
                      f"(numpy float64; the BLAS product on {blas} threads, the elementwise "
                      f"steps on one; {cores} cores in the process's affinity set)"}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def bench_config(binding, torch, inputs, name: str, calls: int = 20, warmup: int = 3) -> dict:
    """One workload end to end: wall time per int8_mixed_matmul call over weights rotated to
    defeat the last-level cache (hook off), then a pass with every kernel of the call
    bracketed by events for the per-kernel breakdown."""
    wl = inputs.WORKLOADS[name]
    copies = max(1, -(-MALL_BYTES // (wl.N * wl.K)))
    _, _, Xd, weights, _ = prepare(binding, torch, wl, inputs, copies)
    ws = binding.make_workspace(wl.M, wl.K, wl.N, MAX_OUTLIERS)
    Y = torch.empty((wl.M, wl.N), dtype=torch.float16, device="cuda")
    # warm up for ~60 ms of calls: after an idle GPU the board's power control lets the
    # first launches run fast and then slow, settling over tens of milliseconds
    est, _ = time_calls(binding, torch, Xd, weights, wl, 2, ws, Y, mode=0)
    warm = max(warmup, int(60.0 / max(est / 2, 1e-3)))
    time_calls(binding, torch, Xd, weights, wl, warm, ws, Y, mode=0)
    wall_ms, _ = time_calls(binding, torch, Xd, weights, wl, calls, ws, Y, mode=0)
    ms = wall_ms / calls
    time_calls(binding, torch, Xd, weights, wl, max(warmup, warm // 4), ws, Y, mode=0)
    wall2, phases = time_calls(binding, torch, Xd, weights, wl, calls, ws, Y, mode=2)
    status, count = binding.read_status(ws)
    assert status == 0 and torch.isfinite(Y).all().item(), f"{name}: bad result (status {status})"
    decode = binding.is_decode(wl.M, wl.K)
    main_ms, main_n = phases["main"]
    main_ms /= max(main_n, 1)
    ops = float(wl.flops)
    res = {"workload": wl.name, "M": wl.M, "K": wl.K, "N": wl.N, "outlier_cols": count,
           "path": "decode kernel" if decode else "activation quantization (pass over X, fix-up) + GEMM",
           "weights_rotated": copies, "calls": calls, "warmup_calls": warm,
           "ms_per_call": ms, "TOPS": ops / (ms * 1e-3) / 1e12,
           "kernels": phase_breakdown(phases, calls, wall2),
           "main_kernel": {"ms": main_ms, "TOPS": ops / (main_ms * 1e-3) / 1e12,
                           "frac_of_int8_peak": ops / (main_ms * 1e-3) / 1e12 / PEAK_INT8_TOPS}}
    if decode:
        alg = wl.M * wl.K * 2 + wl.N * wl.K + wl.N * 4 + wl.M * wl.N * 2
        res["main_kernel"]["GB/s"] = alg / (main_ms * 1e-3) / 1e9
        res["main_kernel"]["frac_of_hbm_peak"] = res["main_kernel"]["GB/s"] / PEAK_HBM_GBS
        # the same calls captured in one HIP graph, as for the decode line: per call without
        # the host's launch overhead
        g_us = graph_per_call_us(binding, torch, Xd, weights, wl, ws, Y)
        res["graph"] = {"us_per_call": g_us, "GB/s": alg / (g_us * 1e-6) / 1e9,
                        "frac_of_hbm_peak": alg / (g_us * 1e-6) / 1e9 / PEAK_HBM_GBS,
                        "note": f"{len(weights)} calls over the rotated weights in one graph"}
    del Xd, weights, ws, Y
    torch.cuda.empty_cache()
    return res


def graph_per_call_us(binding, torch, Xd, weights, wl, ws, Y, reps: int = 20) -> float:
    """int8_mixed_matmul once per prepared weight, captured in one HIP graph and replayed
    reps times between events; per-call time = replay time / calls. The last output is
    checked against an eager call on the same weight."""
    Y_ref = binding.mixed_matmul(Xd, *weights[-1], wl.threshold, MAX_OUTLIERS, workspace=ws).clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for Wq, aw in weights[:2]:
            binding.mixed_matmul(Xd, Wq, aw, wl.threshold, MAX_OUTLIERS, workspace=ws, out=Y)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for Wq, aw in weights:
            binding.mixed_matmul(Xd, Wq, aw, wl.threshold, MAX_OUTLIERS, workspace=ws, out=Y)
    for _ in range(3):
        graph.replay()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    assert torch.equal(Y, Y_ref), "graph replay differs from the eager call"
    return e0.elapsed_time(e1) / (reps * len(weights)) * 1e3


def measured_copy_floor(torch, nbytes: int = 8 << 20, copies: int = 32, reps: int = 20) -> dict:
    """A plain elementwise kernel (bitwise NOT of uint8: reads and writes nbytes, 16 MiB
    moved in all, about what one decode call reads) over rotated buffers, captured like the
    decode calls: what one launch moving that much achieves on this GPU, for comparison
    with the decode kernel."""
    src = [torch.zeros(nbytes, dtype=torch.uint8, device="cuda") for _ in range(copies)]
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    for s in src[:2]:
        torch.bitwise_not(s, out=dst)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for s in src:
            torch.bitwise_not(s, out=dst)
    for _ in range(3):
        g.replay()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / (reps * copies) * 1e3
    del src, dst
    torch.cuda.empty_cache()
    gbs = 2 * nbytes / (us * 1e-6) / 1e9
    return {"kernel": "torch bitwise_not (uint8)", "bytes_read": nbytes, "bytes_written": nbytes,
            "us_per_call": us, "GB/s": gbs, "frac_of_hbm_peak": gbs / PEAK_HBM_GBS}


def vendor_int8_gemm(torch, M: int, K: int, N: int, reps: int = 5) -> dict | None:
    """The vendor int8 GEMM (torch._int_mm, int32 output) on the same shape, without any
    of the decomposition: a measured reference for the MFMA GEMM."""
    try:
        A = torch.randint(-127, 128, (M, K), dtype=torch.int8, device="cuda")
        B = torch.randint(-127, 128, (N, K), dtype=torch.int8, device="cuda").t()
        torch._int_mm(A, B)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            torch._int_mm(A, B)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        del A, B
        torch.cuda.empty_cache()
        return {"op": "torch._int_mm (int8 x int8 -> int32)", "ms": ms,
                "TOPS": 2.0 * M * K * N / (ms * 1e-3) / 1e12}
    except (RuntimeError, AttributeError) as e:  # not every build has a kernel for it
        return {"op": "torch._int_mm", "error": str(e)[:200]}


def bench_projections(binding, torch, inputs, reps: int = 10) -> dict:
    """Three projections of one input (Q, K, V: 2048 x 4096 times three 4096 x 4096
    weights, drawn like opt6.7b_ffn_up): three int8_mixed_matmul calls, one
    activation quantization + three int8_mixed_matmul_q calls, and one quantization +
    one grouped launch. Each alone is 128 tiles of 256 x 256 for 256 CUs."""
    wl = inputs.WORKLOADS["opt6.7b_ffn_up"]
    X, _ = inputs.make_x(wl)
    W = inputs.make_w(wl)
    Xd = torch.from_numpy(X).cuda()
    weights = [binding.prepare_weight(torch.from_numpy(np.ascontiguousarray(W[:, q * 4096:(q + 1) * 4096])).cuda())
               for q in range(3)]
    ws = binding.make_workspace(wl.M, wl.K, 4096, MAX_OUTLIERS)
    outs = [torch.empty((wl.M, 4096), dtype=torch.float16, device="cuda") for _ in range(3)]
    ops = 3 * 2.0 * wl.M * wl.K * 4096

    def separate():
        for (Wq, aw), Y in zip(weights, outs):
            binding.mixed_matmul(Xd, Wq, aw, wl.threshold, MAX_OUTLIERS, workspace=ws, out=Y)

    def quantize_once():
        st = binding.QuantizedActivations(Xd, wl.threshold, MAX_OUTLIERS)
        for (Wq, aw), Y in zip(weights, outs):
            st.matmul(Wq, aw, out=Y)

    def grouped():
        st = binding.QuantizedActivations(Xd, wl.threshold, MAX_OUTLIERS)
        st.matmul_grouped(weights, outs=outs)

    res = {"workload": "opt6.7b qkv: M=2048 K=4096 N=3x4096", "unit": "TOPS"}
    for name, fn in (("three_calls", separate), ("quantize_once", quantize_once),
                     ("grouped_launch", grouped)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        res[name] = {"ms": ms, "TOPS": ops / (ms * 1e-3) / 1e12}
    return res


def bench_decode(binding, torch, inputs, reps: int) -> dict:
    """Decode shape: 32 calls over 32 distinct prepared weights (2x the MALL) captured
    in one HIP graph, as a decode step walks the layers; per-call time = replay time /
    32, from events on the replay stream. The graph's last output is checked against
    an eager call on the same weight."""
    wl = inputs.WORKLOADS["decode_8x4096"]
    wq_bytes = wl.N * wl.K
    copies = max(1, -(-2 * MALL_BYTES // wq_bytes))          # 32 for 16.8 MB weights
    _, _, Xd, weights, _ = prepare(binding, torch, wl, inputs, copies)
    ws = binding.make_workspace(wl.M, wl.K, wl.N, MAX_OUTLIERS)
    Y = torch.empty((wl.M, wl.N), dtype=torch.float16, device="cuda")
    # eager: per-launch kernel time from the library's event hook, for context
    time_calls(binding, torch, Xd, weights, wl, copies * 2, ws, Y)
    wall_ms, phases = time_calls(binding, torch, Xd, weights, wl, copies * 4, ws, Y)
    eager_us = wall_ms / (copies * 4) * 1e3
    hook_us = phases["main"][0] / phases["main"][1] * 1e3
    status, count = binding.read_status(ws)
    assert status == 0, f"decode status {status}"
    Y_ref = binding.mixed_matmul(Xd, *weights[-1], wl.threshold, MAX_OUTLIERS, workspace=ws).clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for Wq, aw in weights[:2]:
            binding.mixed_matmul(Xd, Wq, aw, wl.threshold, MAX_OUTLIERS, workspace=ws, out=Y)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for Wq, aw in weights:
            binding.mixed_matmul(Xd, Wq, aw, wl.threshold, MAX_OUTLIERS, workspace=ws, out=Y)
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    assert torch.equal(Y, Y_ref), "graph replay differs from the eager call"
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    assert torch.equal(Y, Y_ref), "graph replay differs from the eager call"
    per_call_us = e0.elapsed_time(e1) / (reps * copies) * 1e3
    alg_bytes = wl.M * wl.K * 2 + wq_bytes + wl.N * 4 + wl.M * wl.N * 2
    gbs = alg_bytes / (per_call_us * 1e-6) / 1e9

    # the weight-only variant (no activation quantization, no decomposition) on the
    # same 32 weights, the same way: what the decomposition costs at this shape
    Yw = torch.empty_like(Y)
    with torch.cuda.stream(side):
        for Wq, aw in weights[:2]:
            binding.weight_only_matmul(Xd, Wq, aw, out=Yw)
    torch.cuda.current_stream().wait_stream(side)
    gw = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gw):
        for Wq, aw in weights:
            binding.weight_only_matmul(Xd, Wq, aw, out=Yw)
    for _ in range(3):
        gw.replay()
    e0.record()
    for _ in range(reps):
        gw.replay()
    e1.record()
    torch.cuda.synchronize()
    wo_us = e0.elapsed_time(e1) / (reps * copies) * 1e3

    # the same product in separate launches: quantize X once per call (one pass over X,
    # then the fix-up), then the weight-stream GEMM (int8_mixed_matmul_q), same graph
    # scheme: what the single decode launch saves
    import ctypes

    L = binding.lib()
    nb = int(L.int8_quant_state_bytes(wl.M, wl.K, MAX_OUTLIERS))
    state = torch.empty((nb,), dtype=torch.uint8, device="cuda")
    qws = torch.empty((int(L.int8_mixed_matmul_q_workspace_bytes(wl.N, MAX_OUTLIERS)),),
                      dtype=torch.uint8, device="cuda")
    Yq = torch.empty_like(Y)

    def two_launch(Wq, aw):
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        rc = L.int8_quantize_activations(Xd.data_ptr(), wl.M, wl.K, wl.threshold, MAX_OUTLIERS,
                                         state.data_ptr(), nb, st)
        rc = rc or L.int8_mixed_matmul_q(state.data_ptr(), wl.M, wl.K, MAX_OUTLIERS, Wq.data_ptr(),
                                         aw.data_ptr(), wl.N, Yq.data_ptr(), qws.data_ptr(),
                                         qws.numel(), None, st)
        assert rc == 0, f"quantize + GEMM: status {rc}"

    with torch.cuda.stream(side):
        for Wq, aw in weights[:2]:
            two_launch(Wq, aw)
    torch.cuda.current_stream().wait_stream(side)
    gq = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gq):
        for Wq, aw in weights:
            two_launch(Wq, aw)
    for _ in range(3):
        gq.replay()
    e0.record()
    for _ in range(reps):
        gq.replay()
    e1.record()
    torch.cuda.synchronize()
    tl_us = e0.elapsed_time(e1) / (reps * copies) * 1e3
    return {
        "workload": wl.name, "M": wl.M, "K": wl.K, "N": wl.N, "outlier_cols": count,
        "value": gbs, "unit": "GB/s", "us_per_call": per_call_us,
        "weights_rotated": copies, "graph_replays": reps,
        "algorithmic_bytes_per_call": alg_bytes,
        "eager_us_per_call": eager_us, "eager_kernel_us_hook": hook_us,
        "quantize_then_gemm": {"us_per_call": tl_us,
                               "note": "int8_quantize_activations + int8_mixed_matmul_q per "
                                       "call (4 kernels), same graph scheme"},
        "weight_only": {"us_per_call": wo_us,
                        "GB/s": alg_bytes / (wo_us * 1e-6) / 1e9,
                        "frac_of_hbm_peak": alg_bytes / (wo_us * 1e-6) / 1e9 / PEAK_HBM_GBS,
                        "kernel": "k_weight_only"},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": gbs / PEAK_HBM_GBS,
                     "traffic": load_traffic("k_decode", wl.name),
                     "kernel": "k_decode",
                     "time_basis": "per call of a captured graph of 32 calls (the gap between "
                                   "launches included)",
                     "per_call_us": per_call_us,
                     "measured_floor": measured_copy_floor(torch)},
    }


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="175b_layer_share")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the tiny / 6.7B / 13B workloads and the vendor GEMM reference")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="run the copy probe, then the steps, and print no JSON (for --pmc runs)")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/*_hbm_traffic_*.json from two --pmc output dirs")
    ap.add_argument("--command", default="", help="command line recorded by --summarize-traffic")
    args = ap.parse_args()
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic, args.workload, args.command)
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: the "
              "library runs on one GPU (several GPUs would split the weight's output "
              "columns, with no exchange needed before the matmul)", file=sys.stderr)
        return 2

    import torch

    from int8_mixed_precision_col_amd import binding, inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    binding.lib()
    if args.traffic_probe:
        copy_probe(torch)
    wl = inputs.WORKLOADS[args.workload]
    if binding.is_decode(wl.M, wl.K):
        raise SystemExit(f"{wl.name} is a decode shape; the headline workload is a prefill one")
    log(f"workload {wl.name} M={wl.M} K={wl.K} N={wl.N}: drawing inputs")
    copies = max(1, -(-MALL_BYTES // (wl.N * wl.K)))
    X, W, Xd, weights, prep = prepare(binding, torch, wl, inputs, copies, time_prepare=True)
    ws = binding.make_workspace(wl.M, wl.K, wl.N, MAX_OUTLIERS)
    Y = torch.empty((wl.M, wl.N), dtype=torch.float16, device="cuda")

    log(f"warmup {args.warmup}")
    time_calls(binding, torch, Xd, weights, wl, args.warmup, ws, Y)
    log(f"timing {args.steps} steps")
    wall_ms, phases = time_calls(binding, torch, Xd, weights, wl, args.steps, ws, Y)
    kern_ms, launches = phases["main"]
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
                     "traffic": load_traffic("k_gemm", wl.name),
                     "kernel": "k_gemm", "kernel_avg_ms": gemm_avg_ms},
    }
    # per-kernel breakdown of the step, in a pass of its own (every kernel bracketed),
    # after 10 untimed calls: the host checks above leave the GPU idle for ~0.2 s, and the
    # board's power control then lets the next launch run fast and the following ones
    # slow, settling over about 15 launches
    n2 = max(3, args.steps // 4)
    time_calls(binding, torch, Xd, weights, wl, 10, ws, Y, mode=0)
    wall2, ph2 = time_calls(binding, torch, Xd, weights, wl, n2, ws, Y, mode=2)
    result["kernels"] = phase_breakdown(ph2, n2, wall2)
    result["prepare_weight"] = prep
    # the GPU path and the CPU baseline below read these same host arrays
    result["inputs_sha256_16"] = {"X_fp16": array_digest(X), "W_fp16": array_digest(W)}
    del Xd, weights, ws, Y
    torch.cuda.empty_cache()
    if not args.no_decode:
        log("decode workload")
        result["decode"] = bench_decode(binding, torch, inputs, 20)
    if args.traffic_probe:
        log("traffic probe done")
        return 0
    if not args.no_decode:
        log("projections sharing one input")
        result["projections_qkv"] = bench_projections(binding, torch, inputs)
    if not args.no_configs:
        result["configs"] = {}
        for name in ("tiny", "opt6.7b_ffn_up", "13b_ffn_down"):
            log(f"config {name}")
            result["configs"][name] = bench_config(binding, torch, inputs, name)
        log("vendor int8 GEMM on the headline shape")
        result["vendor_int8_gemm"] = vendor_int8_gemm(torch, wl.M, wl.K, wl.N)
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
