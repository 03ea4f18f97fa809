"""Shared helpers of the GPU parity tests (no method arithmetic here)."""

import numpy as np
import torch

# fp16 output tolerance: max |Y - Y_oracle| <= TOL * max |Y_oracle|
TOL = 1e-2


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def announce(msg: str) -> None:
    print(f"\n[gpu case] {msg}", flush=True)


def check_y(y_gpu: np.ndarray, y_ref: np.ndarray, tol: float = TOL) -> float:
    yg = y_gpu.astype(np.float64)
    yr = y_ref.astype(np.float64)
    assert yg.shape == yr.shape
    assert np.all(np.isfinite(yg)), "non-finite output"
    scale = np.abs(yr).max()
    err = np.abs(yg - yr).max()
    assert err <= tol * scale, f"max err {err} > {tol} * {scale}"
    return err / scale if scale else 0.0


def grid_weight(rng, K, N):
    """fp16 W whose int8 conversion is lossless: columns q * 2**-e, |q| <= 127, one |q| = 127."""
    q = rng.integers(-127, 128, size=(K, N))
    q[rng.integers(0, K, size=N), np.arange(N)] = 127 * rng.choice([-1, 1], size=N)
    e = rng.integers(5, 9, size=N)
    return (q * 2.0 ** (-e[None, :].astype(np.float64))).astype(np.float16)
