"""ctypes binding of libint8mm.so (declared in include/int8mm.h).

Argument marshalling only: torch allocates device memory and supplies the
current HIP stream; every step of the computation runs in the library's HIP
kernels. There is no CPU fallback: if the library is missing or fails to load,
every call raises.
"""

from __future__ import annotations

import ctypes
import functools
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libint8mm.so")

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int
_f32 = ctypes.c_float

# name -> (restype, argtypes); exactly the symbols include/int8mm.h declares
SIGNATURES = {
    "int8_prepare_weight": (_int, [_p, _i64, _i64, _int, _p, _p, _p]),
    "int8_tile_weight": (_int, [_p, _i64, _i64, _p, _p]),
    "int8_quant_rows": (_int, [_p, _i64, _i64, _f32, _p, _p, _p, _p, _p, _i64, _p]),
    "int8_prepared_weight_bytes": (ctypes.c_size_t, [_i64, _i64]),
    "int8_mixed_matmul_workspace_bytes": (ctypes.c_size_t, [_i64, _i64, _i64, _i64]),
    "int8_mixed_matmul": (_int, [_p, _i64, _i64, _p, _p, _i64, _f32, _i64, _p, _p,
                                 ctypes.c_size_t, _p, _p]),
    "int8_mixed_matmul_noalloc": (_int, [_p, _i64, _i64, _p, _p, _i64, _f32, _i64, _p, _p, _p]),
    "int8_mixed_matmul_is_decode": (_int, [_i64, _i64]),
    "int8_weight_only_matmul": (_int, [_p, _i64, _i64, _p, _p, _i64, _p, _p]),
    "int8_quant_state_bytes": (ctypes.c_size_t, [_i64, _i64, _i64]),
    "int8_quant_state_layout": (ctypes.c_int, [_i64, _i64, _i64, ctypes.POINTER(_i64)]),
    "int8_quantize_activations": (_int, [_p, _i64, _i64, _f32, _i64, _p, ctypes.c_size_t, _p]),
    "int8_mixed_matmul_q_workspace_bytes": (ctypes.c_size_t, [_i64, _i64]),
    "int8_mixed_matmul_q": (_int, [_p, _i64, _i64, _i64, _p, _p, _i64, _p, _p, ctypes.c_size_t,
                                   _p, _p]),
    "int8_mixed_matmul_q_grouped_workspace_bytes": (ctypes.c_size_t, [_i64, _p, _i64]),
    "int8_mixed_matmul_q_grouped": (_int, [_p, _i64, _i64, _i64, _i64, _p, _p, _p, _p, _p,
                                           ctypes.c_size_t, _p]),
    "int8mm_read_status": (_int, [_p, _p, _p]),
    "int8mm_strerror": (ctypes.c_char_p, [_int]),
    "int8mm_timing_enable": (_int, [_int]),
    "int8mm_timing_read": (_int, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_i64)]),
    "int8mm_timing_read_phases": (_int, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_i64)]),
}

STATUS = {0: "OK", 1: "E_NULL", 2: "E_SHAPE", 3: "E_ALIGN", 4: "E_THRESHOLD",
          5: "E_WORKSPACE", 6: "E_HIP", 7: "E_TOO_MANY_OUTLIERS", 8: "E_SCRATCH"}

_lib = None


class Int8mmError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: int8mm status {code} ({STATUS.get(code, '?')}): "
                         f"{strerror(code)}")


def lib() -> ctypes.CDLL:
    """Load libint8mm.so (built in-tree by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                               "(python -m int8_mixed_precision_col_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().int8mm_strerror(code).decode()


@functools.lru_cache(maxsize=256)
def _prepared_bytes(K: int, N: int) -> int:
    """Size of a prepared weight (asked of the library once per shape)."""
    return int(lib().int8_prepared_weight_bytes(K, N))


def _check(rc: int, where: str) -> None:
    if rc != 0:
        raise Int8mmError(rc, where)


def _stream(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _on_device(t: torch.Tensor) -> bool:
    """True for a tensor in HIP device memory (the only memory the library takes)."""
    return t.is_cuda


def _need(t: torch.Tensor, dtype: torch.dtype, name: str) -> None:
    if not isinstance(t, torch.Tensor) or not _on_device(t):
        raise ValueError(f"{name} must be a HIP device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _need_shape(t: torch.Tensor, dtype: torch.dtype, shape: tuple, device, name: str) -> None:
    """A caller-supplied buffer the kernels write in full: dtype, contiguity, exact shape
    and device are checked before any library call, since the kernels trust them."""
    _need(t, dtype, name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the inputs on {device}")


def _need_matrix(X: torch.Tensor, name: str = "X") -> tuple:
    _need(X, torch.float16, name)
    if X.dim() != 2:
        raise ValueError(f"{name} must be 2-D [M, K], got shape {tuple(X.shape)}")
    return tuple(X.shape)


def _need_weight(Wq: torch.Tensor, a_w: torch.Tensor, K: int, device) -> int:
    """(Wq, a_w) of a prepared weight for K input features; returns N."""
    _need(Wq, torch.int8, "Wq")
    _need(a_w, torch.float32, "a_w")
    if a_w.dim() != 1:
        raise ValueError(f"a_w must be 1-D [N], got shape {tuple(a_w.shape)}")
    N = a_w.shape[0]
    if Wq.numel() != _prepared_bytes(K, N):
        raise ValueError(f"Wq holds {Wq.numel()} bytes; a prepared weight for K={K}, N={N} "
                         f"holds {_prepared_bytes(K, N)}")
    if Wq.device != device or a_w.device != device:
        raise ValueError(f"Wq and a_w must be on {device}")
    return N


def prepare_weight(W: torch.Tensor, layout: int = 0):
    """fp16 W ([K, N] for layout 0, [N, K] for layout 1) -> (Wq, a_w fp32 [N]).

    Wq is the unit-tiled int8 weight the kernels read (include/int8mm.h): a tensor of
    shape (N // 16, ceil(K / 64), 16, 64); untile_weight(Wq, K) gives the [N, K] view.
    """
    _need_matrix(W, "W")
    K, N = (W.shape[0], W.shape[1]) if layout == 0 else (W.shape[1], W.shape[0])
    ks = (K + 63) // 64
    if N % 16:
        raise ValueError("N must be a multiple of 16")
    Wq = torch.empty((N // 16, ks, 16, 64), dtype=torch.int8, device=W.device)
    a_w = torch.empty((N,), dtype=torch.float32, device=W.device)
    _check(lib().int8_prepare_weight(W.data_ptr(), K, N, layout, Wq.data_ptr(), a_w.data_ptr(),
                                     _stream(W)), "int8_prepare_weight")
    return Wq, a_w


def tile_weight(Wq_nk: torch.Tensor) -> torch.Tensor:
    """An already-quantized int8 weight [N, K] (row-major) -> the unit-tiled tensor the
    matmul calls take, (N // 16, ceil(K / 64), 16, 64); pair it with the weight's own fp32
    column constants [N]. Layout only (int8_tile_weight)."""
    _need(Wq_nk, torch.int8, "Wq_nk")
    if Wq_nk.dim() != 2:
        raise ValueError(f"Wq_nk must be 2-D [N, K], got shape {tuple(Wq_nk.shape)}")
    N, K = Wq_nk.shape
    if N % 16 or K % 16:
        raise ValueError("N and K must be multiples of 16")
    Wq = torch.empty((N // 16, (K + 63) // 64, 16, 64), dtype=torch.int8, device=Wq_nk.device)
    _check(lib().int8_tile_weight(Wq_nk.data_ptr(), K, N, Wq.data_ptr(), _stream(Wq_nk)),
           "int8_tile_weight")
    return Wq


def untile_weight(Wq: torch.Tensor, K: int) -> torch.Tensor:
    """The [N, K] int8 matrix held in a unit-tiled weight (a copy; layout only)."""
    g, ks = Wq.shape[0], Wq.shape[1]
    return Wq.permute(0, 2, 1, 3).reshape(g * 16, ks * 64)[:, :K].contiguous()


def quant_rows(X: torch.Tensor, threshold: float, max_outliers: int = 256) -> dict:
    """Outlier columns + row quantization of fp16 X [M, K] (see include/int8mm.h)."""
    M, K = _need_matrix(X)
    dev = X.device
    out = {
        "Xq": torch.empty((M, K), dtype=torch.int8, device=dev),
        "a_x": torch.empty((M,), dtype=torch.float32, device=dev),
        "mask": torch.empty(((K + 31) // 32,), dtype=torch.int32, device=dev),
        "idx": torch.empty((max(max_outliers, 1),), dtype=torch.int32, device=dev),
        "count": torch.empty((4,), dtype=torch.int32, device=dev),
    }
    _check(lib().int8_quant_rows(X.data_ptr(), M, K, float(threshold), out["Xq"].data_ptr(),
                                 out["a_x"].data_ptr(), out["mask"].data_ptr(),
                                 out["idx"].data_ptr() if max_outliers > 0 else None,
                                 out["count"].data_ptr(), max_outliers, _stream(X)),
           "int8_quant_rows")
    return out


def workspace_bytes(M: int, K: int, N: int, max_outliers: int = 256) -> int:
    return int(lib().int8_mixed_matmul_workspace_bytes(M, K, N, max_outliers))


def is_decode(M: int, K: int) -> bool:
    return bool(lib().int8_mixed_matmul_is_decode(M, K))


def make_workspace(M: int, K: int, N: int, max_outliers: int = 256, device="cuda") -> torch.Tensor:
    nbytes = workspace_bytes(M, K, N, max_outliers)
    if nbytes == 0:
        raise ValueError(f"bad shape for int8_mixed_matmul: M={M} K={K} N={N} "
                         f"max_outliers={max_outliers}")
    return torch.empty((nbytes,), dtype=torch.uint8, device=device)


def mixed_matmul(X: torch.Tensor, Wq: torch.Tensor, a_w: torch.Tensor, threshold: float = 6.0,
                 max_outliers: int = 256, workspace: torch.Tensor | None = None,
                 out: torch.Tensor | None = None, acc_out: torch.Tensor | None = None):
    """Y fp16 [M, N] = the decomposed product of X [M, K] and the prepared weight (Wq, a_w)."""
    M, K = _need_matrix(X)
    N = _need_weight(Wq, a_w, K, X.device)
    if out is not None:
        _need_shape(out, torch.float16, (M, N), X.device, "out")
    if acc_out is not None:
        _need_shape(acc_out, torch.int32, (M, N), X.device, "acc_out")
    if workspace is None:
        workspace = make_workspace(M, K, N, max_outliers, X.device)
    _need(workspace, torch.uint8, "workspace")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=X.device)
    _check(lib().int8_mixed_matmul(X.data_ptr(), M, K, Wq.data_ptr(), a_w.data_ptr(), N,
                                   float(threshold), max_outliers, out.data_ptr(),
                                   workspace.data_ptr(), workspace.numel(),
                                   acc_out.data_ptr() if acc_out is not None else None,
                                   _stream(X)), "int8_mixed_matmul")
    return out


def mixed_matmul_noalloc(X: torch.Tensor, Wq: torch.Tensor, a_w: torch.Tensor,
                         threshold: float = 6.0, max_outliers: int = 256,
                         out: torch.Tensor | None = None,
                         acc_out: torch.Tensor | None = None) -> torch.Tensor:
    """mixed_matmul through int8_mixed_matmul_noalloc: the library's fixed per-GPU
    scratch instead of a workspace (nothing is allocated by the call; `out` is
    allocated here only when not given)."""
    M, K = _need_matrix(X)
    N = _need_weight(Wq, a_w, K, X.device)
    if out is not None:
        _need_shape(out, torch.float16, (M, N), X.device, "out")
    if acc_out is not None:
        _need_shape(acc_out, torch.int32, (M, N), X.device, "acc_out")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=X.device)
    _check(lib().int8_mixed_matmul_noalloc(X.data_ptr(), M, K, Wq.data_ptr(), a_w.data_ptr(), N,
                                           float(threshold), max_outliers, out.data_ptr(),
                                           acc_out.data_ptr() if acc_out is not None else None,
                                           _stream(X)), "int8_mixed_matmul_noalloc")
    return out


def weight_only_matmul(X: torch.Tensor, Wq: torch.Tensor, a_w: torch.Tensor,
                       out: torch.Tensor | None = None) -> torch.Tensor:
    """Y fp16 [M, N] = X · (Wq · a_w / 127)ᵀ for M <= 16 (weight-only int8, no decomposition)."""
    M, K = _need_matrix(X)
    N = _need_weight(Wq, a_w, K, X.device)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=X.device)
    _need_shape(out, torch.float16, (M, N), X.device, "out")
    _check(lib().int8_weight_only_matmul(X.data_ptr(), M, K, Wq.data_ptr(), a_w.data_ptr(), N,
                                         out.data_ptr(), _stream(X)), "int8_weight_only_matmul")
    return out


class QuantizedActivations:
    """X quantized once (outlier columns, row constants, Xq, outlier values) for
    several int8_mixed_matmul_q calls; holds the device state buffer."""

    def __init__(self, X: torch.Tensor, threshold: float = 6.0, max_outliers: int = 256):
        self.M, self.K = _need_matrix(X)
        self.device = X.device
        self.max_outliers = max_outliers
        nbytes = int(lib().int8_quant_state_bytes(self.M, self.K, max_outliers))
        if nbytes == 0:
            raise ValueError(f"bad shape: M={self.M} K={self.K} max_outliers={max_outliers}")
        self.state = torch.empty((nbytes,), dtype=torch.uint8, device=X.device)
        _check(lib().int8_quantize_activations(X.data_ptr(), self.M, self.K, float(threshold),
                                               max_outliers, self.state.data_ptr(), nbytes,
                                               _stream(X)), "int8_quantize_activations")

    def contents(self) -> dict:
        """Views of the quantization results inside the state: a_x [M] fp32, Xq [M, K]
        int8 (a row-major copy), Xo [M, o_stride] fp16, idx [max_outliers] int32 and
        count (int)."""
        off = (_i64 * 6)()
        _check(lib().int8_quant_state_layout(self.M, self.K, self.max_outliers, off),
               "int8_quant_state_layout")
        st, M, K = self.state, self.M, self.K
        ks, rows = (K + 63) // 64, (M + 15) // 16 * 16
        a_x = st[off[0]:off[0] + 4 * M].view(torch.float32)
        xq = st[off[1]:off[1] + rows * ks * 64].view(torch.int8).view(rows // 16, ks, 16, 64)
        xo = st[off[2]:off[2] + 2 * M * off[5]].view(torch.float16).view(M, off[5])
        idx = st[off[3]:off[3] + 4 * self.max_outliers].view(torch.int32)
        count = int(st[off[4]:off[4] + 4].view(torch.int32).cpu()[0])
        return {"a_x": a_x, "Xq": untile_weight(xq, K)[:M], "Xo": xo, "idx": idx, "count": count}

    def matmul(self, Wq: torch.Tensor, a_w: torch.Tensor, out: torch.Tensor | None = None,
               workspace: torch.Tensor | None = None,
               acc_out: torch.Tensor | None = None) -> torch.Tensor:
        """Y fp16 [M, N] for one prepared weight, from this quantized X."""
        N = _need_weight(Wq, a_w, self.K, self.device)
        if out is not None:
            _need_shape(out, torch.float16, (self.M, N), self.device, "out")
        if acc_out is not None:
            _need_shape(acc_out, torch.int32, (self.M, N), self.device, "acc_out")
        wb = int(lib().int8_mixed_matmul_q_workspace_bytes(N, self.max_outliers))
        if workspace is None:
            workspace = torch.empty((wb,), dtype=torch.uint8, device=Wq.device)
        _need(workspace, torch.uint8, "workspace")
        if out is None:
            out = torch.empty((self.M, N), dtype=torch.float16, device=Wq.device)
        _check(lib().int8_mixed_matmul_q(self.state.data_ptr(), self.M, self.K, self.max_outliers,
                                         Wq.data_ptr(), a_w.data_ptr(), N, out.data_ptr(),
                                         workspace.data_ptr(), workspace.numel(),
                                         acc_out.data_ptr() if acc_out is not None else None,
                                         _stream(Wq)), "int8_mixed_matmul_q")
        return out

    def matmul_grouped(self, weights: list, outs: list | None = None,
                       workspace: torch.Tensor | None = None) -> list:
        """Y fp16 [M, N_q] for each (Wq, a_w) in `weights` (at most 8), from this
        quantized X, in one GEMM launch (one per weight for a few tokens)."""
        G = len(weights)
        if not 1 <= G <= 8:
            raise ValueError(f"between 1 and 8 weights, got {G}")
        Ns = [_need_weight(Wq, a_w, self.K, self.device) for Wq, a_w in weights]
        dev = self.device
        if outs is None:
            outs = [torch.empty((self.M, n), dtype=torch.float16, device=dev) for n in Ns]
        if len(outs) != G:
            raise ValueError(f"{G} weights but {len(outs)} outputs")
        for q, (o, n) in enumerate(zip(outs, Ns)):
            _need_shape(o, torch.float16, (self.M, n), dev, f"outs[{q}]")
        n_arr = (_i64 * G)(*Ns)
        wb = int(lib().int8_mixed_matmul_q_grouped_workspace_bytes(G, n_arr, self.max_outliers))
        if workspace is None:
            workspace = torch.empty((max(wb, 1),), dtype=torch.uint8, device=dev)
        _need(workspace, torch.uint8, "workspace")
        wq_arr = (_p * G)(*[w.data_ptr() for w, _ in weights])
        aw_arr = (_p * G)(*[a.data_ptr() for _, a in weights])
        y_arr = (_p * G)(*[o.data_ptr() for o in outs])
        _check(lib().int8_mixed_matmul_q_grouped(self.state.data_ptr(), self.M, self.K,
                                                 self.max_outliers, G, wq_arr, aw_arr, n_arr,
                                                 y_arr, workspace.data_ptr(), workspace.numel(),
                                                 _stream(workspace)),
               "int8_mixed_matmul_q_grouped")
        return outs


def read_status(workspace: torch.Tensor) -> tuple[int, int]:
    """(status of the last int8_mixed_matmul call on this workspace, its outlier count)."""
    n = ctypes.c_int32(0)
    rc = lib().int8mm_read_status(workspace.data_ptr(), ctypes.byref(n), _stream(workspace))
    if rc in (1, 6):
        raise Int8mmError(rc, "int8mm_read_status")
    return rc, n.value


def timing_enable(on: bool | int = True) -> None:
    """Event timing of each call's kernels: False/0 off, True/1 the main kernels, 2 also the
    two activation quantization phases (see int8mm_timing_enable)."""
    _check(lib().int8mm_timing_enable(int(on)), "int8mm_timing_enable")


def timing_read() -> tuple[float, int]:
    """(summed main-kernel milliseconds, bracketed calls) since the last read."""
    ms = ctypes.c_double(0.0)
    n = _i64(0)
    _check(lib().int8mm_timing_read(ctypes.byref(ms), ctypes.byref(n)), "int8mm_timing_read")
    return ms.value, n.value


PHASES = ("quant_pass", "quant_fixup", "main")


def timing_read_phases() -> dict:
    """{phase: (summed milliseconds, bracketed calls)} since the last read, for the pass
    over X, the quantization fix-up and the main kernels (see int8mm_timing_read_phases)."""
    ms = (ctypes.c_double * 3)()
    n = (_i64 * 3)()
    _check(lib().int8mm_timing_read_phases(ms, n), "int8mm_timing_read_phases")
    return {p: (ms[i], n[i]) for i, p in enumerate(PHASES)}
