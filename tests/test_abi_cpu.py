"""Host-side checks of libint8mm.so: it loads, exports every declared symbol, and
rejects bad arguments synchronously before any HIP call (no GPU needed).

The pointers below are fake, 16-byte-aligned addresses: every call here fails
validation, which the library does before it touches a pointer or the runtime.
"""

import ctypes
import math
import os
import re

import pytest

from int8_mixed_precision_col_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "int8mm.h")

P = 0x10000          # aligned fake device address
UNALIGNED = 0x10008
OK, E_NULL, E_SHAPE, E_ALIGN, E_THR, E_WS = 0, 1, 2, 3, 4, 5

pytestmark = pytest.mark.skipif(not os.path.exists(binding.LIB_PATH),
                                reason="libint8mm.so not built (run __graft_entry__.build())")


@pytest.fixture(scope="module")
def L():
    return binding.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:int8_|int8mm_)\w+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(binding.SIGNATURES)


def test_every_declared_symbol_is_exported(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_strerror_covers_codes(L):
    texts = {c: binding.strerror(c) for c in range(0, 9)}
    assert texts[0] == "ok"
    assert len(set(texts.values())) == 9
    assert "unknown" in binding.strerror(99)


def mm(L, X=P, M=64, K=256, Wq=P, aw=P, N=256, t=6.0, mo=16, Y=P, ws=P, wsb=1 << 30, acc=None):
    return L.int8_mixed_matmul(X, M, K, Wq, aw, N, t, mo, Y, ws, wsb, acc, None)


@pytest.mark.parametrize("kw,code", [
    (dict(X=None), E_NULL), (dict(Wq=None), E_NULL), (dict(aw=None), E_NULL),
    (dict(Y=None), E_NULL), (dict(ws=None), E_NULL),
    (dict(M=0), E_SHAPE), (dict(K=0), E_SHAPE), (dict(K=24), E_SHAPE), (dict(N=8), E_SHAPE),
    (dict(N=40), E_SHAPE), (dict(K=133152), E_SHAPE), (dict(M=1 << 25), E_SHAPE),
    (dict(mo=-1), E_SHAPE), (dict(mo=257), E_SHAPE), (dict(K=16384, mo=8193), E_SHAPE),
    (dict(t=-1.0), E_THR), (dict(t=math.nan), E_THR),
    (dict(X=UNALIGNED), E_ALIGN), (dict(Y=UNALIGNED), E_ALIGN), (dict(ws=UNALIGNED), E_ALIGN),
    (dict(acc=UNALIGNED), E_ALIGN),
    (dict(wsb=0), E_WS), (dict(M=4096, K=4096, N=4096, wsb=1 << 20), E_WS),
])
def test_mixed_matmul_rejects(L, kw, code):
    assert mm(L, **kw) == code


def test_quant_rows_rejects(L):
    q = L.int8_quant_rows
    assert q(None, 4, 32, 6.0, P, P, P, P, P, 4, None) == E_NULL
    assert q(P, 4, 32, 6.0, P, P, P, None, P, 4, None) == E_NULL   # idx needed when mo > 0
    assert q(P, 4, 30, 6.0, P, P, P, P, P, 4, None) == E_SHAPE
    assert q(P, 4, 32, 6.0, P, P, P, P, P, 33, None) == E_SHAPE
    assert q(P, 4, 32, -0.5, P, P, P, P, P, 4, None) == E_THR
    assert q(P, 4, 32, 6.0, UNALIGNED, P, P, P, P, 4, None) == E_ALIGN


def test_prepare_weight_rejects(L):
    pw = L.int8_prepare_weight
    assert pw(None, 32, 32, 0, P, P, None) == E_NULL
    assert pw(P, 32, 33, 0, P, P, None) == E_SHAPE
    assert pw(P, 32, 32, 2, P, P, None) == E_SHAPE
    assert pw(P, 32, 32, 1, UNALIGNED, P, None) == E_ALIGN


def test_workspace_sizes(L):
    ws = L.int8_mixed_matmul_workspace_bytes
    assert ws(0, 64, 64, 16) == 0 and ws(64, 64, 64, 65) == 0
    # decode path: header only
    assert L.int8_mixed_matmul_is_decode(8, 4096) == 1 and ws(8, 4096, 4096, 256) == 256
    assert L.int8_mixed_matmul_is_decode(16, 1024) == 1
    assert L.int8_mixed_matmul_is_decode(17, 1024) == 0
    # X chunks held per thread: rows held (M rounded up to a power of two) x K / 4096
    assert L.int8_mixed_matmul_is_decode(16, 4096) == 1
    assert L.int8_mixed_matmul_is_decode(9, 4112) == 0
    assert L.int8_mixed_matmul_is_decode(8, 8192) == 1
    assert L.int8_mixed_matmul_is_decode(8, 8208) == 0
    assert L.int8_mixed_matmul_is_decode(4, 8192) == 1
    # prefill: Xq + a_x + Xo + the outlier column list + the gathered outlier weight
    # rows WoT (+ flags, header, alignment)
    M, K, N, mo = 2048, 4096, 16384, 256
    b = ws(M, K, N, mo)
    assert b >= M * K + 4 * M + 2 * M * mo + 4 * mo + 2 * N * mo
    assert b < M * K + 4 * M + 2 * M * mo + 4 * mo + 2 * N * mo + (1 << 20)
    assert ws(M, K, N, 0) < b and ws(M + 1, K, N, mo) > b and ws(M, K, N + 16, mo) > b
    assert b % 256 == 0


def test_binding_prepared_size_matches_library(L):
    # the binding asks the library once per shape and reuses the answer
    for K, N in [(16, 16), (1040, 528), (12288, 49152), (1040, 528)]:
        assert binding._prepared_bytes(K, N) == L.int8_prepared_weight_bytes(K, N)
    assert binding._prepared_bytes(1040, 528) == 528 * 1088


def test_timing_read_without_launches(L):
    ms, n = binding.timing_read()
    assert (ms, n) == (0.0, 0)
    assert L.int8mm_timing_read(None, None) == E_NULL


def test_weight_only_rejects(L):
    wo = L.int8_weight_only_matmul
    assert wo(None, 4, 32, P, P, 32, P, None) == E_NULL
    assert wo(P, 17, 32, P, P, 32, P, None) == E_SHAPE      # decode shapes only
    assert wo(P, 0, 32, P, P, 32, P, None) == E_SHAPE
    assert wo(P, 4, 24, P, P, 32, P, None) == E_SHAPE       # K not a multiple of 16
    assert wo(P, 4, 32, P, P, 24, P, None) == E_SHAPE       # N not a multiple of 16
    assert wo(UNALIGNED, 4, 32, P, P, 32, P, None) == E_ALIGN
    assert wo(P, 4, 32, P, P, 32, UNALIGNED, None) == E_ALIGN


@pytest.mark.parametrize("M,K,mo", [(64, 256, 16), (4096, 12288, 256), (17, 33024, 0),
                                     (4097, 20480, 8192), (1, 16, 1)])
def test_quant_state_layout(L, M, K, mo):
    """The published offsets lie inside the state, 16-byte aligned, in disjoint ranges
    that hold their fields (a_x, unit-tiled Xq, Xo, the column list, the count)."""
    off = (ctypes.c_int64 * 6)()
    assert L.int8_quant_state_layout(M, K, mo, off) == 0
    total = L.int8_quant_state_bytes(M, K, mo)
    o_stride = off[5]
    assert o_stride % 16 == 0 and o_stride >= mo
    rows, ks = (M + 15) // 16 * 16, (K + 63) // 64
    spans = sorted([(off[0], 4 * M), (off[1], rows * ks * 64), (off[2], 2 * M * o_stride),
                    (off[3], 4 * mo), (off[4], 4)])
    for (a, n), (b, _) in zip(spans, spans[1:]):
        assert a + n <= b
    assert spans[-1][0] + spans[-1][1] <= total
    assert all(off[i] % 16 == 0 for i in range(4)) and off[4] % 4 == 0
    assert L.int8_quant_state_layout(M, K, mo, None) == E_NULL
    assert L.int8_quant_state_layout(0, K, mo, off) == E_SHAPE
    assert L.int8_quant_state_layout(M, K + 8, mo, off) == E_SHAPE


def test_quantize_once_rejects_and_sizes(L):
    assert L.int8_quant_state_bytes(0, 64, 16) == 0
    assert L.int8_quant_state_bytes(4096, 12288, 256) > 4096 * 12288   # holds Xq
    # the one-call workspace is the state followed by the gathered weight rows
    assert L.int8_quant_state_bytes(2048, 4096, 256) + 2 * 4096 * 256 == \
        L.int8_mixed_matmul_workspace_bytes(2048, 4096, 4096, 256)
    assert L.int8_mixed_matmul_q_workspace_bytes(512, 256) == 256       # reserved, fixed
    assert L.int8_mixed_matmul_q_workspace_bytes(24, 16) == 0
    qa = L.int8_quantize_activations
    nb = L.int8_quant_state_bytes(64, 256, 16)
    assert qa(None, 64, 256, 6.0, 16, P, nb, None) == E_NULL
    assert qa(P, 64, 250, 6.0, 16, P, nb, None) == E_SHAPE
    assert qa(P, 64, 256, -1.0, 16, P, nb, None) == E_THR
    assert qa(P, 64, 256, 6.0, 16, UNALIGNED, nb, None) == E_ALIGN
    assert qa(P, 64, 256, 6.0, 16, P, nb - 1, None) == E_WS
    mq = L.int8_mixed_matmul_q
    wb = L.int8_mixed_matmul_q_workspace_bytes(128, 16)
    assert mq(P, 64, 256, 16, None, P, 128, P, P, wb, None, None) == E_NULL
    assert mq(P, 64, 256, 16, P, P, 120, P, P, wb, None, None) == E_SHAPE
    assert mq(P, 64, 256, 16, P, P, 128, UNALIGNED, P, wb, None, None) == E_ALIGN
    assert mq(P, 64, 256, 16, P, P, 128, P, P, wb - 1, None, None) == E_WS


def test_grouped_rejects_and_sizes(L):
    I64 = ctypes.c_int64
    P_ = ctypes.c_void_p
    ns = (I64 * 3)(512, 272, 1040)
    wb = L.int8_mixed_matmul_q_grouped_workspace_bytes(3, ns, 16)
    assert wb == sum(L.int8_mixed_matmul_q_workspace_bytes(n, 16) for n in (512, 272, 1040))
    assert L.int8_mixed_matmul_q_grouped_workspace_bytes(0, ns, 16) == 0
    assert L.int8_mixed_matmul_q_grouped_workspace_bytes(9, (I64 * 9)(*[64] * 9), 16) == 0
    assert L.int8_mixed_matmul_q_grouped_workspace_bytes(1, (I64 * 1)(24), 16) == 0
    ptrs = (P_ * 3)(P, P, P)
    g = L.int8_mixed_matmul_q_grouped
    assert g(None, 64, 256, 16, 3, ptrs, ptrs, ns, ptrs, P, wb, None) == E_NULL
    assert g(P, 64, 256, 16, 3, None, ptrs, ns, ptrs, P, wb, None) == E_NULL
    assert g(P, 64, 256, 16, 3, (P_ * 3)(P, None, P), ptrs, ns, ptrs, P, wb, None) == E_NULL
    assert g(P, 64, 256, 16, 0, ptrs, ptrs, ns, ptrs, P, wb, None) == E_SHAPE
    assert g(P, 64, 256, 16, 9, (P_ * 9)(*[P] * 9), (P_ * 9)(*[P] * 9), (I64 * 9)(*[64] * 9),
             (P_ * 9)(*[P] * 9), P, 1 << 30, None) == E_SHAPE
    assert g(P, 64, 256, 16, 3, ptrs, ptrs, (I64 * 3)(512, 24, 1040), ptrs, P, wb, None) == E_SHAPE
    assert g(P, 64, 250, 16, 3, ptrs, ptrs, ns, ptrs, P, wb, None) == E_SHAPE
    assert g(P, 64, 256, 16, 3, ptrs, (P_ * 3)(P, UNALIGNED, P), ns, ptrs, P, wb, None) == E_ALIGN
    assert g(P, 64, 256, 16, 3, ptrs, ptrs, ns, ptrs, P, wb - 1, None) == E_WS


E_SCRATCH = 8
NOALLOC_SCRATCH_BYTES = 64 << 20   # INT8MM_NOALLOC_SCRATCH_BYTES in include/int8mm.h


def test_noalloc_limit_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define INT8MM_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == NOALLOC_SCRATCH_BYTES


def test_noalloc_rejects_before_any_hip_call(L):
    """Argument errors and shapes beyond the fixed scratch are returned before the
    library touches the device (no GPU here: any HIP call would fail differently)."""
    na = L.int8_mixed_matmul_noalloc
    ws = L.int8_mixed_matmul_workspace_bytes
    assert na(None, 64, 256, P, P, 256, 6.0, 16, P, None, None) == E_NULL
    assert na(P, 64, 256, P, P, 256, 6.0, 16, None, None, None) == E_NULL
    assert na(P, 64, 250, P, P, 256, 6.0, 16, P, None, None) == E_SHAPE
    assert na(P, 64, 256, P, P, 256, math.nan, 16, P, None, None) == E_THR
    assert na(P, 64, 256, P, P, 256, 6.0, 16, P, UNALIGNED, None) == E_ALIGN
    # a shape just over the scratch, and the 13B-like and 175B-like prefill shapes
    M, K, N = 4096, 12288, 49152
    assert ws(M, K, N, 256) > NOALLOC_SCRATCH_BYTES
    assert na(P, M, K, P, P, N, 6.0, 256, P, None, None) == E_SCRATCH
    assert ws(4096, 20480, 5120, 256) > NOALLOC_SCRATCH_BYTES
    assert na(P, 4096, 20480, P, P, 5120, 6.0, 256, P, None, None) == E_SCRATCH
    over = next(m for m in range(2048, 1 << 16, 256) if ws(m, 8192, 4096, 256) > NOALLOC_SCRATCH_BYTES)
    assert na(P, over, 8192, P, P, 4096, 6.0, 256, P, None, None) == E_SCRATCH
    # what the limit admits: every decode shape and the 6.7B-like FFN shape
    assert ws(8, 4096, 4096, 256) <= NOALLOC_SCRATCH_BYTES
    assert ws(2048, 4096, 16384, 256) <= NOALLOC_SCRATCH_BYTES


def test_tile_weight_rejects(L):
    tw = L.int8_tile_weight
    assert tw(None, 64, 32, P, None) == E_NULL
    assert tw(P, 64, 32, None, None) == E_NULL
    assert tw(P, 40, 32, P, None) == E_SHAPE       # K not a multiple of 16
    assert tw(P, 64, 24, P, None) == E_SHAPE       # N not a multiple of 16
    assert tw(P, 133152, 32, P, None) == E_SHAPE   # past the int32 guard
    assert tw(UNALIGNED, 64, 32, P, None) == E_ALIGN
    assert tw(P, 64, 32, UNALIGNED, None) == E_ALIGN
