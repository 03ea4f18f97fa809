"""LLM.int8() mixed-precision decomposed matmul for MI355X (gfx950).

The compute lives in ``libint8mm.so`` (hand-written HIP kernels behind a
C ABI, declared in ``include/int8mm.h``); ``binding`` marshals torch tensors
into it. ``inputs`` draws seeded synthetic workloads.
"""
