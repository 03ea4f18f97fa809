"""CPU oracle for the mixed-precision int8 matmul (test infrastructure only).

Importable by the test suite, the package smoke check and the benchmark's
CPU-baseline leg; never by the product path.
"""

from .int8mm_oracle import (  # noqa: F401
    QMAX,
    dequant_outer,
    dequantize,
    int8_matmul,
    mask_words,
    mixed_matmul,
    outlier_columns,
    outlier_matmul,
    prepare_weight,
    quant_rows,
    quantize,
    weight_only_matmul,
)
