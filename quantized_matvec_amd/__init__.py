"""qmv: 4-bit blockwise weight quantization (NF4 / FP4, optional double-quantized
scales) and the fused dequantize-and-multiply, as hand-written HIP for gfx950
behind a C ABI (``libqmv.so``, declared in ``include/qmv.h``).

The library is loaded on first use; every op raises if it is not built."""
from .qmv import (  # noqa: F401
    QmvError, QuantState, code_table, default_code2, dequantize_4bit, dequantize_absmax,
    double_quant, gemm_4bit, gemv_4bit, lib, library_path, quantize_4bit,
)
