"""qmv: 4-bit blockwise weight quantization (NF4 / FP4, optional double-quantized
scales) and the fused dequantize-and-multiply, as hand-written HIP for gfx950
behind a C ABI (``libqmv.so``)."""
