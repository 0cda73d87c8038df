"""Block-scaled FP4 (NVFP4 / MXFP4) quantization and W4A4 GEMM for MI355X."""
