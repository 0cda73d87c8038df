"""Block-scaled FP4 (NVFP4 / MXFP4) quantization and W4A4 GEMM for MI355X.

The compute lives in libfp4.so (HIP kernels for gfx950 behind the C ABI in
include/fp4.h); `fp4` is its Python binding.
"""

from . import fp4
from .fp4 import (quantize, quantize_mse, hadamard_quantize, dequantize, gemm, gemm_w4a16,
                  quantize_gemm, kv_cache, kv_append, attention_decode, gptq_quantize, lib)

__all__ = ["fp4", "quantize", "quantize_mse", "hadamard_quantize", "dequantize", "gemm", "gemm_w4a16",
           "quantize_gemm", "kv_cache", "kv_append", "attention_decode", "gptq_quantize",
           "lib"]
