"""CPU oracle for block-scaled FP4 quantization (NVFP4 / MXFP4).

TEST INFRASTRUCTURE ONLY.  This package is the slow, plain reference that the
HIP library is checked against.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import it; the library itself never
does, and it shares no code, table or helper with the HIP path.

Arithmetic that decides an integer (a block-scale byte, a 4-bit code) is done
in IEEE float32 with NumPy, one rounding per operation and no fused
multiply-add, because that is the precision the kernels decide in.  The GEMM
reference accumulates in float64.

Sources (the web pages this method is described on):
  * aisyndicate.ch, "FP4 auf Blackwell: Was NVFP4 fuer lokale KI wirklich
    aendert", section "Was NVFP4 von frueheren 4-Bit-Formaten unterscheidet"
    (E2M1 layout, MXFP4 power-of-two scale on 32 values, NVFP4 E4M3 scale on
    16 values plus one FP32 scale per tensor).
  * pimento.cloud, "FP8, NVFP4 czy AWQ?", section "Czym roznia sie FP8, NVFP4,
    MXFP4 i AWQ?" (E4M3 = 4 exponent / 3 mantissa bits, E2M1 range about +-6,
    ~4.5 bits per value, MXFP4 = OCP blocks of 32 with an E8M0 scale).
  * hyper.ai, paper 2509.23202 (MR-GPTQ), Abstract (blockwise Hadamard
    transforms, rotation fused into the weights, online for activations;
    MR-GPTQ as a variant of GPTQ).
  * pimento.cloud, section "Czym roznia sie FP8, NVFP4, MXFP4 i AWQ?" (GPTQ
    quantizes layer by layer with error correction).
  * hyper.ai story on the NVFP4 KV cache (new K/V written to the cache in
    NVFP4, dequantization to FP8 before attention).

Parity status per function (what pins it in the CPU tests):
  e2m1_decode / e2m1_encode   closed form + brute-force nearest-value search
  e4m3_decode / e4m3_encode   torch.float8_e4m3fn (library routine)
  e8m0_decode / e8m0_encode   math.ldexp closed form
  nvfp4_quantize              exact-rational properties, invariants, golden
  nvfp4_quantize_mse          exact-rational argmin over all scale bytes,
                              never worse than amax / 6, hand-worked golden
  mxfp4_quantize              brute-force exponent search, invariants, golden
  dequantize                  hand-built golden tensors, exact-rational check
  hadamard_blocks             scipy.linalg.hadamard matmul, involution
  gemm_ref                    integer matmul special case, Fraction brute force
  gemm_w4a16_ref              integer special case, Fraction brute force,
                              equals gemm_ref when X is itself NVFP4-exact
  kv_append_ref               hand-worked NVFP4 / MXFP4 rows at their
                              positions, dropped out-of-range rows
  attention_decode_ref        exact rows, means, 3:1 weights, GQA head map,
                              FP8 ties and saturation, one-hot key
  gptq_quantize               diagonal Hessian = plain quantizer (bit-exact),
                              equals the surgeon form with fresh sub-Hessian
                              inverses, beats round-to-nearest, dead features
"""

from .formats import (
    E2M1_MAGNITUDES,
    e2m1_decode,
    e2m1_encode,
    e4m3_decode,
    e4m3_encode,
    e4m3_encode_signed,
    e8m0_decode,
    e8m0_encode_exponent,
    bf16_round,
)
from .quant import (
    NV_BLOCK,
    MX_BLOCK,
    NV_TSCALE_DIVISOR,
    nvfp4_tensor_scale,
    nvfp4_tensor_scale_from_amax,
    nvfp4_quantize,
    nvfp4_quantize_mse,
    nvfp4_mse_block_error,
    mxfp4_quantize,
    dequantize,
    dequantize_exact_f64,
    pack_nibbles,
    unpack_nibbles,
)
from .hadamard import hadamard_blocks, HADAMARD_NORM
from .gemm import gemm_ref, gemm_ref_entries, gemm_w4a16_ref
from .attention import kv_append_ref, kv_fp8_values, attention_decode_ref
from .gptq import gptq_hessian, gptq_factor, gptq_quantize, gptq_layer_error

__all__ = [
    "E2M1_MAGNITUDES", "e2m1_decode", "e2m1_encode", "e4m3_decode",
    "e4m3_encode", "e4m3_encode_signed", "e8m0_decode", "e8m0_encode_exponent",
    "bf16_round", "NV_BLOCK", "MX_BLOCK", "NV_TSCALE_DIVISOR",
    "nvfp4_tensor_scale", "nvfp4_tensor_scale_from_amax", "nvfp4_quantize", "nvfp4_quantize_mse", "nvfp4_mse_block_error", "mxfp4_quantize", "dequantize",
    "dequantize_exact_f64", "pack_nibbles", "unpack_nibbles",
    "hadamard_blocks", "HADAMARD_NORM", "gemm_ref", "gemm_ref_entries", "gemm_w4a16_ref",
    "kv_append_ref", "kv_fp8_values", "attention_decode_ref",
    "gptq_hessian", "gptq_factor", "gptq_quantize", "gptq_layer_error",
]
