"""W4A4 and W4A16 GEMM references (oracle, test-only).

pimento.cloud "FP8, NVFP4 czy AWQ?", section "Dlaczego W8A8 i W4A16 to nie
to samo?": in W4A4 both weights and activations are 4-bit, so the matrix
products run on low-precision matrix units.  The product computed here is
C = X W^T with X [m, k] and W [n, k] both quantized along k; the reference is
the exact dequantized operands multiplied in float64.
"""

import numpy as np

from .quant import dequantize_exact_f64


def gemm_ref(fmt, a_packed, a_scales, a_tscale, b_packed, b_scales, b_tscale,
             chunk=4096):
    """float64 C [m, n] = deq(A) deq(B)^T, chunked over n to bound memory."""
    A = dequantize_exact_f64(fmt, a_packed, a_scales, a_tscale)
    n = b_packed.shape[0]
    C = np.empty((A.shape[0], n), dtype=np.float64)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        B = dequantize_exact_f64(fmt, b_packed[s:e], b_scales[s:e], b_tscale)
        C[:, s:e] = A @ B.T
    return C


def gemm_ref_entries(fmt, a_packed, a_scales, a_tscale, b_packed, b_scales,
                     b_tscale, rows, cols):
    """float64 C[rows[i], cols[i]] for sampled output positions only."""
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    A = dequantize_exact_f64(fmt, a_packed[rows], a_scales[rows], a_tscale)
    B = dequantize_exact_f64(fmt, b_packed[cols], b_scales[cols], b_tscale)
    return np.einsum("ik,ik->i", A, B)


def gemm_w4a16_ref(fmt, x, b_packed, b_scales, b_tscale, chunk=4096):
    """float64 C [m, n] = X deq(B)^T with 16-bit activations X [m, k] and
    4-bit weights B [n, k].

    pimento.cloud "FP8, NVFP4 czy AWQ?", section "Dlaczego W8A8 i W4A16 to
    nie to samo?": W4A16 shrinks only the weights (which helps token-by-token
    generation, where reading the weights is the bottleneck); the arithmetic
    stays 16-bit.  X holds the activations' exact values (bf16 / fp16 widened
    to float32); the reference multiplies them with the exact dequantized
    weights in float64.
    """
    X = np.asarray(x, dtype=np.float32).astype(np.float64)
    n = b_packed.shape[0]
    C = np.empty((X.shape[0], n), dtype=np.float64)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        B = dequantize_exact_f64(fmt, b_packed[s:e], b_scales[s:e], b_tscale)
        C[:, s:e] = X @ B.T
    return C
