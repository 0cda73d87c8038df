"""W4A4 GEMM reference (oracle, test-only).

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
