"""MR-GPTQ weight quantization (oracle).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
CPU-baseline leg of the benchmark, never by the library.

hyper.ai, paper 2509.23202 (MR-GPTQ), Abstract: a variant of the classical
GPTQ algorithm adapted to FP4 with blockwise Hadamard transforms, the
rotation fused into the weights and computed online for the activations.
pimento.cloud, "FP8, NVFP4 czy AWQ?", section "Czym roznia sie FP8, NVFP4,
MXFP4 i AWQ?": GPTQ quantizes the weights layer by layer with error
correction (Frantar et al., 2022, cited there).

What is computed (the plain column-by-column form of that error correction):

  1. Rotation (when asked): W and the calibration activations X are both
     rotated along k by the blockwise Hadamard transform of the format's
     block size (`hadamard_blocks`, float32), so (X R)(W R)^T = X W^T.
  2. H = 2 / N * X^T X in float64 over the N calibration rows.  A column
     with H_jj = 0 (a feature no calibration row uses) gets H_jj = 1 and its
     weights are zeroed; then H_jj += damp * mean(diag H).
  3. U = the upper-triangular Cholesky factor of H^-1 (U^T U = H^-1).
  4. NVFP4: the tensor scale from the (rotated) weights, once: max|W| / 2688.
  5. For j = 0 .. k-1: when j starts a block (16 for NVFP4, 32 for MXFP4),
     each row's block scale is chosen from the block's current weights with
     the format's own rule; column j is quantized with it exactly as the
     quantizer does (float32 arithmetic on float32(w)); a block whose scale
     came from all-zero weights keeps sign-only codes, whatever the error
     correction adds to it later (as the quantizer treats a zero block,
     both formats); with q the exact
     dequantized value, err = (w_j - q_j) / U_jj and every later column j'
     of the row takes w_j' -= err * U_jj'.

The float64 weights, Hessian and updates are the oracle's precision; the
codes and scales are those the format's quantizer gives the float32 value
of the current weight, so they are bit-comparable with the GPU's.
"""

import numpy as np

from .formats import e2m1_decode, e2m1_encode, e4m3_decode, e4m3_encode, e8m0_decode
from .hadamard import hadamard_blocks
from .quant import (NV_BLOCK, MX_BLOCK, mxfp4_block_exponent, nvfp4_tensor_scale,
                    pack_nibbles, dequantize_exact_f64)


def _block(fmt):
    if fmt == "nvfp4":
        return NV_BLOCK
    if fmt == "mxfp4":
        return MX_BLOCK
    raise ValueError(fmt)


def gptq_hessian(x):
    """2 / N * X^T X in float64 for calibration rows x [N, k]."""
    X = np.asarray(x, dtype=np.float64)
    return (2.0 / X.shape[0]) * (X.T @ X)


def gptq_factor(h, damp):
    """Dead columns, damping and the upper Cholesky factor of the inverse.
    Returns (U, dead) with dead the boolean mask of unused columns."""
    H = np.array(h, dtype=np.float64, copy=True)
    dead = np.diag(H) == 0
    H[dead, dead] = 1.0
    H[np.diag_indices_from(H)] += damp * np.mean(np.diag(H))
    U = np.linalg.cholesky(np.linalg.inv(H)).T
    return U, dead


def _group_scale(fmt, wg, s_t):
    """Rows' block scales from the float32 weights wg [rows, block]:
    (scale bytes, multiplier r applied before E2M1 rounding, dequant factor).
    Exactly the quantizer's rule (see nvfp4_quantize / mxfp4_quantize)."""
    a = np.max(np.abs(wg), axis=1)
    if fmt == "nvfp4":
        d = np.float32(6.0 * s_t)
        with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
            u = (a / d).astype(np.float32)
        sb = e4m3_encode(u)
        with np.errstate(over="ignore", under="ignore"):
            S = (e4m3_decode(sb) * np.float32(s_t)).astype(np.float32)
        with np.errstate(divide="ignore", over="ignore"):
            r = (np.float32(1.0) / S).astype(np.float32)
        usable = (S != 0) & np.isfinite(r)
        r = np.where(usable, r, np.float32(0.0)).astype(np.float32)
        deq = e4m3_decode(sb).astype(np.float64) * float(np.float32(s_t))
        return sb, r, deq, usable
    nonzero = a > 0
    kx = np.where(nonzero, mxfp4_block_exponent(np.where(nonzero, a, 1.0)), -127)
    sb = (kx + 127).astype(np.uint8)
    r = np.where(nonzero, np.ldexp(np.float32(1.0), -kx), 0.0).astype(np.float32)
    deq = e8m0_decode(sb)
    return sb, r, deq, nonzero


def gptq_quantize(fmt, w, x, damp=0.01, rotate=True, rows=None):
    """MR-GPTQ of the weights w [n, k] with calibration activations x [N, k].

    Returns (packed codes [n, k/2], scale bytes [n, k/block], tensor scale
    (NVFP4; None for MXFP4)) of the (rotated) weights: the operand the W4A4
    GEMM takes with activations quantized by the fused Hadamard quantizer.
    rows: only these rows (the rows are independent once H and the tensor
    scale, which are computed from all of w and x, are fixed).
    """
    b = _block(fmt)
    W32 = np.asarray(w, dtype=np.float32)
    X32 = np.asarray(x, dtype=np.float32)
    if rotate:
        W32 = hadamard_blocks(W32, b)
        X32 = hadamard_blocks(X32, b)
    n, k = W32.shape
    U, dead = gptq_factor(gptq_hessian(X32), damp)
    W = W32.astype(np.float64)
    W[:, dead] = 0.0
    s_t = np.float32(nvfp4_tensor_scale(W.astype(np.float32))) if fmt == "nvfp4" else None
    if rows is not None:
        W = W[np.asarray(rows)]
        n = W.shape[0]
    codes = np.zeros((n, k), dtype=np.uint8)
    scales = np.zeros((n, k // b), dtype=np.uint8)
    for j in range(k):
        if j % b == 0:
            wg = W[:, j:j + b].astype(np.float32)
            sb, r, deq, usable = _group_scale(fmt, wg, s_t)
            scales[:, j // b] = sb
        wj = W[:, j].astype(np.float32)
        with np.errstate(over="ignore", under="ignore", invalid="ignore"):
            qv = (wj * r).astype(np.float32)
        c = e2m1_encode(qv)
        c = np.where(usable, c, (np.signbit(wj).astype(np.uint8) << 3)).astype(np.uint8)
        codes[:, j] = c
        q = e2m1_decode(c).astype(np.float64) * deq
        err = (W[:, j] - q) / U[j, j]
        W[:, j + 1:] -= np.outer(err, U[j, j + 1:])
    return pack_nibbles(codes), scales, s_t


def gptq_layer_error(fmt, w, x, packed, scales, s_t, rotate=True):
    """Squared Frobenius error || X W^T - X Q^T ||^2 of a quantized layer in
    float64 (in the rotated basis when rotate: X R and W R)."""
    b = _block(fmt)
    W32 = np.asarray(w, dtype=np.float32)
    X32 = np.asarray(x, dtype=np.float32)
    if rotate:
        W32 = hadamard_blocks(W32, b)
        X32 = hadamard_blocks(X32, b)
    Q = dequantize_exact_f64(fmt, packed, scales, s_t)
    D = X32.astype(np.float64) @ (W32.astype(np.float64) - Q).T
    return float(np.sum(D * D))
