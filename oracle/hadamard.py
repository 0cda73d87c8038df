"""Blockwise Hadamard rotation (oracle, test-only).

hyper.ai, paper 2509.23202 (MR-GPTQ), Abstract: FP4 quantization is adapted
with blockwise Hadamard transforms, fused into the weights offline and
computed online for the activations.  The aisyndicate.ch page, section
"Accuracy ist nicht gleich Accuracy", names the same method.

Reading taken here (the pages give no formula): each row is cut along k into
blocks of b values (b = 16 for NVFP4, 32 for MXFP4, aligned with the
quantization blocks) and every block is multiplied by H_b / sqrt(b), H_b the
Sylvester Hadamard matrix of order b (symmetric, entries +-1), with no random
sign flips.  Because H_b H_b^T = b I, applying the same rotation to X and W
leaves X W^T unchanged.

Arithmetic order (it decides rounding, and the 4-bit codes downstream): in
float32, the butterfly stages h = 1, 2, 4, ..., b/2; in each stage every pair
(j, j+h) inside a group of 2h becomes (y_j + y_{j+h}, y_j - y_{j+h}); then
one multiply by the float32 constant c_b = fp32(1/sqrt(b)) (0.25 exactly for
b = 16).
"""

import numpy as np

HADAMARD_NORM = {
    16: np.float32(0.25),
    32: np.float32(1.0 / np.sqrt(32.0)),
}


def hadamard_blocks(x, b):
    """Rotate every b-block of each row of a [rows, k] array; float32 out."""
    if b not in HADAMARD_NORM:
        raise ValueError("block size must be 16 or 32")
    x = np.asarray(x, dtype=np.float32)
    rows, k = x.shape
    if k % b:
        raise ValueError("k must be a multiple of the block size")
    y = x.reshape(rows, k // b, b).copy()
    h = 1
    while h < b:
        for start in range(0, b, 2 * h):
            for j in range(start, start + h):
                u = y[:, :, j].copy()
                v = y[:, :, j + h].copy()
                y[:, :, j] = u + v          # float32 add
                y[:, :, j + h] = u - v      # float32 subtract
        h *= 2
    y = (y * HADAMARD_NORM[b]).astype(np.float32)
    return y.reshape(rows, k)
