"""Pins for the oracle's MR-GPTQ (CPU only).

hyper.ai, paper 2509.23202 (MR-GPTQ), Abstract: GPTQ adapted to FP4 with
blockwise Hadamard transforms; pimento.cloud "FP8, NVFP4 czy AWQ?": GPTQ
quantizes layer by layer with error correction.  The oracle's Cholesky form
is checked against things fixed independently of it:

  * a diagonal Hessian leaves nothing to correct: the result is the plain
    quantizer's, bit for bit (closed form);
  * the original optimal-brain-surgeon form of the same greedy procedure,
    which inverts the remaining sub-Hessian at every column instead of using
    the rows of the Cholesky factor, gives the same codes and scales;
  * on correlated calibration data the layer error ||X W^T - X Q^T|| is well
    below round-to-nearest's;
  * a feature no calibration row uses gets zero weight.
"""

import numpy as np
import pytest

import oracle
from oracle.gptq import gptq_quantize, gptq_layer_error, gptq_hessian, _group_scale
from oracle.formats import e2m1_decode, e2m1_encode


def _correlated(n, k, N, seed):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    mix = rng.standard_normal((k, k)) / np.sqrt(k)
    x = (rng.standard_normal((N, k)) @ mix + 0.3 * rng.standard_normal((N, k))).astype(np.float32)
    return w, x


def _rtn(fmt, w, rotate=True):
    b = 16 if fmt == "nvfp4" else 32
    wr = oracle.hadamard_blocks(w, b) if rotate else w
    if fmt == "nvfp4":
        return oracle.nvfp4_quantize(wr)
    c, s = oracle.mxfp4_quantize(wr)
    return c, s, None


def _obs_reference(fmt, w, x, damp=0.01, rotate=True):
    """The same greedy quantization in its optimal-brain-surgeon form: after
    quantizing column j, the remaining columns move by
    -(w_j - q_j) * [H_r^-1]_{0,:} / [H_r^-1]_{00} with H_r the Hessian of the
    columns not yet quantized (inverted afresh at every step)."""
    b = 16 if fmt == "nvfp4" else 32
    W32 = np.asarray(w, dtype=np.float32)
    X32 = np.asarray(x, dtype=np.float32)
    if rotate:
        W32 = oracle.hadamard_blocks(W32, b)
        X32 = oracle.hadamard_blocks(X32, b)
    n, k = W32.shape
    H = np.einsum("ti,tj->ij", X32.astype(np.float64), X32.astype(np.float64)) * (2.0 / X32.shape[0])
    dead = np.diag(H) == 0
    H[dead, dead] = 1.0
    H[np.diag_indices_from(H)] += damp * np.mean(np.diag(H))
    W = W32.astype(np.float64)
    W[:, dead] = 0.0
    s_t = np.float32(oracle.nvfp4_tensor_scale(W.astype(np.float32))) if fmt == "nvfp4" else None
    codes = np.zeros((n, k), dtype=np.uint8)
    scales = np.zeros((n, k // b), dtype=np.uint8)
    for j in range(k):
        if j % b == 0:
            sb, r, deq, usable = _group_scale(fmt, W[:, j:j + b].astype(np.float32), s_t)
            scales[:, j // b] = sb
        wj = W[:, j].astype(np.float32)
        with np.errstate(over="ignore", under="ignore", invalid="ignore"):
            c = e2m1_encode((wj * r).astype(np.float32))
        c = np.where(usable, c, np.signbit(wj).astype(np.uint8) << 3).astype(np.uint8)
        codes[:, j] = c
        q = e2m1_decode(c).astype(np.float64) * deq
        Hr_inv = np.linalg.inv(H[j:, j:])
        W[:, j:] -= np.outer(W[:, j] - q, Hr_inv[0, :] / Hr_inv[0, 0])
    return oracle.pack_nibbles(codes), scales, s_t


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_diagonal_hessian_gives_the_plain_quantizer(fmt):
    # X = 3 I: X R stays orthogonal, H is diagonal, U has no off-diagonal
    # entries, so no error is carried and GPTQ is round-to-nearest
    rng = np.random.default_rng(1)
    k = 64
    w = (rng.standard_normal((24, k)) * 0.05).astype(np.float32)
    x = (3.0 * np.eye(k)).astype(np.float32)
    c, s, t = gptq_quantize(fmt, w, x)
    rc, rs, rt = _rtn(fmt, w)
    np.testing.assert_array_equal(c, rc)
    np.testing.assert_array_equal(s, rs)
    if fmt == "nvfp4":
        assert np.float32(t) == np.float32(rt)


@pytest.mark.parametrize("fmt,rotate", [("nvfp4", True), ("mxfp4", True), ("nvfp4", False)])
def test_cholesky_form_equals_the_surgeon_form(fmt, rotate):
    w, x = _correlated(12, 64, 200, seed=2)
    c, s, t = gptq_quantize(fmt, w, x, rotate=rotate)
    oc, os_, ot = _obs_reference(fmt, w, x, rotate=rotate)
    np.testing.assert_array_equal(s, os_)
    np.testing.assert_array_equal(c, oc)


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_error_correction_beats_round_to_nearest(fmt):
    w, x = _correlated(48, 128, 512, seed=3)
    c, s, t = gptq_quantize(fmt, w, x)
    rc, rs, rt = _rtn(fmt, w)
    e = gptq_layer_error(fmt, w, x, c, s, t)
    er = gptq_layer_error(fmt, w, x, rc, rs, rt)
    assert e < 0.8 * er, (e, er)


def test_unused_feature_gets_zero_weight():
    w, x = _correlated(8, 32, 100, seed=4)
    x[:, 5] = 0.0
    c, s, t = gptq_quantize("nvfp4", w, x, rotate=False)
    codes = oracle.unpack_nibbles(c)
    assert np.all((codes[:, 5] & 7) == 0)


def test_hessian_is_twice_the_mean_outer_product():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((7, 5)).astype(np.float32)
    want = sum(np.outer(r, r) for r in x.astype(np.float64)) * 2.0 / 7
    np.testing.assert_allclose(gptq_hessian(x), want, rtol=1e-14)
