"""Pins for the oracle's blockwise Hadamard and GEMM reference (CPU only).

The rotation is checked against scipy.linalg.hadamard (a library routine) and
its algebraic identities; the GEMM reference against an exact integer matmul
special case and an exact-rational triple loop.
"""

from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

import oracle


@pytest.mark.parametrize("b", [16, 32])
def test_hadamard_matrix_identity(b):
    H = scipy.linalg.hadamard(b)
    assert np.array_equal(H @ H.T, b * np.eye(b, dtype=H.dtype))
    assert np.array_equal(H, H.T)


@pytest.mark.parametrize("b", [16, 32])
def test_fwht_matches_matrix_product(b):
    rng = np.random.default_rng(b)
    x = rng.standard_normal((6, 4 * b)).astype(np.float32)
    y = oracle.hadamard_blocks(x, b).astype(np.float64)
    H = scipy.linalg.hadamard(b).astype(np.float64) / np.sqrt(b)
    ref = (x.astype(np.float64).reshape(6, 4, b) @ H).reshape(6, 4 * b)
    # log2(b) fp32 add stages + one multiply: error well under 1e-6 relative
    scale = np.max(np.abs(x))
    assert np.max(np.abs(y - ref)) <= 8 * np.log2(b) * 2.0 ** -24 * scale * np.sqrt(b)
    # blocks are independent and aligned: perturbing block 1 leaves block 0
    x2 = x.copy()
    x2[:, b:2 * b] += 1
    y2 = oracle.hadamard_blocks(x2, b)
    assert np.array_equal(y2[:, :b], y[:, :b].astype(np.float32))


@pytest.mark.parametrize("b", [16, 32])
def test_fwht_is_an_involution(b):
    x = np.random.default_rng(1).standard_normal((4, 2 * b)).astype(np.float32)
    back = oracle.hadamard_blocks(oracle.hadamard_blocks(x, b), b)
    assert np.max(np.abs(back - x)) < 1e-5


def test_fwht_exact_on_integers_for_b16():
    # b = 16: adds of small integers are exact and the 0.25 scale is exact,
    # so the result equals the integer product H x / 4 exactly.
    rng = np.random.default_rng(2)
    x = rng.integers(-50, 50, size=(3, 48)).astype(np.float32)
    H = scipy.linalg.hadamard(16)
    ref = (x.astype(np.int64).reshape(3, 3, 16) @ H).reshape(3, 48) / 4
    assert np.array_equal(oracle.hadamard_blocks(x, 16), ref.astype(np.float32))


def test_rotation_cancels_in_the_product():
    # (X R)(W R)^T = X W^T because R R^T = I (rotation fused into weights)
    rng = np.random.default_rng(3)
    X = rng.standard_normal((5, 64))
    W = rng.standard_normal((7, 64))
    for b in (16, 32):
        H = scipy.linalg.hadamard(b) / np.sqrt(b)
        R = np.kron(np.eye(64 // b), H)
        assert np.allclose((X @ R) @ (W @ R).T, X @ W.T, atol=1e-12, rtol=0)


def test_gemm_integer_special_case():
    # MXFP4 with every scale code 127 (scale 1): 2v are integers in
    # [-12, 12] and 4 C equals the int64 matmul of 2v exactly.
    rng = np.random.default_rng(4)
    m, n, k = 64, 48, 4096
    ca = rng.integers(0, 16, size=(m, k)).astype(np.uint8)
    cb = rng.integers(0, 16, size=(n, k)).astype(np.uint8)
    pa, pb = oracle.pack_nibbles(ca), oracle.pack_nibbles(cb)
    sa = np.full((m, k // 32), 127, np.uint8)
    sb = np.full((n, k // 32), 127, np.uint8)
    C = oracle.gemm_ref("mxfp4", pa, sa, None, pb, sb, None)
    ia = (2 * oracle.e2m1_decode(ca)).astype(np.int64)
    ib = (2 * oracle.e2m1_decode(cb)).astype(np.int64)
    assert np.array_equal((4 * C).astype(np.int64), ia @ ib.T)
    assert np.array_equal(4 * C, (ia @ ib.T).astype(np.float64))


def _fraction_gemm(fmt, pa, sa, ta, pb, sb, tb):
    ca, cb = oracle.unpack_nibbles(pa), oracle.unpack_nibbles(pb)
    mags = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4), Fraction(6)]

    def val(c):
        return -mags[c & 7] if c & 8 else mags[c & 7]

    def scale(s, blk):
        if fmt == "mxfp4":
            return Fraction(2) ** (int(s) - 127)
        e, mt = (int(s) >> 3) & 15, int(s) & 7
        return Fraction(mt, 512) if e == 0 else (1 + Fraction(mt, 8)) * Fraction(2) ** (e - 7)

    bs = 16 if fmt == "nvfp4" else 32
    m, k = ca.shape
    n = cb.shape[0]
    tA = Fraction(float(ta)) if ta is not None else Fraction(1)
    tB = Fraction(float(tb)) if tb is not None else Fraction(1)
    C = [[Fraction(0)] * n for _ in range(m)]
    for i in range(m):
        for j in range(n):
            acc = Fraction(0)
            for kk in range(k):
                acc += val(ca[i, kk]) * scale(sa[i, kk // bs], bs) * val(cb[j, kk]) * scale(sb[j, kk // bs], bs)
            C[i][j] = acc * tA * tB
    return C


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_gemm_matches_exact_triple_loop(fmt):
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 64)).astype(np.float32)
    w = (rng.standard_normal((4, 64)) * 0.05).astype(np.float32)
    if fmt == "nvfp4":
        pa, sa, ta = oracle.nvfp4_quantize(x)
        pb, sb, tb = oracle.nvfp4_quantize(w)
    else:
        (pa, sa), ta = oracle.mxfp4_quantize(x), None
        (pb, sb), tb = oracle.mxfp4_quantize(w), None
    C = oracle.gemm_ref(fmt, pa, sa, ta, pb, sb, tb)
    exact = _fraction_gemm(fmt, pa, sa, ta, pb, sb, tb)
    for i in range(3):
        for j in range(4):
            # float64 holds each product exactly; only the k-sum rounds
            assert abs(Fraction(C[i, j]) - exact[i][j]) <= abs(exact[i][j]) * Fraction(1, 2 ** 45) + Fraction(1, 2 ** 80)
    ent = oracle.gemm_ref_entries(fmt, pa, sa, ta, pb, sb, tb, [0, 2, 1], [3, 0, 1])
    assert np.allclose(ent, [C[0, 3], C[2, 0], C[1, 1]], rtol=1e-12, atol=0)


# --- W4A16 --------------------------------------------------------------------

def test_w4a16_integer_special_case():
    # MXFP4 weights with scale code 127 (scale 1) are half-integers 2v in
    # [-12, 12]/2; integer activations: 2 C is an integer matmul, exactly.
    rng = np.random.default_rng(21)
    m, n, k = 5, 7, 256
    x = rng.integers(-50, 51, size=(m, k)).astype(np.float32)
    cb = rng.integers(0, 16, size=(n, k)).astype(np.uint8)
    pb = oracle.pack_nibbles(cb)
    sb = np.full((n, k // 32), 127, dtype=np.uint8)
    C = oracle.gemm_w4a16_ref("mxfp4", x, pb, sb, None)
    ib = (2 * oracle.e2m1_decode(cb)).astype(np.int64)
    assert np.array_equal((2 * C).astype(np.int64), x.astype(np.int64) @ ib.T)
    assert np.array_equal(2 * C, (x.astype(np.int64) @ ib.T).astype(np.float64))


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_w4a16_matches_exact_triple_loop(fmt):
    rng = np.random.default_rng(22)
    x = rng.standard_normal((3, 64)).astype(np.float32)
    w = (rng.standard_normal((4, 64)) * 0.05).astype(np.float32)
    if fmt == "nvfp4":
        pb, sb, tb = oracle.nvfp4_quantize(w)
    else:
        (pb, sb), tb = oracle.mxfp4_quantize(w), None
    C = oracle.gemm_w4a16_ref(fmt, x, pb, sb, tb)
    cb = oracle.unpack_nibbles(pb)
    mags = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4), Fraction(6)]
    bs = 16 if fmt == "nvfp4" else 32
    for i in range(3):
        for j in range(4):
            acc = Fraction(0)
            for kk in range(64):
                c = int(cb[j, kk])
                v = -mags[c & 7] if c & 8 else mags[c & 7]
                s = int(sb[j, kk // bs])
                if fmt == "mxfp4":
                    sc = Fraction(2) ** (s - 127)
                else:
                    e, mt = (s >> 3) & 15, s & 7
                    sc = Fraction(mt, 512) if e == 0 else (1 + Fraction(mt, 8)) * Fraction(2) ** (e - 7)
                acc += Fraction(float(x[i, kk])) * v * sc
            exact = acc * (Fraction(float(tb)) if tb is not None else 1)
            assert abs(Fraction(C[i, j]) - exact) <= abs(exact) * Fraction(1, 2 ** 40) + Fraction(1, 2 ** 80)


def test_w4a16_equals_w4a4_on_quantized_activations():
    # when the activations are exactly an NVFP4 tensor's values, W4A16 and
    # W4A4 compute the same product (tensor scale 1: the values v * E4M3 have
    # at most 6 significant bits, so float32 holds them exactly)
    rng = np.random.default_rng(23)
    x0 = rng.standard_normal((4, 128)).astype(np.float32)
    w = (rng.standard_normal((6, 128)) * 0.02).astype(np.float32)
    pa, sa, ta = oracle.nvfp4_quantize(x0, np.float32(1.0))
    x = oracle.dequantize("nvfp4", pa, sa, ta, "f32")
    assert np.array_equal(oracle.dequantize_exact_f64("nvfp4", pa, sa, ta), x.astype(np.float64))
    pb, sb, tb = oracle.nvfp4_quantize(w)
    a = oracle.gemm_w4a16_ref("nvfp4", x, pb, sb, tb)
    b = oracle.gemm_ref("nvfp4", pa, sa, ta, pb, sb, tb)
    assert np.allclose(a, b, rtol=1e-13, atol=1e-300)
