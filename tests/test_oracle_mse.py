"""Pins for the oracle's MSE-optimal NVFP4 block scale (CPU only).

The block scale minimizing the block's squared error (aisyndicate.ch "FP4 auf
Blackwell", section "Was NVFP4 von frueheren 4-Bit-Formaten unterscheidet").
Checked against a hand-worked golden block, an exhaustive search in exact
rational arithmetic with its own E2M1 rounding, and the invariant that it is
never worse than the amax / 6 scale.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle.formats import E2M1_MAGNITUDES

from test_oracle_quant import _hex, _load, _num


def _nearest_e2m1(q):
    """E2M1 value for float q by brute force: the nearest magnitude, ties to
    the even code (codes 0, 2, 4, 6), saturating; sign kept."""
    mags = [float(m) for m in E2M1_MAGNITUDES]
    a = abs(float(q))
    best = None
    for code, m in enumerate(mags):
        dist = abs(a - m)
        if best is None or dist < best[0] or (dist == best[0] and code % 2 == 0):
            best = (dist, code, m)
    return -best[2] if q < 0 else best[2]


def _exact_errors(block, s_t):
    """Exact squared error of every candidate byte 1..126 for one block."""
    out = {}
    for c in range(1, 127):
        S_b = np.float32(oracle.e4m3_decode(np.array([c], dtype=np.uint8))[0] * np.float32(s_t))
        if S_b == 0:
            continue
        r_b = np.float32(np.float32(1.0) / S_b)
        if not np.isfinite(r_b):
            continue
        S = Fraction(float(S_b))
        err = Fraction(0)
        for x in block:
            q = np.float32(np.float32(x) * r_b)
            v = _nearest_e2m1(q)
            err += (Fraction(float(x)) - Fraction(v) * S) ** 2
        out[c] = err
    return out


def test_mse_worked_examples(golden_dir):
    g = _load(golden_dir, "nvfp4_mse_worked.json")
    for case in g["cases"]:
        x = np.array([[_num(v) for v in r] for r in case["x"]], dtype=np.float32)
        packed, sb, s_t = oracle.nvfp4_quantize_mse(x, tensor_scale=case["tensor_scale"])
        assert np.array_equal(sb, _hex(case["scales"])), case["name"]
        assert np.array_equal(packed, _hex(case["packed"])), case["name"]
        if "error" in case:
            errs = _exact_errors(x[0, :16], case["tensor_scale"])
            assert errs[int(sb[0, 0])] == Fraction(case["error"])
            assert min(errs.values()) == Fraction(case["error"])
            _, sb6, _ = oracle.nvfp4_quantize(x, tensor_scale=case["tensor_scale"])
            assert errs[int(sb6[0, 0])] == Fraction(case["amax6_error"])


@pytest.mark.parametrize("dist", ["normal", "student_t", "uniform"])
def test_mse_is_the_exact_argmin(dist):
    rng = np.random.default_rng({"normal": 1, "student_t": 2, "uniform": 3}[dist])
    if dist == "normal":
        x = rng.standard_normal((2, 64))
    elif dist == "student_t":
        x = rng.standard_t(3, (2, 64))
    else:
        x = rng.uniform(-2, 2, (2, 64))
    x = x.astype(np.float32)
    packed, sb, s_t = oracle.nvfp4_quantize_mse(x)
    codes = oracle.unpack_nibbles(packed)
    for r in range(x.shape[0]):
        for b in range(x.shape[1] // 16):
            block = x[r, 16 * b:16 * b + 16]
            errs = _exact_errors(block, s_t)
            best = min(errs.values())
            chosen = errs[int(sb[r, b])]
            # the float64 decision may split a near tie, never more
            assert chosen <= best * (1 + Fraction(1, 10 ** 12)), (r, b)
            # exact ties go to the smallest byte
            firsts = [c for c, e in sorted(errs.items()) if e == best]
            if chosen == best:
                assert int(sb[r, b]) == firsts[0]
            # the codes are those of the chosen scale
            S_b = np.float32(oracle.e4m3_decode(sb[r:r + 1, b:b + 1])[0, 0] * s_t)
            r_b = np.float32(np.float32(1.0) / S_b)
            want = [_nearest_e2m1(np.float32(v * r_b)) for v in block]
            got = oracle.e2m1_decode(codes[r, 16 * b:16 * b + 16])
            assert np.array_equal(np.abs(got), np.abs(np.array(want, dtype=np.float32)))


def test_mse_never_worse_than_amax6():
    rng = np.random.default_rng(7)
    x = (rng.standard_t(3, (64, 256)) * 0.02).astype(np.float32)
    x[:, ::37] *= 40.0                                     # outlier channels
    p_mse, sb_mse, s_t = oracle.nvfp4_quantize_mse(x)
    p_def, sb_def, s_t2 = oracle.nvfp4_quantize(x)
    assert s_t == s_t2
    xb = x.reshape(64, 16, 16)

    def err(packed, sb):
        codes = oracle.unpack_nibbles(packed).reshape(64, 16, 16)
        S_b = (oracle.e4m3_decode(sb) * s_t).astype(np.float32)
        return oracle.nvfp4_mse_block_error(xb, codes, S_b)

    e_mse, e_def = err(p_mse, sb_mse), err(p_def, sb_def)
    assert np.all(e_mse <= e_def)
    assert np.mean(e_mse < e_def) > 0.2          # the search changes many blocks
    # whole-tensor error shrinks too
    assert e_mse.sum() < 0.97 * e_def.sum()     # about 5 % less on this data


def test_mse_given_tensor_scale_and_zero_tensor():
    x = np.zeros((3, 32), dtype=np.float32)
    packed, sb, s_t = oracle.nvfp4_quantize_mse(x)
    assert s_t == np.float32(1.0)
    assert not sb.any() and not packed.any()
    y = np.full((1, 16), 3.0, dtype=np.float32)
    packed, sb, s_t = oracle.nvfp4_quantize_mse(y, tensor_scale=np.float32(0.5))
    assert s_t == np.float32(0.5)
    S = oracle.e4m3_decode(sb)[0, 0] * 0.5
    v = oracle.e2m1_decode(oracle.unpack_nibbles(packed))[0]
    assert np.all(v * S == 3.0)                   # 3.0 is representable: error 0
