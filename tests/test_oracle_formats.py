"""Pins for the oracle's element and scale codecs (CPU only).

Each test checks the oracle against something other than itself: the value
set and range the pages give for E2M1, a brute-force nearest-value search,
torch's float8_e4m3fn (a library routine) and math.ldexp.
"""

import math
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle


# --- E2M1 ------------------------------------------------------------------

def test_e2m1_value_set_and_range():
    # 1 sign, 2 exponent, 1 mantissa bit with range about +-6 (aisyndicate.ch
    # "FP4 auf Blackwell", section on the formats; pimento.cloud "FP8, NVFP4
    # czy AWQ?", section on the formats): 16 codes, 8 magnitudes
    # {0, .5, 1, 1.5, 2, 3, 4, 6}, max exactly 6.
    vals = oracle.e2m1_decode(np.arange(16))
    assert sorted(set(np.abs(vals).tolist())) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert np.max(vals) == 6.0 and np.min(vals) == -6.0
    # codes 8..15 are the negatives of 0..7 (sign bit 3)
    assert np.array_equal(vals[8:], -vals[:8])
    assert np.signbit(vals[8])          # code 8 is -0.0
    # magnitudes increase with the code (monotone encoding)
    assert np.all(np.diff(vals[:8]) > 0)
    # the bit fields: exponent bits 2..1, mantissa bit 0; normal codes
    # (e >= 1) are 2^(e-1) * (1 + m/2)
    for c in range(2, 8):
        e, m = c >> 1, c & 1
        assert vals[c] == 2.0 ** (e - 1) * (1 + m / 2)


def _brute_force_e2m1(q):
    """Nearest of the 8 magnitudes, ties to the code with mantissa bit 0,
    anything beyond 6 saturating to 6; sign copied."""
    mags = [Fraction(m) for m in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]
    out = []
    for v in np.asarray(q, dtype=np.float32).tolist():
        a = abs(Fraction(v))
        dist = [abs(a - m) for m in mags]
        best = min(dist)
        cands = [i for i, d in enumerate(dist) if d == best]
        code = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
        sign = 8 if math.copysign(1.0, v) < 0 else 0
        out.append(code | sign)
    return np.array(out, dtype=np.uint8)


def test_e2m1_encode_matches_brute_force():
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float32)
    mids = (mags[:-1] + mags[1:]) / 2
    pts = np.concatenate([mags, mids, [6.5, 7, 8, 100, 1e30, 1e-30, 1e-45]]).astype(np.float32)
    # every point, and its fp32 neighbours one ulp away
    near = np.concatenate([pts, np.nextafter(pts, np.float32(np.inf)),
                           np.nextafter(pts, np.float32(0))])
    rng = np.random.default_rng(0)
    rand = rng.uniform(-8, 8, 4000).astype(np.float32)
    q = np.concatenate([near, -near, rand, np.float32([0.0, -0.0])]).astype(np.float32)
    assert np.array_equal(oracle.e2m1_encode(q), _brute_force_e2m1(q))


def test_e2m1_ties_go_to_even_code():
    ties = np.float32([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    assert oracle.e2m1_encode(ties).tolist() == [0, 2, 2, 4, 4, 6, 6]
    assert oracle.e2m1_encode(-ties).tolist() == [8, 10, 10, 12, 12, 14, 14]


# --- E4M3 ------------------------------------------------------------------

def _torch_e4m3_values(codes):
    t = torch.tensor(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float32).numpy()


def test_e4m3_decode_matches_torch():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(oracle.e4m3_decode(codes), _torch_e4m3_values(codes))
    assert np.isnan(oracle.e4m3_decode([0x7F, 0xFF])).all()
    assert oracle.e4m3_decode([0x7E])[0] == 448.0      # largest finite
    assert oracle.e4m3_decode([0x01])[0] == 2.0 ** -9  # smallest subnormal


def test_e4m3_encode_matches_torch_in_range():
    grid = oracle.e4m3_decode(np.arange(127)).astype(np.float64)
    mids = (grid[:-1] + grid[1:]) / 2
    rng = np.random.default_rng(1)
    u = np.concatenate([
        grid, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
        rng.uniform(0, 448, 20000), np.exp2(rng.uniform(-14, 8.8, 20000)),
    ]).astype(np.float32)
    u = u[(u >= 0) & (u <= 448)]
    ref = torch.from_numpy(u).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode(u), ref)


def test_e4m3_encode_saturates_without_nan():
    big = np.float32([448.0, 449.0, 464.0, 480.0, 1e6, np.inf])
    assert oracle.e4m3_encode(big).tolist() == [0x7E] * 6
    assert oracle.e4m3_encode_signed(-big).tolist() == [0xFE] * 6


# --- E8M0 ------------------------------------------------------------------

def test_e8m0_is_a_power_of_two():
    codes = np.arange(255)
    assert np.array_equal(oracle.e8m0_decode(codes), [math.ldexp(1.0, int(c) - 127) for c in codes])
    # same as an fp32 whose exponent field is the code (normal range)
    for c in (1, 100, 127, 200, 254):
        assert oracle.e8m0_decode([c])[0] == struct.unpack("<f", struct.pack("<I", c << 23))[0]
    assert np.isnan(oracle.e8m0_decode([255])[0])
    assert oracle.e8m0_encode_exponent([-127, 0, 127]).tolist() == [0, 127, 254]
    with pytest.raises(ValueError):
        oracle.e8m0_encode_exponent([128])


# --- storage cost ----------------------------------------------------------

def test_storage_bits_per_value():
    # ~4.5 bits per value for NVFP4, ~3.5x smaller than FP16 and ~1.8x than
    # FP8 (pimento.cloud, section on the formats); FP4 is 0.5 byte per
    # parameter (cloudmagazin.com, the table of formats).
    x = np.ones((4, 1024), dtype=np.float32)
    packed, sb, s_t = oracle.nvfp4_quantize(x)
    nbytes = packed.nbytes + sb.nbytes
    bits = 8 * nbytes / x.size
    assert packed.nbytes / x.size == 0.5
    assert bits == 4.5
    assert round(16 / bits, 1) == 3.6 and 3.5 <= 16 / bits < 3.6
    assert round(8 / bits, 1) == 1.8
    pm, sm = oracle.mxfp4_quantize(x)
    assert 8 * (pm.nbytes + sm.nbytes) / x.size == 4.25
    assert sb.shape == (4, 1024 // 16) and sm.shape == (4, 1024 // 32)
