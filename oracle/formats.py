"""Element and scale encodings used by NVFP4 and MXFP4 (oracle, test-only).

E2M1 (the 4-bit element): 1 sign bit, 2 exponent bits, 1 mantissa bit, range
about +-6 -- aisyndicate.ch "FP4 auf Blackwell", section "Was NVFP4 von
frueheren 4-Bit-Formaten unterscheidet"; pimento.cloud "FP8, NVFP4 czy AWQ?",
section "Czym roznia sie FP8, NVFP4, MXFP4 i AWQ?".  The exponent bias that
makes the largest magnitude 6 is 1; with the usual subnormal rule this gives
the magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}.

E4M3 (the NVFP4 block scale and the FP8 output of the KV dequantization):
4 exponent and 3 mantissa bits after Micikevicius et al., cited on the
pimento.cloud page in the same section.  Bias 7, subnormals, no infinity,
the all-ones pattern S.1111.111 is NaN, largest finite 448.

E8M0 (the MXFP4 block scale): a bare power of two, OCP Microscaling, named on
both pages above.  Bias 127, code 255 is NaN.

Rounding is not stated on the pages.  Everything here rounds to nearest with
ties to even and saturates instead of overflowing (E2M1 and E4M3 scales have
no infinity to overflow into).
"""

import math

import numpy as np
import torch

# Magnitude of E2M1 code 0..7: code = e1 e0 m (exponent bits then mantissa).
# e == 0 -> subnormal m * 0.5 ; e > 0 -> 2**(e-1) * (1 + m/2).
E2M1_MAGNITUDES = tuple(
    (m * 0.5) if e == 0 else (2.0 ** (e - 1)) * (1.0 + m / 2.0)
    for e in range(4) for m in range(2)
)


def e2m1_decode(codes):
    """4-bit codes (any integer array, values 0..15) -> float32 values.

    Bit 3 is the sign, bits 2..1 the exponent, bit 0 the mantissa.
    """
    codes = np.asarray(codes, dtype=np.int64)
    mag = np.asarray(E2M1_MAGNITUDES, dtype=np.float32)[codes & 7]
    return np.where((codes & 8) != 0, -mag, mag).astype(np.float32)


def e2m1_encode(q):
    """float32 array -> 4-bit codes (uint8 0..15), round to nearest, ties to
    the even code, saturating at 6.

    Magnitude intervals (a = |q|):
        a <= 0.25        -> 0 (0)      0.25 < a < 0.75 -> 1 (0.5)
        0.75 <= a <= 1.25 -> 2 (1)     1.25 < a < 1.75 -> 3 (1.5)
        1.75 <= a <= 2.5  -> 4 (2)     2.5 < a < 3.5   -> 5 (3)
        3.5 <= a <= 5     -> 6 (4)     a > 5           -> 7 (6, saturating)
    A tie sits on the closed end of the even code's interval.  The sign bit is
    copied from q, so a negative value that rounds to zero keeps its sign.
    """
    q = np.asarray(q, dtype=np.float32)
    a = np.abs(q)
    mag = np.select(
        [a <= 0.25, a < 0.75, a <= 1.25, a < 1.75, a <= 2.5, a < 3.5, a <= 5.0],
        [0, 1, 2, 3, 4, 5, 6],
        default=7,
    ).astype(np.uint8)
    sign = np.signbit(q).astype(np.uint8) << 3
    return (mag | sign).astype(np.uint8)


def e4m3_decode(codes):
    """8-bit E4M3 codes -> float32 values (sign bit 7; 0x7F/0xFF are NaN)."""
    codes = np.asarray(codes, dtype=np.int64)
    e = (codes >> 3) & 15
    m = codes & 7
    sub = m.astype(np.float64) * 2.0 ** -9
    norm = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    mag = np.where(e == 0, sub, norm)
    mag = np.where((codes & 0x7F) == 0x7F, np.nan, mag)
    return np.where((codes & 0x80) != 0, -mag, mag).astype(np.float32)


# The 127 non-negative finite E4M3 values, indexed by code 0..126 (increasing).
_E4M3_GRID = e4m3_decode(np.arange(127)).astype(np.float64)
E4M3_MAX = 448.0


def e4m3_encode(u):
    """Non-negative float32 -> E4M3 code 0..126, nearest value, ties to the
    even code, saturating at 448 (code 0x7E).  Never produces NaN.

    Negative zero maps to code 0; the caller only passes magnitudes.
    """
    u = np.asarray(u, dtype=np.float32).astype(np.float64)
    if np.any(u < 0) or np.any(np.isnan(u)):
        raise ValueError("e4m3_encode takes non-negative, non-NaN magnitudes")
    grid = _E4M3_GRID
    # hi = first grid index with grid[hi] >= u ; lo = hi - 1.
    hi = np.searchsorted(grid, u, side="left")
    hi = np.clip(hi, 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    glo, ghi = grid[lo], grid[hi]
    mid = (glo + ghi) / 2.0          # exact in float64
    pick_hi = (u > mid) | ((u == mid) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(u >= grid[126], 126, code)   # saturate (covers +inf)
    code = np.where(u <= 0.0, 0, code)
    return code.astype(np.uint8)


def e4m3_encode_signed(y):
    """float32 -> signed E4M3 byte (fp8 output), RNE, saturating to +-448."""
    y = np.asarray(y, dtype=np.float32)
    mag = e4m3_encode(np.abs(y))
    return (mag | (np.signbit(y).astype(np.uint8) << 7)).astype(np.uint8)


def e8m0_decode(codes):
    """E8M0 codes -> float64 powers of two 2**(c-127); 255 is NaN."""
    codes = np.asarray(codes, dtype=np.int64)
    val = np.exp2(codes.astype(np.float64) - 127.0)
    return np.where(codes == 255, np.nan, val)


def e8m0_encode_exponent(k):
    """Integer exponent k in [-127, 127] -> E8M0 code k + 127."""
    k = np.asarray(k, dtype=np.int64)
    if np.any(k < -127) or np.any(k > 127):
        raise ValueError("E8M0 exponent out of range")
    return (k + 127).astype(np.uint8)


def bf16_round(y):
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even,
    via torch's own conversion (a library routine)."""
    t = torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def f16_round(y):
    """float32 -> IEEE half bit patterns (uint16), round to nearest even."""
    return np.asarray(y, dtype=np.float32).astype(np.float16).view(np.uint16)


def ldexp1(k):
    """2**k as a Python float (exact for the exponents used here)."""
    return math.ldexp(1.0, int(k))
