"""NVFP4 and MXFP4 quantization and dequantization (oracle, test-only).

Formats (aisyndicate.ch "FP4 auf Blackwell", section "Was NVFP4 von frueheren
4-Bit-Formaten unterscheidet"; pimento.cloud "FP8, NVFP4 czy AWQ?", section
"Czym roznia sie FP8, NVFP4, MXFP4 i AWQ?"):
  * NVFP4: blocks of 16 E2M1 values, one E4M3 scale per block and a second,
    FP32 scale per tensor.
  * MXFP4: blocks of 32 E2M1 values sharing one power-of-two (E8M0) scale.
Blocks run along the last (reduction) dimension of a row-major [rows, k]
tensor.  Packed codes: byte j of a row holds element 2j in its low nibble and
element 2j+1 in its high nibble.  Scales: one byte per block, row-major
[rows, k / block].

Readings taken where the pages are silent (each is a stated choice):
  * NVFP4 tensor scale s_t = fp32(A / 2688) with A the tensor's max |x|, so
    that the block holding A gets the largest E4M3 scale, 448 (2688 = 6*448);
    s_t = 1 when that quotient is 0 (all-zero tensor).
  * NVFP4 block scale: nearest E4M3 to a_b / (6 s_t), a_b the block's max |x|
    (amax / 6 scaling); nvfp4_quantize_mse is the MSE-searching variant the
    aisyndicate.ch page describes.
  * Element scaling: one correctly rounded reciprocal per block,
    r_b = fp32(1 / S_b) with S_b = fp32(dec(sb) * s_t), then one fp32
    multiply per element, q = fp32(x * r_b).  A block whose S_b is 0 or
    whose reciprocal overflows keeps only the sign bits.
  * MXFP4 scale: "rounded to the next power of two" read as rounding UP: the
    smallest 2**k with a_b <= 6 * 2**k, so no element is clipped.
"""

import numpy as np

from .formats import (
    e2m1_decode,
    e2m1_encode,
    e4m3_decode,
    e4m3_encode,
    e4m3_encode_signed,
    e8m0_decode,
    e8m0_encode_exponent,
    bf16_round,
    f16_round,
)

NV_BLOCK = 16
MX_BLOCK = 32
E2M1_MAX = np.float32(6.0)
NV_TSCALE_DIVISOR = np.float32(6.0 * 448.0)   # 2688


def _as_f32_2d(x, block):
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 2:
        raise ValueError("expected a [rows, k] array")
    if x.shape[1] % block != 0:
        raise ValueError("k must be a multiple of the block size")
    return x


def pack_nibbles(codes):
    """[rows, k] codes 0..15 -> [rows, k/2] bytes, even element in the low
    nibble."""
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed):
    """[rows, k/2] bytes -> [rows, k] codes."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty((packed.shape[0], packed.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = packed & 0xF
    out[:, 1::2] = packed >> 4
    return out


def nvfp4_tensor_scale_from_amax(a):
    """FP32 second-level scale for a tensor whose max |x| is a:
    fp32(a / 2688), or 1.0 when that is zero."""
    s_t = np.float32(np.float32(a) / NV_TSCALE_DIVISOR)
    if s_t == 0:
        s_t = np.float32(1.0)
    return s_t


def nvfp4_tensor_scale(x):
    """FP32 second-level scale of a tensor x."""
    a = np.float32(np.max(np.abs(np.asarray(x, dtype=np.float32)))) if np.size(x) else np.float32(0)
    return nvfp4_tensor_scale_from_amax(a)


def nvfp4_quantize(x, tensor_scale=None):
    """NVFP4 quantization of a [rows, k] array.

    tensor_scale=None computes the per-tensor scale from x (dynamic scaling);
    a given float32 value is used as is.
    Returns (packed codes uint8 [rows, k/2], scale bytes uint8 [rows, k/16],
    tensor scale float32).
    """
    x = _as_f32_2d(x, NV_BLOCK)
    rows, k = x.shape
    s_t = nvfp4_tensor_scale(x) if tensor_scale is None else np.float32(tensor_scale)
    d = np.float32(E2M1_MAX * s_t)

    xb = x.reshape(rows, k // NV_BLOCK, NV_BLOCK)
    a_b = np.max(np.abs(xb), axis=2)                       # exact
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        u_b = (a_b / d).astype(np.float32)                 # one fp32 division
    sb = e4m3_encode(u_b)
    with np.errstate(over="ignore", under="ignore"):
        S_b = (e4m3_decode(sb) * s_t).astype(np.float32)
    with np.errstate(divide="ignore", over="ignore"):
        r_b = (np.float32(1.0) / S_b).astype(np.float32)
    usable = (S_b != 0) & np.isfinite(r_b)
    r_b = np.where(usable, r_b, np.float32(0.0)).astype(np.float32)

    with np.errstate(over="ignore", under="ignore", invalid="ignore"):
        q = (xb * r_b[:, :, None]).astype(np.float32)      # one fp32 multiply
    codes = e2m1_encode(q)
    # unusable blocks: magnitude 0, sign bit of x kept
    sign_only = (np.signbit(xb).astype(np.uint8) << 3)
    codes = np.where(usable[:, :, None], codes, sign_only).astype(np.uint8)
    return pack_nibbles(codes.reshape(rows, k)), sb.astype(np.uint8), np.float32(s_t)


def nvfp4_mse_block_error(xb, codes, S_b):
    """Squared error of quantized blocks: sum_i (x_i - v_i S_b)^2 in float64,
    one IEEE rounding per operation, summed in element order i = 0 .. 15.
    xb float32 [..., 16]; codes E2M1 codes of the same shape; S_b the float32
    block scale (broadcastable to [...]).  v_i S_b is exact in float64 (2 and
    24 significant bits)."""
    x64 = np.asarray(xb, dtype=np.float32).astype(np.float64)
    v = e2m1_decode(codes).astype(np.float64)
    d = x64 - v * np.asarray(S_b, dtype=np.float32).astype(np.float64)[..., None]
    err = np.zeros(d.shape[:-1], dtype=np.float64)
    for i in range(d.shape[-1]):
        err = err + d[..., i] * d[..., i]
    return err


def nvfp4_quantize_mse(x, tensor_scale=None):
    """NVFP4 quantization with each block scale chosen to minimize the
    block's squared error.

    aisyndicate.ch "FP4 auf Blackwell", section "Was NVFP4 von frueheren
    4-Bit-Formaten unterscheidet": instead of jumping to a power of two, the
    NVFP4 scaling looks for the factor that minimizes the mean squared error
    over the 16 values of a block.  Readings (where the page is silent):
      * candidates are all positive finite E4M3 scale bytes 1 .. 126 under the
        same tensor scale s_t as nvfp4_quantize;
      * a candidate quantizes the block exactly as nvfp4_quantize does for that
        byte (S_b = fp32(dec(sb) s_t), r_b = fp32(1 / S_b), q = fp32(x r_b),
        E2M1 round to nearest even, saturating);
      * its error is nvfp4_mse_block_error (float64, fixed order), the float
        precision that decides the byte on both sides;
      * the least error wins, ties going to the smaller byte (the smaller
        scale); a block whose max |x| is 0 keeps byte 0 and sign-only codes,
        as in nvfp4_quantize.
    Returns (packed codes, scale bytes, tensor scale) like nvfp4_quantize.
    """
    x = _as_f32_2d(x, NV_BLOCK)
    rows, k = x.shape
    s_t = nvfp4_tensor_scale(x) if tensor_scale is None else np.float32(tensor_scale)
    xb = x.reshape(rows, k // NV_BLOCK, NV_BLOCK)
    best_err = np.full(xb.shape[:2], np.inf)
    best_sb = np.zeros(xb.shape[:2], dtype=np.uint8)
    best_codes = np.zeros(xb.shape, dtype=np.uint8)
    for c in range(1, 127):                              # ascending scale
        sb = np.uint8(c)
        with np.errstate(over="ignore", under="ignore"):
            S_b = np.float32(e4m3_decode(np.array([sb], dtype=np.uint8))[0] * s_t)
        with np.errstate(divide="ignore", over="ignore"):
            r_b = np.float32(np.float32(1.0) / S_b)
        if S_b == 0 or not np.isfinite(r_b):
            continue
        with np.errstate(over="ignore", under="ignore", invalid="ignore"):
            q = (xb * r_b).astype(np.float32)
        codes = e2m1_encode(q)
        err = nvfp4_mse_block_error(xb, codes, np.full(xb.shape[:2], S_b, dtype=np.float32))
        better = err < best_err
        best_err = np.where(better, err, best_err)
        best_sb = np.where(better, sb, best_sb).astype(np.uint8)
        best_codes = np.where(better[:, :, None], codes, best_codes).astype(np.uint8)
    a_b = np.max(np.abs(xb), axis=2)
    zero = a_b == 0
    best_sb = np.where(zero, np.uint8(0), best_sb).astype(np.uint8)
    sign_only = (np.signbit(xb).astype(np.uint8) << 3)
    best_codes = np.where(zero[:, :, None], sign_only, best_codes).astype(np.uint8)
    return pack_nibbles(best_codes.reshape(rows, k)), best_sb, np.float32(s_t)


def mxfp4_block_exponent(a_b):
    """Smallest integer k with a_b <= 6 * 2**k, clamped to [-127, 127]
    (a_b > 0).  From frexp: a_b = m * 2**e, m in [0.5, 1): k = e-3 when
    m <= 0.75, else e-2."""
    a_b = np.asarray(a_b, dtype=np.float32)
    m, e = np.frexp(a_b)
    k = np.where(m <= 0.75, e - 3, e - 2)
    return np.clip(k, -127, 127).astype(np.int64)


def mxfp4_quantize(x):
    """MXFP4 quantization of a [rows, k] array.

    Returns (packed codes uint8 [rows, k/2], E8M0 scale bytes uint8
    [rows, k/32]).  An all-zero block gets scale code 0 and sign-only codes.
    """
    x = _as_f32_2d(x, MX_BLOCK)
    rows, k = x.shape
    xb = x.reshape(rows, k // MX_BLOCK, MX_BLOCK)
    a_b = np.max(np.abs(xb), axis=2)
    nonzero = a_b > 0
    kexp = np.where(nonzero, mxfp4_block_exponent(np.where(nonzero, a_b, 1.0)), -127)
    sc = e8m0_encode_exponent(kexp)
    inv = np.exp2(-kexp.astype(np.float64)).astype(np.float32)   # 2**-k, exact
    with np.errstate(under="ignore"):
        q = (xb * inv[:, :, None]).astype(np.float32)             # exact scaling
    codes = e2m1_encode(q)
    sign_only = (np.signbit(xb).astype(np.uint8) << 3)
    codes = np.where(nonzero[:, :, None], codes, sign_only).astype(np.uint8)
    return pack_nibbles(codes.reshape(rows, k)), sc.astype(np.uint8)


def dequantize(fmt, packed, scales, tensor_scale=None, out_dtype="f32"):
    """Packed codes + scales -> values.

    NVFP4: t = fp32(v * dec(sb)) (exact: at most 6 significant bits), then
    y = fp32(t * s_t), i.e. the exact product rounded once to fp32.
    MXFP4: y = v * 2**(c-127) (exact).
    The fp32 result is then converted: "f32" as is, "bf16"/"f16" round to
    nearest even (returned as uint16 bit patterns), "e4m3" round to nearest
    even saturating to +-448 (uint8 bytes) -- the FP8 form the hyper.ai NVFP4
    KV-cache story says the cache is dequantized to before attention.
    """
    codes = unpack_nibbles(packed)
    rows, k = codes.shape
    v = e2m1_decode(codes)
    if fmt == "nvfp4":
        if tensor_scale is None:
            raise ValueError("NVFP4 needs a tensor scale")
        sbv = np.repeat(e4m3_decode(scales), NV_BLOCK, axis=1)
        t = (v * sbv).astype(np.float32)
        with np.errstate(over="ignore", under="ignore"):
            y = (t * np.float32(tensor_scale)).astype(np.float32)
    elif fmt == "mxfp4":
        with np.errstate(over="ignore"):
            sv = np.repeat(e8m0_decode(scales), MX_BLOCK, axis=1)
            y = (v.astype(np.float64) * sv).astype(np.float32)
    else:
        raise ValueError(fmt)
    if out_dtype == "f32":
        return y
    if out_dtype == "bf16":
        return bf16_round(y)
    if out_dtype == "f16":
        return f16_round(y)
    if out_dtype == "e4m3":
        return e4m3_encode_signed(y)
    raise ValueError(out_dtype)


def dequantize_exact_f64(fmt, packed, scales, tensor_scale=None):
    """The exact dequantized values v * scale (* s_t) in float64 (at most 30
    significant bits, so float64 holds them exactly)."""
    v = e2m1_decode(unpack_nibbles(packed)).astype(np.float64)
    if fmt == "nvfp4":
        s = np.repeat(e4m3_decode(scales).astype(np.float64), NV_BLOCK, axis=1)
        return v * s * float(np.float32(tensor_scale))
    if fmt == "mxfp4":
        return v * np.repeat(e8m0_decode(scales), MX_BLOCK, axis=1)
    raise ValueError(fmt)
