"""FP4 KV cache: append and decode attention (oracle).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
CPU-baseline leg of the benchmark, never by the library.

hyper.ai story on the NVFP4 KV cache: new K and V vectors are written into
the cache in NVFP4 form, and the cached K and V are dequantized to FP8 before
the attention is computed.  What is computed here:

  * append: row i of the new K (or V) of sequence b goes to cache position
    positions[b] + i, quantized with the format's own rule; NVFP4 uses a
    given tensor scale, because a cache cannot re-scale the tokens it already
    holds as new ones arrive.  Rows whose position falls outside the cache
    are dropped.
  * attention: one new query token per sequence attends over the first
    seq_lens[b] cached tokens with the usual scaled dot-product softmax
    attention.  K and V enter as the FP8 E4M3 values that `dequantize(...,
    out_dtype="e4m3")` produces from the cache, i.e. exactly the FP8 form the
    story describes.  Grouped-query attention: query head j reads K/V head
    j // G with G = q_heads / kv_heads.

The arithmetic on those FP8 values (dot products, softmax, weighted sum) is
done in float64 with NumPy: it is the exact attention of the FP8 cache up to
float64 rounding.
"""

import numpy as np

from .formats import e4m3_decode
from .quant import NV_BLOCK, MX_BLOCK, nvfp4_quantize, mxfp4_quantize, dequantize


def _block(fmt):
    if fmt == "nvfp4":
        return NV_BLOCK
    if fmt == "mxfp4":
        return MX_BLOCK
    raise ValueError(fmt)


def kv_append_ref(fmt, cache_codes, cache_scales, kv_new, positions, tensor_scale=None):
    """Copies of the cache arrays with kv_new written in.

    cache_codes [B, H, T_max, D/2] uint8, cache_scales [B, H, T_max, D/block]
    uint8, kv_new [B, H, T_new, D] (the exact values, e.g. bf16 widened to
    float32), positions [B] integers.  NVFP4 needs `tensor_scale`.
    """
    codes = np.array(cache_codes, dtype=np.uint8, copy=True)
    scales = np.array(cache_scales, dtype=np.uint8, copy=True)
    kv_new = np.asarray(kv_new, dtype=np.float32)
    B, H, Tn, D = kv_new.shape
    t_max = codes.shape[2]
    if fmt == "nvfp4" and tensor_scale is None:
        raise ValueError("the NVFP4 cache needs its given tensor scale")
    _block(fmt)
    for b in range(B):
        for i in range(Tn):
            p = int(positions[b]) + i
            if p < 0 or p >= t_max:
                continue
            rows = kv_new[b, :, i, :]                      # [H, D]
            if fmt == "nvfp4":
                c, s, _ = nvfp4_quantize(rows, tensor_scale=tensor_scale)
            else:
                c, s = mxfp4_quantize(rows)
            codes[b, :, p, :] = c
            scales[b, :, p, :] = s
    return codes, scales


def kv_fp8_values(fmt, codes, scales, tensor_scale=None):
    """Cache rows [..., D/2] codes + [..., D/block] scales -> float64 values
    of the FP8 E4M3 bytes they dequantize to (same leading shape, last dim D)."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    lead = codes.shape[:-1]
    d = codes.shape[-1] * 2
    c2 = codes.reshape(-1, codes.shape[-1])
    s2 = scales.reshape(-1, scales.shape[-1])
    fp8 = dequantize(fmt, c2, s2, tensor_scale, out_dtype="e4m3")
    return e4m3_decode(fp8).astype(np.float64).reshape(*lead, d)


def attention_decode_ref(fmt, q, k_codes, k_scales, k_tscale, v_codes, v_scales,
                         v_tscale, seq_lens, softmax_scale, with_abs=False):
    """Decode attention over the FP8 form of an FP4 KV cache.

    q [B, Hq, D] (exact values); caches [B, Hkv, T_max, ...]; seq_lens [B].
    out[b, j] = sum_t p_t V[t] with p = softmax(softmax_scale * K q) over
    t < seq_lens[b], K and V the FP8 values of kv head j // G; a sequence of
    length 0 gives zeros.  with_abs also returns the two scales of the
    rounding error of a weighted sum, same shape: sum_t p_t |V[t]| (errors
    relative to each weight) and max_t p_t * sum_t |V[t]| (errors absolute
    against the largest weight).
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv = k_codes.shape[1]
    if Hq % Hkv:
        raise ValueError("q_heads must be a multiple of kv_heads")
    G = Hq // Hkv
    scale = float(np.float32(softmax_scale))
    out = np.zeros((B, Hq, D), dtype=np.float64)
    absw = np.zeros((B, Hq, D), dtype=np.float64)
    flat = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        if L <= 0:
            continue
        for h in range(Hkv):
            K = kv_fp8_values(fmt, k_codes[b, h, :L], k_scales[b, h, :L], k_tscale)
            V = kv_fp8_values(fmt, v_codes[b, h, :L], v_scales[b, h, :L], v_tscale)
            for j in range(G):
                hq = h * G + j
                s = (K @ q[b, hq]) * scale
                w = np.exp(s - np.max(s))
                w /= np.sum(w)
                out[b, hq] = w @ V
                absw[b, hq] = w @ np.abs(V)
                flat[b, hq] = np.max(w) * np.sum(np.abs(V), axis=0)
    if with_abs:
        return out, absw, flat
    return out
