"""Thin Python binding of libfp4.so (include/fp4.h) for torch tensors.

Argument marshalling only: every step of the computation runs in the HIP
kernels of libfp4.so.  torch supplies device memory and the current stream.
There is no fallback: if the library is missing or a call fails, an error is
raised.
"""

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfp4.so")

NVFP4, MXFP4 = 0, 1
F32, BF16, F16, E4M3 = 0, 1, 2, 3
TSCALE_COMPUTE, TSCALE_GIVEN = 0, 1
OK, EINVAL, EUNSUPPORTED, EHIP = 0, 1, 2, 3

FORMATS = {"nvfp4": NVFP4, "mxfp4": MXFP4}
BLOCK = {NVFP4: 16, MXFP4: 32}
_IN_DTYPES = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}
_OUT_DTYPES = {"f32": (F32, torch.float32), "bf16": (BF16, torch.bfloat16),
               "f16": (F16, torch.float16), "e4m3": (E4M3, torch.float8_e4m3fn)}

EXPORTS = ("fp4_status_string", "fp4_quantize_workspace_size", "fp4_quantize",
           "fp4_hadamard_quantize", "fp4_dequantize", "fp4_gemm_workspace_size",
           "fp4_gemm", "fp4_quantize_gemm_workspace_size", "fp4_quantize_gemm",
           "fp4_quantize_mse", "fp4_gemm_w4a16", "fp4_kv_append",
           "fp4_attention_workspace_size", "fp4_attention_decode", "fp4_gptq_workspace_size",
           "fp4_gptq_quantize", "fp4_quantize_noalloc", "fp4_gemm_w4a16_workspace_size")

_lib = None


class Fp4Error(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__("%s: %s" % (what, lib().fp4_status_string(status).decode()))


def lib():
    """Load libfp4.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libfp4.so is not built (%s); run "
                           "python -m microscaled_fp4_quantization_amd.build" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    L.fp4_status_string.argtypes = [i32]
    L.fp4_status_string.restype = ctypes.c_char_p
    L.fp4_quantize_workspace_size.argtypes = [i32, i32, i64, i64]
    L.fp4_quantize_workspace_size.restype = sz
    for name in ("fp4_quantize", "fp4_hadamard_quantize"):
        f = getattr(L, name)
        f.argtypes = [i32, vp, i32, i64, i64, vp, vp, vp, i32, vp, sz, vp]
        f.restype = i32
    L.fp4_quantize_noalloc.argtypes = [i32, vp, i32, i64, i64, vp, vp, vp, i32, vp]
    L.fp4_quantize_noalloc.restype = i32
    L.fp4_quantize_mse.argtypes = [vp, i32, i64, i64, vp, vp, vp, i32, vp, sz, vp]
    L.fp4_quantize_mse.restype = i32
    L.fp4_gemm_w4a16.argtypes = [i32, vp, i32, i64, i64, i64, vp, vp, vp, vp, i32, vp, sz, vp]
    L.fp4_gemm_w4a16.restype = i32
    L.fp4_gemm_w4a16_workspace_size.argtypes = [i32, i64, i64, i64]
    L.fp4_gemm_w4a16_workspace_size.restype = sz
    L.fp4_dequantize.argtypes = [i32, vp, vp, vp, i64, i64, vp, i32, vp]
    L.fp4_dequantize.restype = i32
    L.fp4_gemm_workspace_size.argtypes = [i32, i64, i64, i64]
    L.fp4_gemm_workspace_size.restype = sz
    L.fp4_gemm.argtypes = [i32, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, i32, vp, sz, vp]
    L.fp4_gemm.restype = i32
    L.fp4_quantize_gemm_workspace_size.argtypes = [i32, i64, i64, i64]
    L.fp4_quantize_gemm_workspace_size.restype = sz
    L.fp4_quantize_gemm.argtypes = [i32, vp, i32, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, i32,
                                    vp, sz, vp]
    L.fp4_quantize_gemm.restype = i32
    L.fp4_kv_append.argtypes = [i32, vp, i32, i64, i64, i64, i64, vp, vp, vp, vp, i64, vp]
    L.fp4_kv_append.restype = i32
    L.fp4_attention_workspace_size.argtypes = [i64, i64, i64, i64, i64]
    L.fp4_attention_workspace_size.restype = sz
    L.fp4_attention_decode.argtypes = [i32, vp, i32, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp,
                                       i64, vp, ctypes.c_float, vp, i32, vp, sz, vp]
    L.fp4_attention_decode.restype = i32
    L.fp4_gptq_workspace_size.argtypes = [i64, i64, i64]
    L.fp4_gptq_workspace_size.restype = sz
    L.fp4_gptq_quantize.argtypes = [i32, vp, i32, i64, i64, vp, i32, i64, ctypes.c_double, i32,
                                    vp, vp, vp, vp, sz, vp]
    L.fp4_gptq_quantize.restype = i32
    _lib = L
    return L


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _fmt(fmt):
    return FORMATS[fmt] if isinstance(fmt, str) else int(fmt)


def _check(status, what):
    if status != OK:
        raise Fp4Error(status, what)


def quantize(x, fmt="nvfp4", tensor_scale=None, hadamard=False, workspace=None):
    """Quantize a CUDA tensor x [rows, k] (fp32 / bf16 / fp16, contiguous).

    NVFP4: tensor_scale=None computes the FP32 tensor scale from the data;
    a one-element float32 CUDA tensor is used as the given scale.
    Returns (codes uint8 [rows, k/2], scales uint8 [rows, k/block],
    tensor_scale float32 [1] or None for MXFP4).
    """
    f = _fmt(fmt)
    if x.dim() != 2:
        raise ValueError("x must be [rows, k]")
    rows, k = x.shape
    codes = torch.empty((rows, k // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((rows, k // BLOCK[f]), dtype=torch.uint8, device=x.device)
    mode = TSCALE_COMPUTE
    ts = None
    if f == NVFP4:
        if tensor_scale is None:
            ts = torch.empty(1, dtype=torch.float32, device=x.device)
        else:
            ts = tensor_scale
            mode = TSCALE_GIVEN
    L = lib()
    need = L.fp4_quantize_workspace_size(f, mode, rows, k)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    fn = L.fp4_hadamard_quantize if hadamard else L.fp4_quantize
    st = fn(f, _ptr(x), _IN_DTYPES[x.dtype], rows, k, _ptr(codes), _ptr(scales),
            _ptr(ts), mode, _ptr(workspace) if need else None, need, _stream(x))
    _check(st, "fp4_hadamard_quantize" if hadamard else "fp4_quantize")
    return codes, scales, ts


def quantize_mse(x, tensor_scale=None, workspace=None):
    """NVFP4 quantization with the least-squared-error block scale (see
    fp4_quantize_mse).  Arguments and result as quantize(x, "nvfp4", ...)."""
    if x.dim() != 2:
        raise ValueError("x must be [rows, k]")
    rows, k = x.shape
    codes = torch.empty((rows, k // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((rows, k // 16), dtype=torch.uint8, device=x.device)
    if tensor_scale is None:
        ts, mode = torch.empty(1, dtype=torch.float32, device=x.device), TSCALE_COMPUTE
    else:
        ts, mode = tensor_scale, TSCALE_GIVEN
    L = lib()
    need = L.fp4_quantize_workspace_size(NVFP4, mode, rows, k)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    st = L.fp4_quantize_mse(_ptr(x), _IN_DTYPES[x.dtype], rows, k, _ptr(codes), _ptr(scales),
                            _ptr(ts), mode, _ptr(workspace) if need else None, need, _stream(x))
    _check(st, "fp4_quantize_mse")
    return codes, scales, ts


def hadamard_quantize(x, fmt="nvfp4", tensor_scale=None, workspace=None):
    """Blockwise Hadamard (16 for NVFP4, 32 for MXFP4) then quantize."""
    return quantize(x, fmt, tensor_scale, hadamard=True, workspace=workspace)


def dequantize(codes, scales, tensor_scale=None, fmt="nvfp4", out_dtype="f32"):
    """Codes [rows, k/2] + scales (+ tensor scale) -> [rows, k] of out_dtype
    ("f32", "bf16", "f16" or "e4m3")."""
    f = _fmt(fmt)
    rows, k = codes.shape[0], codes.shape[1] * 2
    code, tdt = _OUT_DTYPES[out_dtype]
    out = torch.empty((rows, k), dtype=tdt, device=codes.device)
    st = lib().fp4_dequantize(f, _ptr(codes), _ptr(scales), _ptr(tensor_scale),
                              rows, k, _ptr(out), code, _stream(codes))
    _check(st, "fp4_dequantize")
    return out


def gemm(a, b, fmt="nvfp4", out_dtype="bf16", out=None):
    """C = A B^T for quantized A = (codes [m, k/2], scales, tscale) and
    B = (codes [n, k/2], scales, tscale).  Returns C [m, n]."""
    f = _fmt(fmt)
    ac, asc, at = a
    bc, bsc, bt = b
    m, n, k = ac.shape[0], bc.shape[0], ac.shape[1] * 2
    code, tdt = _OUT_DTYPES[out_dtype]
    if out is None:
        out = torch.empty((m, n), dtype=tdt, device=ac.device)
    L = lib()
    need = L.fp4_gemm_workspace_size(f, m, n, k)
    ws = torch.empty(need, dtype=torch.uint8, device=ac.device) if need else None
    st = L.fp4_gemm(f, m, n, k, _ptr(ac), _ptr(asc), _ptr(at), _ptr(bc), _ptr(bsc),
                    _ptr(bt), _ptr(out), code, _ptr(ws), need, _stream(ac))
    _check(st, "fp4_gemm")
    return out


def gemm_w4a16(x, b, fmt="nvfp4", out_dtype="bf16", out=None):
    """C = X B^T with X [m, k] as it is (bf16 / fp16 / fp32) and the
    quantized weights B = (codes [n, k/2], scales, tscale).  Returns C [m, n]."""
    f = _fmt(fmt)
    if x.dim() != 2:
        raise ValueError("x must be [m, k]")
    m, k = x.shape
    bc, bsc, bt = b
    n = bc.shape[0]
    code, tdt = _OUT_DTYPES[out_dtype]
    if out is None:
        out = torch.empty((m, n), dtype=tdt, device=x.device)
    L = lib()
    need = L.fp4_gemm_w4a16_workspace_size(f, m, n, k)
    ws = torch.empty(need, dtype=torch.uint8, device=x.device) if need else None
    st = L.fp4_gemm_w4a16(f, _ptr(x), _IN_DTYPES[x.dtype], m, n, k, _ptr(bc), _ptr(bsc),
                          _ptr(bt), _ptr(out), code, _ptr(ws), need, _stream(x))
    _check(st, "fp4_gemm_w4a16")
    return out


def quantize_gemm(x, b, fmt="nvfp4", out_dtype="bf16", out=None):
    """Quantize the activations x [m, k] (tensor scale from the data for
    NVFP4) and multiply by the quantized B = (codes [n, k/2], scales, tscale).
    Returns ((codes, scales, tscale) of x, C [m, n]); same results as
    quantize() followed by gemm(), in one launch for the decode shapes."""
    f = _fmt(fmt)
    if x.dim() != 2:
        raise ValueError("x must be [m, k]")
    m, k = x.shape
    bc, bsc, bt = b
    n = bc.shape[0]
    code, tdt = _OUT_DTYPES[out_dtype]
    codes = torch.empty((m, k // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((m, k // BLOCK[f]), dtype=torch.uint8, device=x.device)
    ts = torch.empty(1, dtype=torch.float32, device=x.device) if f == NVFP4 else None
    if out is None:
        out = torch.empty((m, n), dtype=tdt, device=x.device)
    L = lib()
    need = L.fp4_quantize_gemm_workspace_size(f, m, n, k)
    ws = torch.empty(need, dtype=torch.uint8, device=x.device) if need else None
    st = L.fp4_quantize_gemm(f, _ptr(x), _IN_DTYPES[x.dtype], m, n, k, _ptr(codes), _ptr(scales),
                             _ptr(ts), _ptr(bc), _ptr(bsc), _ptr(bt), _ptr(out), code, _ptr(ws),
                             need, _stream(x))
    _check(st, "fp4_quantize_gemm")
    return (codes, scales, ts), out


def kv_cache(batch, heads, t_max, head_dim=128, fmt="nvfp4", device="cuda"):
    """An empty 4-bit KV cache: (codes [batch, heads, t_max, head_dim/2],
    scales [batch, heads, t_max, head_dim/block]), zero-filled."""
    f = _fmt(fmt)
    codes = torch.zeros((batch, heads, t_max, head_dim // 2), dtype=torch.uint8, device=device)
    scales = torch.zeros((batch, heads, t_max, head_dim // BLOCK[f]), dtype=torch.uint8,
                         device=device)
    return codes, scales


def kv_append(x, cache, positions, fmt="nvfp4", tensor_scale=None):
    """Quantize the new rows x [batch, heads, t_new, head_dim] into
    cache = (codes, scales) at positions[b] + i (int32 CUDA tensor [batch]);
    NVFP4 needs tensor_scale (one-element float32 CUDA tensor).  Rows whose
    position is outside the cache are not written.  Returns the cache."""
    f = _fmt(fmt)
    if x.dim() != 4:
        raise ValueError("x must be [batch, heads, t_new, head_dim]")
    codes, scales = cache
    B, H, tn, d = x.shape
    st = lib().fp4_kv_append(f, _ptr(x), _IN_DTYPES[x.dtype], B, H, tn, d, _ptr(positions),
                             _ptr(codes), _ptr(scales), _ptr(tensor_scale), codes.shape[2],
                             _stream(x))
    _check(st, "fp4_kv_append")
    return cache


def attention_decode(q, k_cache, v_cache, seq_lens, fmt="nvfp4", k_tscale=None, v_tscale=None,
                     softmax_scale=None, out_dtype="bf16", out=None, workspace=None):
    """One query token per sequence, q [batch, q_heads, head_dim] (bf16 /
    fp16), over the 4-bit caches k_cache, v_cache = (codes, scales) of shape
    [batch, kv_heads, t_max, ...] dequantized to FP8; seq_lens int32 CUDA
    tensor [batch].  softmax_scale defaults to 1 / sqrt(head_dim).  Returns
    out [batch, q_heads, head_dim]."""
    f = _fmt(fmt)
    if q.dim() != 3:
        raise ValueError("q must be [batch, q_heads, head_dim]")
    B, hq, d = q.shape
    kc, ks = k_cache
    vc, vs = v_cache
    hkv, t_max = kc.shape[1], kc.shape[2]
    if softmax_scale is None:
        softmax_scale = 1.0 / float(d) ** 0.5
    code, tdt = _OUT_DTYPES[out_dtype]
    if out is None:
        out = torch.empty((B, hq, d), dtype=tdt, device=q.device)
    L = lib()
    need = L.fp4_attention_workspace_size(B, hq, hkv, d, t_max)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    st = L.fp4_attention_decode(f, _ptr(q), _IN_DTYPES[q.dtype], B, hq, hkv, d, _ptr(kc), _ptr(ks),
                                _ptr(k_tscale), _ptr(vc), _ptr(vs), _ptr(v_tscale), t_max,
                                _ptr(seq_lens), float(softmax_scale), _ptr(out), code,
                                _ptr(workspace), workspace.numel() * workspace.element_size(),
                                _stream(q))
    _check(st, "fp4_attention_decode")
    return out


def gptq_quantize(w, x, fmt="nvfp4", damp=0.01, rotate=True, workspace=None):
    """MR-GPTQ of the weights w [n, k] with calibration activations x
    [n_calib, k] (CUDA tensors, fp32 / bf16 / fp16).  Returns (codes,
    scales, tensor scale or None) of the (rotated) weights."""
    f = _fmt(fmt)
    if w.dim() != 2 or x.dim() != 2 or w.shape[1] != x.shape[1]:
        raise ValueError("w must be [n, k] and x [n_calib, k]")
    n, k = w.shape
    N = x.shape[0]
    codes = torch.empty((n, k // 2), dtype=torch.uint8, device=w.device)
    scales = torch.empty((n, k // BLOCK[f]), dtype=torch.uint8, device=w.device)
    ts = torch.empty(1, dtype=torch.float32, device=w.device) if f == NVFP4 else None
    L = lib()
    need = L.fp4_gptq_workspace_size(n, k, N)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=w.device)
    st = L.fp4_gptq_quantize(f, _ptr(w), _IN_DTYPES[w.dtype], n, k, _ptr(x), _IN_DTYPES[x.dtype], N,
                             float(damp), 1 if rotate else 0, _ptr(codes), _ptr(scales), _ptr(ts),
                             _ptr(workspace), workspace.numel() * workspace.element_size(),
                             _stream(w))
    _check(st, "fp4_gptq_quantize")
    return codes, scales, ts
