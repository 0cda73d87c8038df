"""GPU parity for block-scale bytes the quantizers never write: NVFP4 E4M3
bytes with the sign bit set and the NaN bytes 0x7F / 0xFF, MXFP4's NaN byte
0xFF.  Every kernel that reads caller-supplied scales is run on them
(fp4_dequantize, each fp4_gemm path, each fp4_gemm_w4a16 path) and compared
with the oracle, which decodes the bytes by the formats' definitions: NaN
exactly where the oracle has NaN, every other value to the usual bar
(bit-exact for dequantize, relative Frobenius <= 1e-3 for the products)."""

import numpy as np
import pytest
import torch

import oracle
import microscaled_fp4_quantization_amd as fq
from gpu_helpers import DEV, bf16_round_f64, note, rel_fro, require_gpu

pytestmark = pytest.mark.gpu

TOL = 1e-3


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def special_scales(fmt, rows, nblk, rng, nan_rows=()):
    """Scale bytes: NVFP4 magnitudes 0.5 .. 1.9 with random signs; MXFP4
    exponents -3 .. 3.  Rows in nan_rows get one NaN byte (NVFP4 0x7F or
    0xFF, MXFP4 0xFF) in a random block."""
    if fmt == "nvfp4":
        s = rng.integers(0x30, 0x3F, size=(rows, nblk)) | (rng.integers(0, 2, size=(rows, nblk)) << 7)
    else:
        s = rng.integers(124, 131, size=(rows, nblk))
    s = s.astype(np.uint8)
    for i, r in enumerate(nan_rows):
        s[r, rng.integers(0, nblk)] = (0x7F if i % 2 == 0 else 0xFF) if fmt == "nvfp4" else 0xFF
    return s


def operand(fmt, rows, k, rng, nan_rows=()):
    bs = 16 if fmt == "nvfp4" else 32
    codes = rng.integers(0, 256, size=(rows, k // 2)).astype(np.uint8)
    return codes, special_scales(fmt, rows, k // bs, rng, nan_rows)


def compare(got, ref, out_dtype):
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan), "NaN positions differ"
    assert nan.any() and not nan.all()
    target = ref if out_dtype == "f32" else bf16_round_f64(np.where(nan, 0.0, ref))
    err = rel_fro(np.where(nan, 0.0, got), np.where(nan, 0.0, target))
    assert err <= TOL, err


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


# (m, n, k) per fp4_gemm path: NVFP4 m <= 8 with k 2048 / 4096 (streaming
# kernel), m <= 8 with k a multiple of 1024 (LDS-staged decode kernel),
# m <= 16 (skinny), the large tiled kernel, the generic kernel.
NV_SHAPES = [(5, 64, 2048), (5, 64, 3072), (12, 48, 160), (160, 192, 512), (40, 72, 96)]
MX_SHAPES = [(7, 64, 256), (256, 256, 512), (40, 72, 96)]


@pytest.mark.parametrize("fmt,shape", [("nvfp4", s) for s in NV_SHAPES] + [("mxfp4", s) for s in MX_SHAPES])
def test_gemm_special_scale_bytes(fmt, shape):
    m, n, k = shape
    rng = np.random.default_rng(m * 1000 + n + k)
    ca, sa = operand(fmt, m, k, rng, nan_rows=(m // 2,))
    cb, sb = operand(fmt, n, k, rng, nan_rows=(1, n - 2))
    ta = tb = None
    if fmt == "nvfp4":
        ta, tb = np.float32(0.5), np.float32(0.25)
    ref = oracle.gemm_ref(fmt, ca, sa, ta, cb, sb, tb)
    for out_dtype in ("f32", "bf16"):
        note("gemm special scale bytes %s m=%d n=%d k=%d -> %s" % (fmt, m, n, k, out_dtype))
        qa = (dev(ca), dev(sa), None if ta is None else torch.tensor([float(ta)], device=DEV))
        qb = (dev(cb), dev(sb), None if tb is None else torch.tensor([float(tb)], device=DEV))
        c = fq.gemm(qa, qb, fmt, out_dtype=out_dtype)
        torch.cuda.synchronize()
        compare(c.double().cpu().numpy(), ref, out_dtype)


# fp4_gemm_w4a16: NVFP4 with bf16 or fp16 X and MXFP4 with bf16 X, k 2048
# (the streaming kernels); fp32 X and k 256 (the generic kernel).
@pytest.mark.parametrize("fmt,x_dtype,k", [("nvfp4", torch.bfloat16, 2048), ("nvfp4", torch.float32, 256),
                                           ("mxfp4", torch.bfloat16, 256), ("mxfp4", torch.bfloat16, 2048),
                                           ("nvfp4", torch.float16, 2048)])
def test_w4a16_special_scale_bytes(fmt, x_dtype, k):
    m, n = 6, 80
    rng = np.random.default_rng(k + n)
    cb, sb = operand(fmt, n, k, rng, nan_rows=(3, n - 1))
    tb = np.float32(0.75) if fmt == "nvfp4" else None
    x = torch.from_numpy(rng.standard_normal((m, k)).astype(np.float32)).to(x_dtype)
    ref = oracle.gemm_w4a16_ref(fmt, x.float().numpy(), cb, sb, tb)
    note("w4a16 special scale bytes %s %s k=%d" % (fmt, x_dtype, k))
    c = fq.gemm_w4a16(x.to(DEV), (dev(cb), dev(sb), None if tb is None else torch.tensor([float(tb)], device=DEV)),
                      fmt, out_dtype="f32")
    torch.cuda.synchronize()
    got = c.double().cpu().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and nan.any()
    assert rel_fro(np.where(nan, 0.0, got), np.where(nan, 0.0, ref)) <= TOL


_BITS = {"f32": (torch.int32, np.uint32), "bf16": (torch.int16, np.uint16), "f16": (torch.int16, np.uint16)}
_FLOAT = {"f32": np.float32, "f16": np.float16}


def _as_float(bits, out_dtype):
    if out_dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32)
    return bits.view(_FLOAT[out_dtype])


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16", "f16"])
def test_dequantize_special_scale_bytes(fmt, out_dtype):
    # NaN scale bytes give NaN values (any NaN); everything else bit-exact.
    rng = np.random.default_rng(7)
    rows, k = 33, 256
    codes, scales = operand(fmt, rows, k, rng, nan_rows=(0, 5, 32))
    ts = np.float32(0.375) if fmt == "nvfp4" else None
    exp = oracle.dequantize(fmt, codes, scales, ts, out_dtype)
    exp_bits = exp.view(np.uint32) if out_dtype == "f32" else exp
    note("dequantize special scale bytes %s -> %s" % (fmt, out_dtype))
    y = fq.dequantize(dev(codes), dev(scales), None if ts is None else torch.tensor([float(ts)], device=DEV),
                      fmt, out_dtype)
    torch.cuda.synchronize()
    tview, nview = _BITS[out_dtype]
    got_bits = y.view(tview).cpu().numpy().view(nview)
    nan_e, nan_g = np.isnan(_as_float(exp_bits, out_dtype)), np.isnan(_as_float(got_bits, out_dtype))
    assert nan_e.any() and np.array_equal(nan_g, nan_e)
    assert np.array_equal(got_bits[~nan_e], exp_bits[~nan_e])
