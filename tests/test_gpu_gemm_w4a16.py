"""GPU parity: fp4_gemm_w4a16 (16-bit activations x 4-bit weights) against the
float64 oracle.  Tolerance: relative Frobenius error <= 1e-3 against the
oracle rounded to the output type (fp32 output: the raw float64 result)."""

import numpy as np
import pytest
import torch

import oracle
import microscaled_fp4_quantization_amd as fq
from microscaled_fp4_quantization_amd import workloads
from gpu_helpers import DEV, bf16_round_f64, host_f32, note, np_u8, rel_fro, require_gpu

pytestmark = pytest.mark.gpu

TOL = 1e-3


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def check(fmt, x, w, out_dtype="bf16", wq=None):
    note("w4a16 %s x%s %s w%s -> %s" % (fmt, tuple(x.shape), x.dtype, tuple(w.shape), out_dtype))
    if wq is None:
        wq = fq.quantize(w.to(DEV), fmt)
    c = fq.gemm_w4a16(x.to(DEV), wq, fmt, out_dtype=out_dtype)
    torch.cuda.synchronize()
    pb, sb = np_u8(wq[0]), np_u8(wq[1])
    tb = None if wq[2] is None else np.float32(wq[2].item())
    ref = oracle.gemm_w4a16_ref(fmt, host_f32(x), pb, sb, tb)
    got = c.double().cpu().numpy()
    target = ref if out_dtype == "f32" else bf16_round_f64(ref)
    err = rel_fro(got, target)
    assert err <= TOL, err
    return c, wq


def randn(shape, dtype, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(dtype)


def test_decode_shape():
    # the decode workload: X bf16 [8, 4096], W [14336, 4096] ~ N(0, 0.02); the streaming path
    d = workloads.decode()
    check("nvfp4", d["x"], d["w"])
    check("nvfp4", d["x"], d["w"], out_dtype="f32")


@pytest.mark.parametrize("m,n,k", [
    (1, 100, 4096),          # one row, a partial share of weight rows
    (5, 333, 2048),          # k = 2048
    (16, 4096, 4096),        # 16 rows in one launch
    (13, 16384, 4096),       # 13 rows, one round of 64-row workgroups
    (3, 20000, 4096),        # beyond it: workgroups of up to 64 rows in whole rounds
    (8, 28672, 2048),        # the same with k = 2048 (two workgroups per CU)
    (8, 4096, 14336),        # a down projection: k split in 7 chunks of 2048
    (16, 4096, 14336),       # the same for 16 rows (one workgroup per CU)
    (20, 1000, 8192),        # 2 chunks of 4096; launches of 16 and 4 rows reuse the workspace
    (6, 17000, 6144),        # 3 chunks of 2048 over more than one round
    (16, 20000, 2048),       # 16 rows past 16384 weight rows (one workgroup per CU)
    (11, 3000, 12288),       # 11 rows, 3 chunks of 4096
    (4, 200, 96),            # k outside the streaming path
    (4, 200, 5120),          # 3 chunks of 2048, the last half empty
    (8, 5120, 13824),        # 7 chunks, the last three quarters full
    (12, 2000, 3072),        # one chunk of 4096, 12 of 16 slices
    (40, 1000, 5120),        # three launches of up to 16 rows
    (4, 200, 4160),          # k not a multiple of 128: the fallback kernel
])
def test_shapes(m, n, k):
    if k > 4096 and k % 2048 == 0:
        assert fq.fp4.lib().fp4_gemm_w4a16_workspace_size(fq.fp4.NVFP4, m, n, k) > 0
    x = randn((m, k), torch.bfloat16, m + n)
    w = randn((n, k), torch.bfloat16, k, 0.02)
    check("nvfp4", x, w, "f32" if m % 2 else "bf16")


@pytest.mark.parametrize("m,n,k", [
    (8, 14336, 4096),        # the decode shape with MXFP4 weights
    (16, 333, 2048),         # 16 rows, ragged shares
    (20, 1000, 4096),        # launches of 16 and 4 rows
    (8, 4096, 14336),        # k split in 7 chunks of 2048
    (20, 17000, 8192),       # 2 chunks of 4096 past 16384 weight rows, two launches
    (8, 5120, 13824),        # 7 chunks, the last three quarters full
    (12, 2000, 3072),        # one chunk of 4096, 12 of 16 slices
])
def test_mxfp4_stream(m, n, k):
    # W4A16 with MXFP4 weights on the decode stream kernel (bf16 products of
    # the exactly widened weights); scale bytes at both ends of E8M0 in some
    # blocks: 0 (2^-127), 1, 2 and 200 (2^73)
    x = randn((m, k), torch.bfloat16, m + n + 1)
    w = randn((n, k), torch.bfloat16, k + 1, 0.02)
    codes, scales, _ = fq.quantize(w.to(DEV), "mxfp4")
    sc = scales.cpu()
    for i, byte in enumerate((0, 1, 2, 200)):
        sc[(7 * i + 3) % n, (5 * i) % (k // 32)] = byte
    wq = (codes, sc.to(DEV), None)
    check("mxfp4", x, w, "f32" if m % 2 else "bf16", wq=wq)


@pytest.mark.parametrize("m,n,k", [
    (8, 14336, 4096),        # the decode shape with fp16 activations
    (16, 333, 2048),         # 16 rows in one launch
    (5, 4096, 14336),        # k split in 7 chunks of 2048
    (16, 2000, 2304),        # one chunk of 4096, 9 of 16 slices
])
def test_fp16_activations_stream(m, n, k):
    # NVFP4 weights and fp16 X on the decode stream kernel: X widened
    # exactly from fp16, one row near fp16's largest value, one row tiny
    x = randn((m, k), torch.float32, m + n + 2)
    x[0] *= 5.0e3                            # up to ~2.5e4, below fp16's 65504
    x[m - 1] *= 1.0e-5
    x = x.to(torch.float16)
    w = randn((n, k), torch.bfloat16, k + 2, 0.02)
    check("nvfp4", x, w, "f32" if m % 2 else "bf16")


def test_mxfp4_and_other_activation_types():
    w = randn((300, 1024), torch.bfloat16, 1, 0.02)
    for dt in (torch.bfloat16, torch.float16, torch.float32):
        x = randn((6, 1024), dt, 2)
        check("mxfp4", x, w, "f32")
        check("nvfp4", x, w, "f32")


def test_activation_range():
    # large and tiny activations in one tensor: the power-of-two prescale
    x = randn((8, 4096), torch.float32, 3)
    x[0] *= 3.0e4
    x[1] *= 1.0e-6
    x[2, ::5] = 0.0
    x = x.to(torch.bfloat16)
    w = randn((2048, 4096), torch.bfloat16, 4, 0.02)
    check("nvfp4", x, w, "f32")
    check("nvfp4", torch.zeros((8, 4096), dtype=torch.bfloat16), w, "f32")
    big = randn((2, 2048), torch.float32, 5) * 1.0e30      # far beyond fp16 range
    check("nvfp4", big.to(torch.bfloat16), randn((512, 2048), torch.bfloat16, 6, 0.02), "f32")
    # 16 rows in one launch: each row of the second group of 8 on its own scale
    x16 = randn((16, 4096), torch.float32, 9)
    for i in range(8, 16):
        x16[i] *= 10.0 ** (i - 11)
    x16[13, ::3] = 0.0
    x16[15] = 0.0
    check("nvfp4", x16.to(torch.bfloat16), w, "f32")
    check("nvfp4", x16[:11].to(torch.bfloat16), w, "f32")


def test_agrees_with_w4a4_on_nvfp4_activations():
    # activations that are exactly an NVFP4 tensor's values (tensor scale 1):
    # W4A16 on them and W4A4 on their codes compute the same product
    x0 = randn((8, 4096), torch.float32, 7)
    one = torch.ones(1, dtype=torch.float32, device=DEV)
    qx = fq.quantize(x0.to(DEV), "nvfp4", tensor_scale=one)
    x = fq.dequantize(*qx, fmt="nvfp4", out_dtype="bf16")
    w = randn((1024, 4096), torch.bfloat16, 8, 0.02)
    wq = fq.quantize(w.to(DEV), "nvfp4")
    c16 = fq.gemm_w4a16(x, wq, "nvfp4", out_dtype="f32")
    c4 = fq.gemm(qx, wq, "nvfp4", out_dtype="f32")
    torch.cuda.synchronize()
    a, b = c16.double().cpu().numpy(), c4.double().cpu().numpy()
    assert rel_fro(a, b) <= 1e-5
