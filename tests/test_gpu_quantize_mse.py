"""GPU parity: fp4_quantize_mse (NVFP4 with the least-squared-error block
scale) against the oracle, codes, scale bytes and tensor scale bit-exact."""

import json
import os

import numpy as np
import pytest
import torch

import oracle
import microscaled_fp4_quantization_amd as fq
from microscaled_fp4_quantization_amd import workloads
from gpu_helpers import DEV, host_f32, note, np_u8, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def check(x, tensor_scale=None, rows=None):
    """MSE-quantize x (CPU tensor) on the GPU; compare all rows, or only
    `rows` (then with the GPU's tensor scale as the given one)."""
    note("quantize_mse %s %s given=%s" % (tuple(x.shape), x.dtype, tensor_scale is not None))
    ts_dev = None if tensor_scale is None else torch.tensor([tensor_scale], dtype=torch.float32, device=DEV)
    codes, scales, ts = fq.quantize_mse(x.to(DEV), tensor_scale=ts_dev)
    torch.cuda.synchronize()
    x32 = host_f32(x)
    if rows is None:
        p, s, t = oracle.nvfp4_quantize_mse(x32, None if tensor_scale is None else np.float32(tensor_scale))
        gc, gs = np_u8(codes), np_u8(scales)
    else:
        t = oracle.nvfp4_tensor_scale(x32) if tensor_scale is None else np.float32(tensor_scale)
        assert ts.item() == float(t)
        p, s, _ = oracle.nvfp4_quantize_mse(x32[rows], t)
        gc, gs = np_u8(codes)[rows], np_u8(scales)[rows]
    assert np.array_equal(gs, s), "scale bytes differ at %s" % (np.argwhere(gs != s)[:5],)
    assert np.array_equal(gc, p), "codes differ at %s" % (np.argwhere(gc != p)[:5],)
    assert ts.item() == float(t)
    return codes, scales, ts


def randn(shape, dtype, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(dtype)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_random_shapes(dtype):
    # one block, a ragged last workgroup, several workgroups
    for seed, (rows, k) in enumerate([(1, 16), (3, 96), (37, 160), (257, 1024)]):
        check(randn((rows, k), dtype, seed, 3.0))


def test_heavy_tails_and_outliers():
    g = torch.Generator().manual_seed(5)
    x = torch.distributions.StudentT(3.0).sample((128, 512)) * 0.02
    x[:, ::37] *= 50.0
    check(x.to(torch.bfloat16))


def test_worked_example(golden_dir):
    with open(os.path.join(golden_dir, "nvfp4_mse_worked.json")) as f:
        g = json.load(f)
    case = g["cases"][0]
    x = torch.tensor([case["x"][0]], dtype=torch.float32)
    codes, scales, _ = check(x, tensor_scale=case["tensor_scale"])
    assert np_u8(scales)[0, 0] == int(case["scales"][0][0], 16)


def test_edge_values():
    k = 128
    x = torch.zeros((5, k), dtype=torch.float32)
    x[0] = torch.linspace(-7, 7, k)
    x[1, :] = -0.0                                        # negative-zero row
    x[2, ::7] = 1e-40                                     # fp32 subnormals
    x[3, ::16] = 1.0                                      # one value per block
    x[4, :16] = torch.tensor([6.0] + [5.0] * 15)
    check(x)
    check(torch.zeros((2, 32), dtype=torch.float32))


def test_given_tensor_scale():
    x = randn((32, 256), torch.bfloat16, 11, 2.0)
    for ts in (0.001, 1.0 / 448, 7.5, 1e-38):
        check(x, tensor_scale=ts)


def test_output_dequantizes_and_multiplies_as_nvfp4():
    x = randn((64, 512), torch.bfloat16, 13)
    w = randn((256, 512), torch.bfloat16, 14, 0.02)
    qx = fq.quantize_mse(x.to(DEV))
    qw = fq.quantize_mse(w.to(DEV))
    c = fq.gemm(qx, qw, "nvfp4", out_dtype="f32")
    torch.cuda.synchronize()
    ref = oracle.gemm_ref("nvfp4", np_u8(qx[0]), np_u8(qx[1]), np.float32(qx[2].item()),
                          np_u8(qw[0]), np_u8(qw[1]), np.float32(qw[2].item()))
    got = c.double().cpu().numpy()
    assert np.linalg.norm(got - ref) <= 1e-3 * np.linalg.norm(ref)
    # and it is closer to the unquantized product than the amax/6 scales
    exact = x.double().numpy() @ w.double().numpy().T
    qx6, qw6 = fq.quantize(x.to(DEV), "nvfp4"), fq.quantize(w.to(DEV), "nvfp4")
    c6 = fq.gemm(qx6, qw6, "nvfp4", out_dtype="f32").double().cpu().numpy()
    assert np.linalg.norm(got - exact) < np.linalg.norm(c6 - exact)


def test_weight_full_size_sampled():
    # the decode/prefill weight shape, W ~ N(0, 0.02); rows sampled for the oracle
    w = workloads.decode()["w"]
    rows = np.array([0, 1, 777, 8191, w.shape[0] - 1])
    check(w, rows=rows)
