"""GPU parity: fp4_quantize / fp4_hadamard_quantize codes, scale bytes and
tensor scale bit-exact against the CPU oracle."""

import numpy as np
import pytest
import torch

import oracle
import microscaled_fp4_quantization_amd as fq
from microscaled_fp4_quantization_amd import workloads
from gpu_helpers import DEV, host_f32, note, np_u8, require_gpu

pytestmark = pytest.mark.gpu


def oracle_quant(fmt, x32, hadamard=False, tensor_scale=None):
    if hadamard:
        x32 = oracle.hadamard_blocks(x32, 16 if fmt == "nvfp4" else 32)
    if fmt == "nvfp4":
        return oracle.nvfp4_quantize(x32, tensor_scale)
    p, s = oracle.mxfp4_quantize(x32)
    return p, s, None


def check(fmt, x, hadamard=False, tensor_scale=None):
    """Quantize x (a CPU tensor) on the GPU and with the oracle; compare."""
    note("quantize %s %s %s had=%s given=%s" % (fmt, tuple(x.shape), x.dtype, hadamard,
                                                 tensor_scale is not None))
    ts_dev = None if tensor_scale is None else torch.tensor([tensor_scale], dtype=torch.float32, device=DEV)
    codes, scales, ts = fq.quantize(x.to(DEV), fmt, tensor_scale=ts_dev, hadamard=hadamard)
    torch.cuda.synchronize()
    p, s, t = oracle_quant(fmt, host_f32(x), hadamard,
                           None if tensor_scale is None else np.float32(tensor_scale))
    gc, gs = np_u8(codes), np_u8(scales)
    bad = np.nonzero(gc != p)
    assert np.array_equal(gs, s), "scale bytes differ at %s" % (np.argwhere(gs != s)[:5],)
    assert np.array_equal(gc, p), "codes differ at %s: gpu %s oracle %s" % (
        np.stack(bad, 1)[:5], gc[bad][:5], p[bad][:5])
    if fmt == "nvfp4":
        assert ts.item() == float(t)
    return codes, scales, ts


def randn(shape, dtype, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(dtype)


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
@pytest.mark.parametrize("hadamard", [False, True])
def test_random_shapes(fmt, dtype, hadamard):
    # several workgroups, a ragged last trip, and tiny tensors
    for seed, (rows, k) in enumerate([(1, 32), (3, 96), (37, 160), (1000, 4096), (2049, 1056)]):
        check(fmt, randn((rows, k), dtype, seed, 3.0), hadamard)


def test_tiny_workload():
    d = workloads.tiny()
    for name in ("x", "w"):
        check("nvfp4", d[name])
        check("mxfp4", d[name])


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_edge_values(fmt):
    k = 256
    x = torch.zeros((6, k), dtype=torch.float32)
    x[0] = torch.linspace(-7, 7, k)                       # crosses every E2M1 tie
    x[1, :64] = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] * 8)
    x[1, 64:] = -x[1, :64].repeat(3)
    x[2] = -0.0                                           # negative-zero row
    x[3, ::7] = 1e-40                                     # fp32 subnormals
    x[3, 1::7] = -3e-39
    x[4, :] = 3.0e38                                      # near the fp32 max
    x[4, 1::2] = -1.0e-30                                 # tiny next to huge
    x[5, ::32] = 1.0                                      # sparse blocks
    check(fmt, x)
    check(fmt, x[2:4].contiguous())                       # all-zero / subnormal tensor
    check(fmt, torch.zeros((2, 64), dtype=torch.float32))


def test_given_tensor_scale():
    x = randn((64, 512), torch.bfloat16, 11, 2.0)
    for ts in (0.001, 1.0 / 448, 1e-6, 7.5, 1e-38):   # fits, too small (saturates), subnormal products
        check("nvfp4", x, tensor_scale=ts)
        check("nvfp4", x, hadamard=True, tensor_scale=ts)


def test_rows_zero_is_noop():
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    c, s, t = fq.quantize(x, "nvfp4")
    assert c.shape == (0, 32) and s.shape == (0, 4)


def test_deterministic():
    x = randn((512, 2048), torch.bfloat16, 3).to(DEV)
    a = fq.quantize(x, "nvfp4")
    b = fq.quantize(x, "nvfp4")
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])


# --- full workload sizes --------------------------------------------------

def test_decode_full_size():
    d = workloads.decode(device=DEV)
    check("nvfp4", d["x"].cpu())
    check("nvfp4", d["w"].cpu())


def test_prefill_activation_full_size():
    d = workloads.prefill(device=DEV, n=16)
    check("nvfp4", d["x"].cpu())
    check("mxfp4", d["x"].cpu())


def test_rotated_activation_full_size():
    d = workloads.rotated(device=DEV, n=16)
    check("nvfp4", d["x"].cpu(), hadamard=True)
    check("mxfp4", d["x"].cpu(), hadamard=True)


def _bits16(t):
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_rotated_weight_full_size(fmt):
    # W [28672, 8192] bf16 rotated offline (Hadamard 16 / 32) and quantized:
    # every row of the codes and scales against the oracle (rows checked in
    # parallel host processes).  NVFP4's tensor scale comes from the whole
    # rotated tensor: the oracle's exact amax over all rows decides it.
    from oracle_pool import OracleRun
    b = 16 if fmt == "nvfp4" else 32
    d = workloads.rotated(device=DEV, m=16)
    w = d["w"]
    note("rotated W %s, whole tensor" % fmt)
    codes, scales, ts = fq.hadamard_quantize(w, fmt)
    torch.cuda.synchronize()
    with OracleRun(_bits16(w), "bf16", np_u8(codes), np_u8(scales)) as run:
        t = None
        if fmt == "nvfp4":
            t = oracle.nvfp4_tensor_scale_from_amax(np.float32(run.amax(b)))
            assert ts.item() == float(t)
        assert run.check(fmt, t, b) is None


# --- compute mode: a workspace reused across calls ----------------------------

def test_compute_workspace_reused_across_calls():
    # One workspace (uninitialized) for a run of calls of different sizes,
    # dtypes and rotations, including tensors that need more than one pass
    # of the max kernel per workgroup: every result bit-exact.
    need = fq.lib().fp4_quantize_workspace_size(fq.fp4.NVFP4, fq.fp4.TSCALE_COMPUTE, 1, 16)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device=DEV)
    cases = [((2048, 8192), torch.bfloat16, True, 21), ((300, 2048), torch.float32, False, 22),
             ((4096, 4096), torch.bfloat16, False, 23), ((77, 1024), torch.float16, True, 24),
             ((8192, 4160), torch.bfloat16, True, 26), ((2048, 8192), torch.bfloat16, True, 25)]
    for (rows, k), dtype, had, seed in cases:
        x = randn((rows, k), dtype, seed, 2.0)
        note("compute-mode quantize with a shared workspace %s %s had=%s" % ((rows, k), dtype, had))
        codes, scales, ts = fq.quantize(x.to(DEV), "nvfp4", hadamard=had, workspace=ws)
        torch.cuda.synchronize()
        p, s, t = oracle_quant("nvfp4", host_f32(x), had)
        assert ts.item() == float(t)
        assert np.array_equal(np_u8(scales), s) and np.array_equal(np_u8(codes), p)


# --- compute mode: calls queued back to back, and graph capture ---------------

def test_compute_back_to_back():
    # Calls queued on one stream with no wait between them, one workspace
    # (uninitialized), inputs whose tensor scales differ by 10^4: a launch
    # must never take an earlier launch's maxima for its own.
    need = fq.lib().fp4_quantize_workspace_size(fq.fp4.NVFP4, fq.fp4.TSCALE_COMPUTE, 1, 16)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    xs = [randn((2048, 8192), torch.bfloat16, 70 + i, sc) for i, sc in enumerate((1.0, 100.0, 0.01, 1.0))]
    xd = [x.to(DEV) for x in xs]
    torch.cuda.synchronize()
    note("four compute-mode calls back to back")
    outs = [fq.quantize(x, "nvfp4", hadamard=True, workspace=ws) for x in xd]
    torch.cuda.synchronize()
    for x, (codes, scales, ts) in zip(xs, outs):
        p, s, t = oracle_quant("nvfp4", host_f32(x), True)
        assert ts.item() == float(t)
        assert np.array_equal(np_u8(scales), s) and np.array_equal(np_u8(codes), p)


def test_compute_under_graph_capture():
    # Captured into a HIP graph, replayed with new data in the captured
    # input, with eager calls on the same workspace between the replays:
    # every replay and every eager call bit-exact.
    need = fq.lib().fp4_quantize_workspace_size(fq.fp4.NVFP4, fq.fp4.TSCALE_COMPUTE, 1, 16)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    x_static = randn((1024, 4096), torch.bfloat16, 80).to(DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fq.quantize(x_static, "nvfp4", hadamard=True, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    note("compute-mode quantize captured into a graph")
    with torch.cuda.graph(g):
        codes, scales, ts = fq.quantize(x_static, "nvfp4", hadamard=True, workspace=ws)
    for i, sc in enumerate((1.0, 1000.0, 0.001)):
        x = randn((1024, 4096), torch.bfloat16, 81 + i, sc)
        x_static.copy_(x.to(DEV))
        note("graph replay %d" % i)
        g.replay()
        torch.cuda.synchronize()
        p, s, t = oracle_quant("nvfp4", host_f32(x), True)
        assert ts.item() == float(t)
        assert np.array_equal(np_u8(scales), s) and np.array_equal(np_u8(codes), p)
        e_codes, e_scales, e_ts = fq.quantize(x_static, "nvfp4", hadamard=True, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(e_codes, codes) and torch.equal(e_scales, scales) and torch.equal(e_ts, ts)
