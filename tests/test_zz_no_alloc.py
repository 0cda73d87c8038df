"""GPU check of fp4_quantize_noalloc (the entry point that allocates
nothing: its compute-mode scratch is the library's own device array) through
the C ABI: codes, scale bytes and tensor scale bit-identical to fp4_quantize
with a caller workspace, over consecutive calls that reuse the scratch (the
second smaller than the first), and when the max pass runs more than one
trip per workgroup."""

import ctypes

import numpy as np
import pytest
import torch

import microscaled_fp4_quantization_amd as fq
from microscaled_fp4_quantization_amd import fp4
from gpu_helpers import DEV, note, require_gpu

pytestmark = pytest.mark.gpu

_DT = {torch.float32: fp4.F32, torch.bfloat16: fp4.BF16, torch.float16: fp4.F16}


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def noalloc(x, fmt, mode, ts=None):
    rows, k = x.shape
    bs = 16 if fmt == fp4.NVFP4 else 32
    codes = torch.empty((rows, k // 2), dtype=torch.uint8, device=DEV)
    scales = torch.empty((rows, k // bs), dtype=torch.uint8, device=DEV)
    if fmt == fp4.NVFP4 and ts is None:
        ts = torch.empty(1, dtype=torch.float32, device=DEV)
    st = fq.lib().fp4_quantize_noalloc(fmt, _p(x), _DT[x.dtype], rows, k, _p(codes), _p(scales), _p(ts),
                                       mode, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == fp4.OK, fq.lib().fp4_status_string(st)
    return codes, scales, ts


def reference(x, fmt, mode, ts=None):
    rows, k = x.shape
    bs = 16 if fmt == fp4.NVFP4 else 32
    codes = torch.empty((rows, k // 2), dtype=torch.uint8, device=DEV)
    scales = torch.empty((rows, k // bs), dtype=torch.uint8, device=DEV)
    if fmt == fp4.NVFP4 and ts is None:
        ts = torch.empty(1, dtype=torch.float32, device=DEV)
    L = fq.lib()
    need = L.fp4_quantize_workspace_size(fmt, mode, rows, k)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=DEV)
    st = L.fp4_quantize(fmt, _p(x), _DT[x.dtype], rows, k, _p(codes), _p(scales), _p(ts), mode,
                        _p(ws) if need else None, need, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == fp4.OK
    return codes, scales, ts


def same(a, b):
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    if a[2] is not None:
        assert a[2].item() == b[2].item()


def test_noalloc_matches_quantize():
    g = torch.Generator(device="cpu").manual_seed(40)
    cases = [  # (shape, dtype, format, mode): consecutive calls share the scratch
        ((2048, 8192), torch.bfloat16, fp4.NVFP4, fp4.TSCALE_COMPUTE),   # 1024 max-pass workgroups
        ((300, 2048), torch.float32, fp4.NVFP4, fp4.TSCALE_COMPUTE),     # smaller, right after
        ((8192, 4160), torch.bfloat16, fp4.NVFP4, fp4.TSCALE_COMPUTE),   # several trips per workgroup
        ((7, 256), torch.float16, fp4.NVFP4, fp4.TSCALE_COMPUTE),        # one-workgroup kernel
        ((513, 1024), torch.bfloat16, fp4.MXFP4, fp4.TSCALE_COMPUTE),
        ((640, 512), torch.bfloat16, fp4.NVFP4, fp4.TSCALE_COMPUTE),
    ]
    for (rows, k), dtype, fmt, mode in cases:
        x = (torch.randn((rows, k), generator=g) * 3.0).to(dtype).to(DEV)
        note("fp4_quantize_noalloc %s %s fmt=%d" % ((rows, k), dtype, fmt))
        same(noalloc(x, fmt, mode), reference(x, fmt, mode))
    # given tensor scale: no scratch involved
    x = torch.randn((256, 1024), generator=g).to(torch.bfloat16).to(DEV)
    ts = torch.tensor([0.002], dtype=torch.float32, device=DEV)
    same(noalloc(x, fp4.NVFP4, fp4.TSCALE_GIVEN, ts), reference(x, fp4.NVFP4, fp4.TSCALE_GIVEN, ts))


def test_noalloc_under_graph_capture():
    # The caller it is for: fp4_quantize_noalloc captured into a HIP graph
    # (compute mode, so the kernels use the library's scratch), replayed
    # with new data in the captured input, fp4_quantize with a workspace run
    # eagerly between the replays: every replay bit-identical to it.
    g = torch.Generator(device="cpu").manual_seed(41)
    x_static = torch.randn((1024, 4096), generator=g).to(torch.bfloat16).to(DEV)
    noalloc(x_static, fp4.NVFP4, fp4.TSCALE_COMPUTE)   # scratch located before capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    note("fp4_quantize_noalloc captured into a graph")
    with torch.cuda.graph(graph):
        out = noalloc(x_static, fp4.NVFP4, fp4.TSCALE_COMPUTE)
    for i, scale in enumerate((1.0, 500.0, 0.002)):
        x_static.copy_((torch.randn((1024, 4096), generator=g) * scale).to(torch.bfloat16).to(DEV))
        note("graph replay %d" % i)
        graph.replay()
        same(out, reference(x_static, fp4.NVFP4, fp4.TSCALE_COMPUTE))
