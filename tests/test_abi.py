"""C-ABI checks that need no GPU: the library loads, exports every entry
point include/fp4.h declares, and rejects bad arguments on the host before
any HIP call (every case below fails validation, so nothing is launched)."""

import ctypes
import os
import re

import pytest

from microscaled_fp4_quantization_amd import fp4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

NV, MX = fp4.NVFP4, fp4.MXFP4
FAKE = ctypes.c_void_p(0x10000)        # aligned, never dereferenced
FAKE_ODD = ctypes.c_void_p(0x10001)    # misaligned


def header_functions():
    src = open(os.path.join(ROOT, "include", "fp4.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fp4_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    L = fp4.lib()
    names = header_functions()
    assert set(names) == set(fp4.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    L = fp4.lib()
    for s in range(4):
        assert L.fp4_status_string(s).decode().startswith("FP4_")
    assert L.fp4_status_string(99) == b"unknown fp4_status"


def test_workspace_sizes():
    L = fp4.lib()
    assert L.fp4_quantize_workspace_size(NV, fp4.TSCALE_COMPUTE, 4096, 4096) == 4096
    assert L.fp4_quantize_workspace_size(NV, fp4.TSCALE_GIVEN, 4096, 4096) == 0
    assert L.fp4_quantize_workspace_size(MX, fp4.TSCALE_COMPUTE, 4096, 4096) == 0
    assert L.fp4_gemm_workspace_size(NV, 16, 16, 256) >= 0
    # NVFP4 decode shapes with k > 4096 split k into chunks of 4096 (k a
    # multiple of 4096) or 2048, each chunk's fp32 sums m n (rounded up to a
    # multiple of 4) floats, when one round of workgroups covers the chunks
    assert L.fp4_gemm_workspace_size(NV, 8, 4096, 14336) == 7 * 8 * 4096 * 4
    assert L.fp4_gemm_workspace_size(NV, 3, 777, 12288) == 3 * 2332 * 4
    assert L.fp4_gemm_workspace_size(NV, 8, 8192, 6144) == 3 * 8 * 8192 * 4   # 384 of 512 slots
    assert L.fp4_gemm_workspace_size(NV, 8, 14336, 4096) == 0      # one chunk: no split
    assert L.fp4_gemm_workspace_size(NV, 8, 14336, 8192) == 0      # 448 workgroups for 256 slots
    assert L.fp4_gemm_workspace_size(NV, 8, 16384, 6144) == 0      # 768 for 512
    # 9..16 rows: 16 activation rows per workgroup, any n (whole rounds)
    assert L.fp4_gemm_workspace_size(NV, 9, 4096, 14336) == 7 * 9 * 4096 * 4
    assert L.fp4_gemm_workspace_size(NV, 16, 14336, 8192) == 2 * 16 * 14336 * 4
    assert L.fp4_gemm_workspace_size(NV, 32, 4096, 14336) == 7 * 16 * 4096 * 4   # groups of 16 rows
    assert L.fp4_gemm_workspace_size(NV, 16, 4096, 4096) == 0      # one chunk: no split
    # k not a multiple of 2048: chunks of 2048 (4096 when k is a multiple of
    # 4096), the last one short; a k that is no multiple of 1024 in any round count
    assert L.fp4_gemm_workspace_size(NV, 8, 5120, 5120) == 0       # the older kernel takes k = 5120
    assert L.fp4_gemm_workspace_size(NV, 8, 5120, 4608) == 3 * 8 * 5120 * 4   # it does not take 4608
    assert L.fp4_gemm_workspace_size(NV, 8, 5120, 13824) == 7 * 8 * 5120 * 4
    assert L.fp4_gemm_workspace_size(NV, 8, 13824, 5120) == 0      # 648 workgroups: the older kernel
    assert L.fp4_gemm_workspace_size(NV, 16, 2000, 5120) == 3 * 16 * 2000 * 4
    assert L.fp4_gemm_workspace_size(NV, 4, 3000, 3072) == 0       # one chunk
    assert L.fp4_gemm_workspace_size(NV, 8, 64, 4160) == 0         # k % 128 != 0: not the stream kernel
    assert L.fp4_gemm_workspace_size(NV, 8, 4096, 5120) == 0       # a short last chunk: the older kernel
    assert L.fp4_gemm_workspace_size(MX, 8, 4096, 14336) == 7 * 8 * 4096 * 4   # MXFP4: m <= 16, any n
    assert L.fp4_gemm_workspace_size(MX, 16, 16384, 6144) == 3 * 16 * 16384 * 4
    assert L.fp4_gemm_workspace_size(MX, 32, 4096, 14336) == 7 * 16 * 4096 * 4   # groups of 16 rows
    assert L.fp4_gemm_workspace_size(MX, 33, 4096, 14336) == 0   # the large kernel, one row of tiles
    assert L.fp4_gemm_workspace_size(MX, 8, 4096, 5120) == 3 * 8 * 4096 * 4     # a short last chunk
    assert L.fp4_gemm_workspace_size(MX, 24, 4096, 13824) == 7 * 16 * 4096 * 4  # groups of 16 rows
    assert L.fp4_gemm_workspace_size(MX, 24, 4096, 5120) == 0    # the generic kernel
    assert L.fp4_gemm_workspace_size(MX, 8, 4096, 3072) == 0     # one chunk


def _q(fn, fmt=NV, x=FAKE, dt=fp4.BF16, rows=4, k=64, codes=FAKE, scales=FAKE,
       ts=FAKE, mode=fp4.TSCALE_GIVEN, ws=None, wsb=0):
    return fn(fmt, x, dt, rows, k, codes, scales, ts, mode, ws, wsb, None)


@pytest.mark.parametrize("name", ["fp4_quantize", "fp4_hadamard_quantize"])
def test_quantize_rejects_bad_arguments(name):
    f = getattr(fp4.lib(), name)
    E = fp4.EINVAL
    assert _q(f, fmt=7) == E
    assert _q(f, dt=fp4.E4M3) == E                       # not an input dtype
    assert _q(f, k=40) == E                              # k % 16
    assert _q(f, fmt=MX, ts=None, k=48) == E             # k % 32
    assert _q(f, k=0) == E
    assert _q(f, rows=-1) == E
    assert _q(f, rows=1 << 30, k=1 << 20) == E           # over 2^40 elements
    assert _q(f, x=None) == E
    assert _q(f, codes=None) == E
    assert _q(f, scales=None) == E
    assert _q(f, ts=None) == E                           # NVFP4 needs the tensor scale
    assert _q(f, fmt=MX) == E                            # MXFP4 takes none
    assert _q(f, x=FAKE_ODD) == E
    assert _q(f, codes=FAKE_ODD) == E
    assert _q(f, mode=5) == E
    # COMPUTE mode without enough workspace
    assert _q(f, mode=fp4.TSCALE_COMPUTE) == E
    assert _q(f, mode=fp4.TSCALE_COMPUTE, ws=FAKE, wsb=16) == E
    # zero rows is a valid no-op (nothing launched)
    assert _q(f, rows=0, x=None, codes=None, scales=None) == fp4.OK


def test_quantize_noalloc_rejects_bad_arguments():
    # as fp4_quantize, without the workspace arguments: every check runs on
    # the host before any HIP call (compute mode included)
    f = fp4.lib().fp4_quantize_noalloc

    def q(fmt=NV, x=FAKE, dt=fp4.BF16, rows=4, k=64, codes=FAKE, scales=FAKE, ts=FAKE,
          mode=fp4.TSCALE_COMPUTE):
        return f(fmt, x, dt, rows, k, codes, scales, ts, mode, None)

    E = fp4.EINVAL
    assert q(fmt=7) == E
    assert q(dt=fp4.E4M3) == E
    assert q(k=40) == E
    assert q(rows=-1) == E
    assert q(rows=1 << 30, k=1 << 20) == E
    assert q(x=None) == E
    assert q(codes=FAKE_ODD) == E
    assert q(ts=None) == E
    assert q(fmt=MX) == E                                # MXFP4 takes no tensor scale
    assert q(mode=5) == E
    assert q(rows=0, x=None, codes=None, scales=None) == fp4.OK


def test_quantize_mse_rejects_bad_arguments():
    f = fp4.lib().fp4_quantize_mse

    def q(x=FAKE, dt=fp4.BF16, rows=4, k=64, codes=FAKE, scales=FAKE, ts=FAKE,
          mode=fp4.TSCALE_GIVEN, ws=None, wsb=0):
        return f(x, dt, rows, k, codes, scales, ts, mode, ws, wsb, None)

    E = fp4.EINVAL
    assert q(dt=fp4.E4M3) == E
    assert q(k=40) == E                                  # k % 16
    assert q(k=0) == E
    assert q(rows=-1) == E
    assert q(x=None) == E
    assert q(codes=None) == E
    assert q(ts=None) == E
    assert q(x=FAKE_ODD) == E
    assert q(mode=5) == E
    assert q(mode=fp4.TSCALE_COMPUTE) == E               # no workspace
    assert q(rows=0, x=None, codes=None, scales=None) == fp4.OK


def test_gemm_w4a16_rejects_bad_arguments():
    f = fp4.lib().fp4_gemm_w4a16

    def g(fmt=NV, x=FAKE, dt=fp4.BF16, m=8, n=64, k=256, bc=FAKE, bs=FAKE, bt=FAKE, c=FAKE,
          cdt=fp4.BF16, ws=None, wsb=0):
        return f(fmt, x, dt, m, n, k, bc, bs, bt, c, cdt, ws, wsb, None)

    E = fp4.EINVAL
    assert g(fmt=9) == E
    assert g(dt=fp4.E4M3) == E
    assert g(cdt=fp4.F16) == fp4.EUNSUPPORTED
    assert g(cdt=7) == E
    assert g(k=40) == E                                  # k % 16
    assert g(fmt=MX, bt=None, k=48) == E                 # k % 32
    assert g(m=-1) == E
    assert g(x=None) == E
    assert g(bc=None) == E
    assert g(bt=None) == E                               # NVFP4 needs the weights' tensor scale
    assert g(fmt=MX) == E                                # MXFP4 takes none
    assert g(x=FAKE_ODD) == E
    assert g(m=0, x=None, c=None) == fp4.OK
    # NVFP4 with more than one chunk of k: chunk sums of up to 16 rows
    ws = fp4.lib().fp4_gemm_w4a16_workspace_size
    assert ws(NV, 8, 64, 8192) == 2 * 8 * 64 * 4
    assert ws(NV, 20, 64, 14336) == 7 * 16 * 64 * 4
    assert ws(NV, 12, 5, 14336) == 7 * 60 * 4
    assert ws(NV, 3, 5, 6144) == 3 * 16 * 4
    assert ws(NV, 8, 64, 4096) == 0 and ws(NV, 8, 64, 3072) == 0
    assert ws(NV, 8, 64, 5120) == 3 * 8 * 64 * 4                  # the last chunk half empty
    assert ws(NV, 8, 64, 4160) == 0                               # k % 128 != 0: the fallback kernel
    assert ws(MX, 8, 64, 8192) == 2 * 8 * 64 * 4 and ws(MX, 20, 64, 14336) == 7 * 16 * 64 * 4
    assert ws(MX, 8, 64, 5120) == 3 * 8 * 64 * 4 and ws(MX, 8, 64, 4160) == 0
    assert g(k=8192) == E                                # workspace missing
    assert g(k=8192, ws=FAKE, wsb=2 * 8 * 64 * 4 - 1) == E
    assert g(k=8192, ws=FAKE_ODD, wsb=2 * 8 * 64 * 4) == E


def test_dequantize_rejects_bad_arguments():
    f = fp4.lib().fp4_dequantize
    E = fp4.EINVAL

    def d(fmt=NV, codes=FAKE, scales=FAKE, ts=FAKE, rows=4, k=64, out=FAKE, dt=fp4.E4M3):
        return f(fmt, codes, scales, ts, rows, k, out, dt, None)

    assert d(fmt=3) == E
    assert d(dt=9) == E
    assert d(k=24) == E
    assert d(codes=None) == E
    assert d(out=None) == E
    assert d(ts=None) == E
    assert d(fmt=MX) == E
    assert d(out=FAKE_ODD) == E
    assert d(rows=0, codes=None, out=None) == fp4.OK


def test_gemm_rejects_bad_arguments():
    f = fp4.lib().fp4_gemm

    def g(fmt=NV, m=8, n=8, k=64, a=FAKE, asc=FAKE, at=FAKE, b=FAKE, bsc=FAKE, bt=FAKE,
          c=FAKE, dt=fp4.BF16, ws=None, wsb=0):
        return f(fmt, m, n, k, a, asc, at, b, bsc, bt, c, dt, ws, wsb, None)

    E = fp4.EINVAL
    assert g(fmt=2) == E
    assert g(k=48) == E                       # k % 32
    assert g(m=-1) == E
    assert g(a=None) == E
    assert g(bsc=None) == E
    assert g(c=FAKE_ODD) == E
    assert g(at=None) == E
    assert g(fmt=MX) == E                     # MXFP4 takes no tensor scales
    assert g(dt=fp4.F16) == fp4.EUNSUPPORTED
    assert g(dt=fp4.E4M3) == fp4.EUNSUPPORTED
    assert g(dt=11) == E
    assert g(m=0, a=None, c=None) == fp4.OK
    # a split k needs its workspace (decode shapes with k > 4096)
    need = fp4.lib().fp4_gemm_workspace_size(MX, 8, 64, 8192)
    assert need == 2 * 8 * 64 * 4
    assert g(fmt=MX, at=None, bt=None, n=64, k=8192) == E
    assert g(fmt=MX, at=None, bt=None, n=64, k=8192, ws=FAKE, wsb=need - 1) == E
    assert g(fmt=MX, at=None, bt=None, n=64, k=8192, ws=FAKE_ODD, wsb=need) == E
    assert g(n=64, k=8192) == E                                            # NVFP4 likewise
    assert g(n=64, k=8192, ws=FAKE, wsb=fp4.lib().fp4_gemm_workspace_size(NV, 8, 64, 8192) - 1) == E
    # 9..16 NVFP4 rows with a long k, and the 16-row groups of a small batch
    for m in (12, 40):
        need = fp4.lib().fp4_gemm_workspace_size(NV, m, 64, 14336)
        assert need == 7 * min(m, 16) * 64 * 4
        assert g(m=m, n=64, k=14336) == E
        assert g(m=m, n=64, k=14336, ws=FAKE, wsb=need - 1) == E
        assert g(m=m, n=64, k=14336, ws=FAKE_ODD, wsb=need) == E


def test_quantize_gemm_rejects_bad_arguments():
    f = fp4.lib().fp4_quantize_gemm

    def g(fmt=NV, x=FAKE, dt=fp4.BF16, m=8, n=8, k=64, ac=FAKE, asc=FAKE, at=FAKE, b=FAKE,
          bsc=FAKE, bt=FAKE, c=FAKE, cdt=fp4.BF16, ws=FAKE, wsb=1 << 20):
        return f(fmt, x, dt, m, n, k, ac, asc, at, b, bsc, bt, c, cdt, ws, wsb, None)

    E = fp4.EINVAL
    assert g(fmt=2) == E
    assert g(k=48) == E                       # quantizes (k % 16) but the GEMM needs k % 32
    assert g(k=40) == E
    assert g(x=FAKE_ODD) == E
    assert g(dt=fp4.E4M3) == E                # not an input dtype
    assert g(at=None) == E                    # NVFP4 writes the tensor scale
    assert g(ws=None, wsb=0) == E             # the computed tensor scale needs the workspace
    assert g(b=None) == E
    assert g(bt=None) == E
    assert g(c=FAKE_ODD) == E
    assert g(n=-1) == E
    assert g(fmt=MX, at=None) == E            # MXFP4 takes no tensor scale for B either
    assert g(cdt=fp4.F16) == fp4.EUNSUPPORTED
    assert g(m=0, x=None, ac=None) == fp4.OK   # nothing to do, nothing enqueued
    assert fp4.lib().fp4_quantize_gemm_workspace_size(NV, 8, 8, 64) >= \
        fp4.lib().fp4_quantize_workspace_size(NV, fp4.TSCALE_COMPUTE, 8, 64)


def test_kv_append_rejects_bad_arguments():
    f = fp4.lib().fp4_kv_append

    def g(fmt=NV, x=FAKE, dt=fp4.BF16, b=2, h=8, tn=1, k=128, pos=FAKE, codes=FAKE, scales=FAKE,
          ts=FAKE, t_max=64):
        return f(fmt, x, dt, b, h, tn, k, pos, codes, scales, ts, t_max, None)

    E = fp4.EINVAL
    assert g(fmt=2) == E
    assert g(k=24) == E                       # not whole NVFP4 blocks
    assert g(fmt=MX, ts=None, k=48) == E      # not whole MXFP4 blocks
    assert g(dt=fp4.E4M3) == E
    assert g(x=FAKE_ODD) == E
    assert g(codes=FAKE_ODD) == E
    assert g(pos=None) == E
    assert g(ts=None) == E                    # NVFP4 uses the cache's given tensor scale
    assert g(fmt=MX) == E                     # MXFP4 has none
    assert g(t_max=0) == E
    assert g(tn=-1) == E
    assert g(tn=0, x=None, pos=None) == fp4.OK
    assert g(b=1 << 14, h=64, tn=1 << 10, t_max=1 << 10) == fp4.EUNSUPPORTED   # 2^34 values
    assert g(b=0, x=None) == fp4.OK


def test_attention_decode_rejects_bad_arguments():
    L = fp4.lib()
    f = L.fp4_attention_decode
    need = L.fp4_attention_workspace_size(2, 16, 2, 128, 1000)
    assert need > 0

    def g(fmt=NV, q=FAKE, qdt=fp4.BF16, b=2, hq=16, hkv=2, d=128, kc=FAKE, ks=FAKE, kt=FAKE,
          vc=FAKE, vs=FAKE, vt=FAKE, t_max=1000, lens=FAKE, scale=0.088, out=FAKE,
          odt=fp4.BF16, ws=FAKE, wsb=None):
        return f(fmt, q, qdt, b, hq, hkv, d, kc, ks, kt, vc, vs, vt, t_max, lens, scale, out, odt,
                 ws, need if wsb is None else wsb, None)

    E, U = fp4.EINVAL, fp4.EUNSUPPORTED
    assert g(fmt=2) == E
    assert g(hq=15) == E                      # q heads not a multiple of kv heads
    assert g(d=64) == U                       # head_dim 128 only
    assert g(hq=34) == U                      # more than 16 query heads per kv head
    assert g(t_max=(1 << 26) + 1) == U        # token offsets are 32-bit inside a sequence
    assert g(qdt=fp4.F32) == U
    assert g(qdt=fp4.E4M3) == E
    assert g(odt=fp4.F16) == U
    assert g(q=FAKE_ODD) == E
    assert g(kc=FAKE_ODD) == E
    assert g(vs=None) == E
    assert g(lens=None) == E
    assert g(kt=None) == E                    # NVFP4 caches carry tensor scales
    assert g(fmt=MX) == E                     # MXFP4 caches do not
    assert g(ws=None) == E
    assert g(wsb=need - 1) == E
    assert g(t_max=0) == E
    assert g(b=0, q=None, out=None) == fp4.OK
    assert L.fp4_attention_workspace_size(2, 16, 2, 64, 1000) == 0


def test_gptq_rejects_bad_arguments():
    L = fp4.lib()
    f = L.fp4_gptq_quantize
    need = L.fp4_gptq_workspace_size(64, 256, 128)
    assert need > 64 * 256 * 8

    def g(fmt=NV, w=FAKE, wdt=fp4.BF16, n=64, k=256, x=FAKE, xdt=fp4.BF16, N=128, damp=0.01,
          rot=1, codes=FAKE, scales=FAKE, ts=FAKE, ws=FAKE, wsb=None):
        return f(fmt, w, wdt, n, k, x, xdt, N, damp, rot, codes, scales, ts, ws,
                 need if wsb is None else wsb, None)

    E = fp4.EINVAL
    assert g(fmt=2) == E
    assert g(k=192) == E                      # k % 128
    assert g(n=0) == E
    assert g(N=0) == E
    assert g(damp=-1.0) == E
    assert g(damp=float("nan")) == E
    assert g(wdt=fp4.E4M3) == E
    assert g(w=FAKE_ODD) == E
    assert g(x=None) == E
    assert g(ts=None) == E                    # NVFP4 writes its tensor scale
    assert g(fmt=MX) == E                     # MXFP4 has none
    assert g(ws=None) == E
    assert g(wsb=need - 1) == E
    assert g(k=16384 + 128) == fp4.EUNSUPPORTED
    assert L.fp4_gptq_workspace_size(64, 100, 128) == 0


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(fp4, "_lib", None)
    monkeypatch.setattr(fp4, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        fp4.lib()
