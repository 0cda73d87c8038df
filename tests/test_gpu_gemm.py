"""GPU parity: fp4_gemm against the float64 oracle of the same dequantized
operands.  Tolerance: relative Frobenius error <= 1e-3 against the oracle
rounded to the output type (fp32 output: the raw float64 result).  The
MXFP4 integer special case must be bit-exact."""

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


def quant_pair(fmt, x, w, hadamard=False):
    qx = fq.quantize(x.to(DEV), fmt, hadamard=hadamard)
    qw = fq.quantize(w.to(DEV), fmt, hadamard=hadamard)
    return qx, qw


def host_q(q):
    c, s, t = q
    return np_u8(c), np_u8(s), (None if t is None else np.float32(t.item()))


def ref_full(fmt, qx, qw):
    pa, sa, ta = host_q(qx)
    pb, sb, tb = host_q(qw)
    return oracle.gemm_ref(fmt, pa, sa, ta, pb, sb, tb)


def check_full(fmt, qx, qw, out_dtype, tol=TOL):
    note("gemm %s m=%d n=%d k=%d -> %s" % (fmt, qx[0].shape[0], qw[0].shape[0], qx[0].shape[1] * 2, out_dtype))
    c = fq.gemm(qx, qw, fmt, out_dtype=out_dtype)
    torch.cuda.synchronize()
    ref = ref_full(fmt, qx, qw)
    got = c.double().cpu().numpy()
    target = ref if out_dtype == "f32" else bf16_round_f64(ref)
    err = rel_fro(got, target)
    assert err <= tol, err
    return err


def test_mx_integer_special_case_bit_exact():
    # all scale codes 127 (scale 1): 2v are integers in [-12, 12] and every
    # partial sum of 4C is an integer below 2^24, so fp32 accumulation in any
    # order is exact and C must equal int64(2vA) @ int64(2vB)^T / 4 exactly.
    g = torch.Generator().manual_seed(0)
    m = n = 256
    k = 4096
    ca = torch.randint(0, 256, (m, k // 2), generator=g, dtype=torch.uint8)
    cb = torch.randint(0, 256, (n, k // 2), generator=g, dtype=torch.uint8)
    sa = torch.full((m, k // 32), 127, dtype=torch.uint8)
    sb = torch.full((n, k // 32), 127, dtype=torch.uint8)
    note("gemm mx integer special case")
    c = fq.gemm((ca.to(DEV), sa.to(DEV), None), (cb.to(DEV), sb.to(DEV), None), "mxfp4", out_dtype="f32")
    torch.cuda.synchronize()
    ia = (2 * oracle.e2m1_decode(oracle.unpack_nibbles(ca.numpy()))).astype(np.int64)
    ib = (2 * oracle.e2m1_decode(oracle.unpack_nibbles(cb.numpy()))).astype(np.int64)
    exact = (ia @ ib.T).astype(np.float64) / 4
    assert np.array_equal(c.cpu().double().numpy(), exact)


def test_nv_integer_special_case_bit_exact():
    # NVFP4 with scale byte 0x38 (1.0) and tensor scales 1: same integer
    # argument through the fp16 path.
    g = torch.Generator().manual_seed(1)
    m, n, k = 128, 192, 2048
    ca = torch.randint(0, 256, (m, k // 2), generator=g, dtype=torch.uint8)
    cb = torch.randint(0, 256, (n, k // 2), generator=g, dtype=torch.uint8)
    sa = torch.full((m, k // 16), 0x38, dtype=torch.uint8)
    sb = torch.full((n, k // 16), 0x38, dtype=torch.uint8)
    one = torch.ones(1, dtype=torch.float32, device=DEV)
    note("gemm nv integer special case")
    c = fq.gemm((ca.to(DEV), sa.to(DEV), one), (cb.to(DEV), sb.to(DEV), one), "nvfp4", out_dtype="f32")
    torch.cuda.synchronize()
    ia = (2 * oracle.e2m1_decode(oracle.unpack_nibbles(ca.numpy()))).astype(np.int64)
    ib = (2 * oracle.e2m1_decode(oracle.unpack_nibbles(cb.numpy()))).astype(np.int64)
    assert np.array_equal(c.cpu().double().numpy(), (ia @ ib.T).astype(np.float64) / 4)


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_random_shapes(fmt, out_dtype):
    g = torch.Generator().manual_seed(2)
    for m, n, k in [(1, 1, 32), (7, 9, 64), (16, 100, 4128), (3, 1000, 800), (16, 17, 160), (17, 33, 96),
                    (8, 100, 4096), (1, 33, 2048), (5, 64, 6144), (4, 47, 8192), (6, 16000, 4096), (8, 517, 2048),
                    (37, 50, 96), (64, 64, 128), (130, 257, 544), (256, 512, 2048),
                    (300, 600, 1024), (1000, 129, 512), (128, 2048, 256), (513, 700, 2304)]:
        x = torch.randn((m, k), generator=g).to(torch.bfloat16)
        w = (torch.randn((n, k), generator=g) * 0.02).to(torch.bfloat16)
        qx, qw = quant_pair(fmt, x, w)
        check_full(fmt, qx, qw, out_dtype)


@pytest.mark.parametrize("m,n,k,out_dtype", [
    (1100, 16000, 512, "bf16"),    # more tiles than CUs, k = 512 mod 1024
    (2048, 9000, 1024, "f32"),     # tile count a multiple of 8: XCD-ordered tiles
    (520, 30001, 1536, "bf16"),    # n not a multiple of 8
    (500, 3000, 1024, "f32"),      # few tiles: every tile half-width
    (600, 2100, 2560, "bf16"),     # few tiles, half-width, k = 512 mod 1024
])
def test_mxfp4_many_tiles(m, n, k, out_dtype):
    # the MXFP4 large-m kernel over more tiles than CUs (256-wide tiles for
    # the whole rounds, 128-wide ones after them) or so few that every tile
    # is 128 wide, with tiles moved back at the edges and a half scale group
    # at the end of k (k = 512 mod 1024)
    g = torch.Generator().manual_seed(11)
    x = torch.randn((m, k), generator=g).to(torch.bfloat16)
    w = (torch.randn((n, k), generator=g) * 0.02).to(torch.bfloat16)
    qx, qw = quant_pair("mxfp4", x, w)
    check_full("mxfp4", qx, qw, out_dtype)


@pytest.mark.parametrize("m,n,k,out_dtype", [
    (8, 14336, 4096, "bf16"),      # the decode shape
    (16, 16384, 2048, "f32"),      # 16 rows, the largest n
    (1, 333, 4096, "bf16"),        # ragged shares
    (11, 70, 2048, "f32"),
    (8, 4096, 14336, "bf16"),      # a down projection: k split in 7 chunks of 2048
    (16, 20000, 2048, "f32"),      # past 16384 weight rows: whole rounds of workgroups
    (3, 777, 12288, "bf16"),       # 3 chunks of 4096
    (8, 5120, 13824, "f32"),       # 7 chunks, the last three quarters full
    (16, 3000, 5120, "bf16"),      # 3 chunks, the last half empty
    (3, 1000, 3072, "f32"),        # one chunk of 4096, 12 of 16 slices
    (12, 777, 2176, "bf16"),       # 2 chunks, the second with one slice
])
def test_mxfp4_decode_stream(m, n, k, out_dtype):
    # the MXFP4 decode kernel on the block-scaled FP4 matrix instruction
    g = torch.Generator().manual_seed(14)
    x = torch.randn((m, k), generator=g).to(torch.bfloat16)
    x[m - 1] *= 1.0e4                                # a row far from the others
    w = (torch.randn((n, k), generator=g) * 0.02).to(torch.bfloat16)
    qx, qw = quant_pair("mxfp4", x, w)
    check_full("mxfp4", qx, qw, out_dtype)


@pytest.mark.parametrize("fmt,m,n,k,out_dtype", [
    ("nvfp4", 17, 1000, 4096, "bf16"),    # 16 + 1 rows
    ("nvfp4", 40, 14336, 2048, "f32"),
    ("nvfp4", 33, 28672, 4096, "bf16"),   # groups past 16384 weight rows
    ("nvfp4", 95, 333, 4096, "bf16"),     # the last group of 15 rows, ragged shares
    ("nvfp4", 96, 14336, 4096, "bf16"),   # 96..127 rows: the large kernel, one partly filled row of tiles
    ("nvfp4", 127, 3000, 8192, "f32"),    # the same with k split over workgroups
    ("nvfp4", 100, 60000, 512, "bf16"),   # the same with 256-column tiles
    ("nvfp4", 40, 4096, 14336, "bf16"),   # a long k: 16-row groups, k split in 7 chunks
    ("nvfp4", 17, 777, 6144, "f32"),      # the last group of one row (8-row split)
    ("nvfp4", 63, 1000, 8192, "f32"),     # the last group of 15 rows
    ("nvfp4", 64, 4096, 14336, "bf16"),   # four groups
    ("nvfp4", 65, 4096, 14336, "bf16"),   # a long k from 65 rows: the large kernel
    ("nvfp4", 100, 2000, 12288, "f32"),
    ("nvfp4", 40, 5120, 13824, "bf16"),   # a k that is no multiple of 2048: 16-row groups, 7 chunks
    ("nvfp4", 33, 3000, 3072, "f32"),     # one short chunk per group
    ("mxfp4", 17, 777, 4096, "f32"),
    ("mxfp4", 32, 5000, 8192, "bf16"),    # two groups, each with k split in 2 chunks
    ("mxfp4", 24, 3000, 9216, "f32"),     # two groups, 5 chunks of 2048, the last half full
    ("mxfp4", 24, 3000, 5120, "f32"),     # a short last chunk of a k up to 8192: the generic kernel
    ("mxfp4", 33, 14336, 4096, "f32"),    # 33..255 rows: the large kernel, one row of tiles at row 0
    ("mxfp4", 48, 5000, 8192, "bf16"),
    ("mxfp4", 128, 28672, 2048, "bf16"),  # the same, every tile half-width
    ("mxfp4", 255, 3000, 1536, "bf16"),   # the same, k = 512 mod 1024, split k
    ("mxfp4", 100, 300, 512, "f32"),      # the same, n just past one tile
])
def test_small_batch_groups(fmt, m, n, k, out_dtype):
    # a small batch past 16 rows: the decode kernels over groups of 16 rows
    # (NVFP4 96..127 rows: the large kernel)
    g = torch.Generator().manual_seed(15)
    x = torch.randn((m, k), generator=g).to(torch.bfloat16)
    x[m // 2] *= 300.0
    w = (torch.randn((n, k), generator=g) * 0.02).to(torch.bfloat16)
    qx, qw = quant_pair(fmt, x, w)
    check_full(fmt, qx, qw, out_dtype)


@pytest.mark.parametrize("m,n,k,out_dtype", [
    (16, 14336, 4096, "bf16"),     # all 16 columns of the MFMA tile
    (9, 1000, 2048, "f32"),        # one row past 8
    (12, 16384, 2048, "bf16"),     # the largest n of one round
    (16, 20000, 4096, "f32"),      # past it: whole rounds of workgroups
    (16, 333, 4096, "f32"),        # ragged shares
    (4, 3000, 3072, "bf16"),       # one chunk of 4096, 12 of 16 slices
    (11, 20000, 3072, "f32"),      # the same with 11 rows, whole rounds of workgroups
    (3, 1000, 2304, "bf16"),       # 9 of 16 slices
])
def test_nvfp4_decode_16_rows(m, n, k, out_dtype):
    # the NVFP4 decode stream kernel with 9 to 16 activation rows
    g = torch.Generator().manual_seed(13)
    x = torch.randn((m, k), generator=g).to(torch.bfloat16)
    x[m - 1] *= 100.0                                # the last row on its own scale
    w = (torch.randn((n, k), generator=g) * 0.02).to(torch.bfloat16)
    qx, qw = quant_pair("nvfp4", x, w)
    check_full("nvfp4", qx, qw, out_dtype)


@pytest.mark.parametrize("m,n,k,out_dtype", [
    (8, 4096, 14336, "bf16"),      # a down projection: 7 chunks of 2048
    (1, 2000, 8192, "f32"),        # 2 chunks of 4096
    (6, 8192, 6144, "bf16"),       # 3 chunks of 2048, 384 workgroups
    (3, 777, 12288, "f32"),        # 3 chunks of 4096, ragged n
    (16, 4096, 14336, "bf16"),     # 16 rows: 7 chunks of 2048
    (9, 20000, 8192, "f32"),       # 9 rows, whole rounds of workgroups
    (12, 777, 6144, "bf16"),       # ragged n
    (13, 3000, 16384, "f32"),      # 4 chunks of 4096
    (8, 5120, 4608, "bf16"),       # k no multiple of 1024: 3 chunks, the last a quarter full
    (8, 5120, 13824, "f32"),       # 7 chunks over more than one round (k % 1024 != 0)
    (16, 2000, 5120, "bf16"),      # 16 rows, 3 chunks
    (12, 777, 2176, "f32"),        # 2 chunks, the second with one slice of 128 values
])
def test_nvfp4_decode_split_k(m, n, k, out_dtype):
    # the NVFP4 decode kernel with k split over workgroup rows (fp32 partial
    # sums in the workspace, added by the reduction pass)
    assert fq.fp4.lib().fp4_gemm_workspace_size(fq.fp4.NVFP4, m, n, k) > 0
    g = torch.Generator().manual_seed(12)
    x = torch.randn((m, k), generator=g).to(torch.bfloat16)
    w = (torch.randn((n, k), generator=g) * 0.02).to(torch.bfloat16)
    qx, qw = quant_pair("nvfp4", x, w)
    check_full("nvfp4", qx, qw, out_dtype)


@pytest.mark.parametrize("m,n,k,out_dtype", [
    (256, 60000, 512, "bf16"),     # 235 tiles of 256 columns: one round (224 would need two)
    (300, 30000, 1024, "f32"),     # ragged m and n, 236 tiles of 256 columns
])
def test_nvfp4_wide_tiles(m, n, k, out_dtype):
    # the NVFP4 large-m kernel with 256-column tiles (8 B fragments per wave
    # and k-step), chosen where 224-column tiles would need another round
    g = torch.Generator().manual_seed(12)
    x = torch.randn((m, k), generator=g).to(torch.bfloat16)
    w = (torch.randn((n, k), generator=g) * 0.02).to(torch.bfloat16)
    qx, qw = quant_pair("nvfp4", x, w)
    check_full("nvfp4", qx, qw, out_dtype)


@pytest.mark.parametrize("fmt,m,n,k,out_dtype", [
    ("nvfp4", 512, 1024, 4096, "bf16"),   # 10 tiles: k in four slices of 1024
    ("nvfp4", 300, 700, 2048, "f32"),     # ragged, four slices of 512
    ("mxfp4", 512, 512, 4096, "f32"),     # 4 tiles: four slices of 1024
    ("mxfp4", 300, 700, 2048, "bf16"),    # ragged, four slices of 512 (two stages each)
])
def test_split_k(fmt, m, n, k, out_dtype):
    # few output tiles: the large kernels split k over several workgroups per
    # tile, fp32 partial sums in the workspace, added by a second pass
    from microscaled_fp4_quantization_amd import fp4
    assert fp4.lib().fp4_gemm_workspace_size(fp4.NVFP4 if fmt == "nvfp4" else fp4.MXFP4, m, n, k) > 0
    g = torch.Generator().manual_seed(m + n + k)
    x = torch.randn((m, k), generator=g).to(torch.bfloat16)
    w = (torch.randn((n, k), generator=g) * 0.02).to(torch.bfloat16)
    qx, qw = quant_pair(fmt, x, w)
    check_full(fmt, qx, qw, out_dtype)


def test_split_k_sampled_tp8_share():
    # one GPU's share of a column-parallel split of the rotated weight over 8
    # GPUs: 2048 x 3584 x 8192, 128 tiles; NVFP4 splits k in two slices,
    # MXFP4 (a quarter of the time per tile) does not
    from microscaled_fp4_quantization_amd import fp4
    m, n, k = 2048, 3584, 8192
    g = torch.Generator(device=DEV).manual_seed(5)
    x = torch.randn((m, k), generator=g, device=DEV).to(torch.bfloat16)
    w = (torch.randn((n, k), generator=g, device=DEV) * 0.015).to(torch.bfloat16)
    assert fp4.lib().fp4_gemm_workspace_size(fp4.NVFP4, m, n, k) == 2 * m * n * 4
    assert fp4.lib().fp4_gemm_workspace_size(fp4.MXFP4, m, n, k) == 0
    for fmt in ("nvfp4", "mxfp4"):
        qx = fq.quantize(x, fmt, hadamard=True)
        qw = fq.quantize(w, fmt, hadamard=True)
        note("gemm split-k %s m=%d n=%d k=%d" % (fmt, m, n, k))
        c = fq.gemm(qx, qw, fmt, out_dtype="bf16")
        torch.cuda.synchronize()
        got, ref = _sampled(fmt, qx, qw, c)
        assert rel_fro(got, bf16_round_f64(ref)) <= TOL
        assert torch.isfinite(c).all()


def test_tiny_workload():
    d = workloads.tiny()
    qx, qw = quant_pair("nvfp4", d["x"], d["w"])
    check_full("nvfp4", qx, qw, "f32")
    qx, qw = quant_pair("mxfp4", d["x"], d["w"])
    check_full("mxfp4", qx, qw, "f32")


def test_block_scales_vary_per_block():
    # each block of A and B on its own scale, including E4M3 subnormal scales
    g = torch.Generator().manual_seed(3)
    m, n, k = 96, 80, 512
    for fmt, bs in (("nvfp4", 16), ("mxfp4", 32)):
        ca = torch.randint(0, 256, (m, k // 2), generator=g, dtype=torch.uint8)
        cb = torch.randint(0, 256, (n, k // 2), generator=g, dtype=torch.uint8)
        if fmt == "nvfp4":
            sa = torch.randint(1, 127, (m, k // bs), generator=g, dtype=torch.uint8)
            sb = torch.randint(1, 127, (n, k // bs), generator=g, dtype=torch.uint8)
            ta = torch.tensor([0.37], device=DEV)
            tb = torch.tensor([1.9e-3], device=DEV)
        else:
            sa = torch.randint(110, 140, (m, k // bs), generator=g, dtype=torch.uint8)
            sb = torch.randint(110, 140, (n, k // bs), generator=g, dtype=torch.uint8)
            ta = tb = None
        qx = (ca.to(DEV), sa.to(DEV), ta)
        qw = (cb.to(DEV), sb.to(DEV), tb)
        check_full(fmt, qx, qw, "f32")


def _sampled(fmt, qx, qw, c, count=3000, seed=0):
    pa, sa, ta = host_q(qx)
    pb, sb, tb = host_q(qw)
    m, n = c.shape
    rng = np.random.default_rng(seed)
    rows = rng.integers(0, m, count)
    cols = rng.integers(0, n, count)
    # always include the corners and the last tile edges
    rows = np.concatenate([rows, [0, m - 1, 0, m - 1]])
    cols = np.concatenate([cols, [0, n - 1, n - 1, 0]])
    ref = oracle.gemm_ref_entries(fmt, pa, sa, ta, pb, sb, tb, rows, cols)
    got = c[torch.from_numpy(rows).to(DEV), torch.from_numpy(cols).to(DEV)].double().cpu().numpy()
    return got, ref


def full_size_case(fmt, x, w, hadamard, out_dtype="bf16"):
    note("full-size gemm %s m=%d n=%d k=%d" % (fmt, x.shape[0], w.shape[0], x.shape[1]))
    qx = fq.quantize(x, fmt, hadamard=hadamard)
    qw = fq.quantize(w, fmt, hadamard=hadamard)
    c = fq.gemm(qx, qw, fmt, out_dtype=out_dtype)
    torch.cuda.synchronize()
    got, ref = _sampled(fmt, qx, qw, c)
    target = ref if out_dtype == "f32" else bf16_round_f64(ref)
    assert rel_fro(got, target) <= TOL
    assert torch.isfinite(c).all()


def test_decode_full_size():
    d = workloads.decode(device=DEV)
    full_size_case("nvfp4", d["x"], d["w"], False)
    full_size_case("mxfp4", d["x"], d["w"], False)


def test_prefill_full_size():
    d = workloads.prefill(device=DEV)
    full_size_case("nvfp4", d["x"], d["w"], False)


def test_rotated_full_size():
    d = workloads.rotated(device=DEV)
    full_size_case("nvfp4", d["x"], d["w"], True)
    full_size_case("mxfp4", d["x"], d["w"], True)


@pytest.mark.parametrize("fmt,m,n,k,xdt", [
    ("nvfp4", 8, 14336, 4096, torch.bfloat16),   # decode shape: one launch
    ("nvfp4", 1, 100, 4096, torch.bfloat16),     # partial share of rows
    ("nvfp4", 5, 333, 2048, torch.bfloat16),
    ("nvfp4", 8, 16384, 4096, torch.bfloat16),   # largest n of the one-launch path
    ("nvfp4", 7, 1025, 2048, torch.bfloat16),    # 3 rows per share, last share partial
    ("nvfp4", 16, 64, 256, torch.bfloat16),      # m > 8: quantize + GEMM calls
    ("nvfp4", 8, 4096, 14336, torch.bfloat16),   # long k: quantize + split-k GEMM
    ("nvfp4", 12, 4096, 14336, torch.bfloat16),  # the same with 16 activation rows per workgroup
    ("nvfp4", 40, 1000, 8192, torch.bfloat16),   # quantize + 16-row groups of the split-k GEMM
    ("nvfp4", 16, 2000, 4096, torch.bfloat16),   # 16 rows in one launch
    ("nvfp4", 9, 16384, 4096, torch.bfloat16),   # 9 rows in one launch, the largest n
    ("nvfp4", 12, 1000, 2048, torch.bfloat16),
    ("nvfp4", 3, 50, 96, torch.bfloat16),
    ("nvfp4", 8, 200, 4096, torch.float32),      # not bf16: two calls
    ("mxfp4", 8, 100, 4096, torch.bfloat16),
    ("mxfp4", 16, 2000, 2048, torch.bfloat16),   # one launch, 16 rows
    ("mxfp4", 3, 16384, 4096, torch.bfloat16),
    ("mxfp4", 5, 64, 1024, torch.bfloat16),      # k outside the one-launch path: two calls
    ("mxfp4", 8, 4096, 14336, torch.bfloat16),   # one launch over 7 chunks of k + the reduction
    ("mxfp4", 8, 5120, 13824, torch.bfloat16),   # the last chunk three quarters full (its codes too)
    ("mxfp4", 12, 1000, 3072, torch.bfloat16),   # one chunk, 12 of 16 slices
])
def test_quantize_gemm(fmt, m, n, k, xdt):
    g = torch.Generator().manual_seed(4)
    x = torch.randn((m, k), generator=g).to(xdt)
    x[0, :16] = 0.0                                  # a zero block
    w = (torch.randn((n, k), generator=g) * 0.02).to(torch.bfloat16)
    qw = fq.quantize(w.to(DEV), fmt)
    note("quantize_gemm %s m=%d n=%d k=%d %s" % (fmt, m, n, k, xdt))
    qx, c = fq.quantize_gemm(x.to(DEV), qw, fmt, out_dtype="f32")
    torch.cuda.synchronize()
    xf = x.float().numpy()
    if fmt == "nvfp4":
        px, sx, tx = oracle.nvfp4_quantize(xf)
        assert np.float32(qx[2].item()).tobytes() == np.float32(tx).tobytes()
    else:
        (px, sx), tx = oracle.mxfp4_quantize(xf), None
    assert np.array_equal(np_u8(qx[0]), px)
    assert np.array_equal(np_u8(qx[1]), sx)
    pw, sw, tw = host_q(qw)
    ref = oracle.gemm_ref(fmt, px, sx, tx, pw, sw, tw)
    assert rel_fro(c.double().cpu().numpy(), ref) <= TOL
