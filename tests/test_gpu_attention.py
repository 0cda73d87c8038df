"""GPU parity: fp4_kv_append (bit-exact against the oracle) and
fp4_attention_decode (against the float64 attention of the FP8-dequantized
cache; hyper.ai story on the NVFP4 KV cache).

Tolerance of the attention output, from the kernel's arithmetic: the softmax
weights, 2^(x - max) <= 1, are rounded to fp16 before the weighted sum of V:
relative error at most 2^-11, and for weights below 2^-14 (fp16 subnormals)
an absolute error of at most 2^-25 against the largest weight.  Everything
else runs in fp32 (FP8 K times 16-bit q is exact, sums and exp2 err near
2^-20 relative).  So per element, with both terms doubled,
|out - ref| <= 2^-10 sum_t p_t |V_t| + 2^-24 max_t p_t sum_t |V_t|;
bf16 output adds its own rounding, 2^-8 |ref|.  The caches the attention reads are written by
the oracle's quantizer (or are random bytes), never by the library.
"""

import numpy as np
import pytest
import torch

import oracle
import microscaled_fp4_quantization_amd as fq
from microscaled_fp4_quantization_amd import workloads
from gpu_helpers import DEV, host_f32, note, np_u8, require_gpu

pytestmark = pytest.mark.gpu

FP16_WEIGHT_BOUND = 2.0 ** -10
FP16_SUBNORMAL_BOUND = 2.0 ** -24
BF16_OUT = 2.0 ** -8


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def oracle_cache(fmt, x, ts):
    """x [B, H, T, D] float32 numpy -> oracle-quantized (codes, scales)."""
    B, H, T, D = x.shape
    rows = x.reshape(-1, D)
    if fmt == "nvfp4":
        c, s, _ = oracle.nvfp4_quantize(rows, tensor_scale=ts)
    else:
        c, s = oracle.mxfp4_quantize(rows)
    return c.reshape(B, H, T, D // 2), s.reshape(B, H, T, -1)


def dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def dev_scalar(v):
    return None if v is None else torch.tensor([v], dtype=torch.float32, device=DEV)


def check_attention(fmt, q, kc, ks, kts, vc, vs, vts, lens, scale, out_dtype="f32",
                    workspace_fill=None):
    note("attention %s q%s %s cache%s lens=%s -> %s" % (fmt, tuple(q.shape), q.dtype,
                                                      tuple(kc.shape), list(lens)[:6], out_dtype))
    lens_d = torch.tensor(lens, dtype=torch.int32, device=DEV)
    ws = None
    if workspace_fill is not None:
        need = fq.lib().fp4_attention_workspace_size(q.shape[0], q.shape[1], kc.shape[1], 128,
                                                      kc.shape[2])
        ws = torch.full((need,), workspace_fill, dtype=torch.uint8, device=DEV)
    out = fq.attention_decode(q.to(DEV), (dev_u8(kc), dev_u8(ks)), (dev_u8(vc), dev_u8(vs)),
                              lens_d, fmt, dev_scalar(kts), dev_scalar(vts), scale,
                              out_dtype=out_dtype, workspace=ws)
    torch.cuda.synchronize()
    ref, absw, flat = oracle.attention_decode_ref(fmt, host_f32(q), kc, ks, kts, vc, vs, vts,
                                                  lens, scale, with_abs=True)
    got = out.double().cpu().numpy()
    bound = FP16_WEIGHT_BOUND * absw + FP16_SUBNORMAL_BOUND * flat
    if out_dtype == "bf16":
        bound = bound + BF16_OUT * np.abs(ref)
    err = np.abs(got - ref)
    worst = float(np.max(err / np.maximum(bound, 1e-300)))
    assert np.all(err <= bound), "worst err / bound = %g" % worst
    return out, ref


def cache_inputs(fmt, B, Hkv, G, T, seed, qdtype=torch.bfloat16, q_mul=1.0):
    d = workloads.attention(seed=seed, batch=B, kv_heads=Hkv, q_heads=Hkv * G, tokens=T)
    k = host_f32(d["k"])
    v = host_f32(d["v"])
    kts = vts = None
    if fmt == "nvfp4":
        kts = float(oracle.nvfp4_tensor_scale(k))
        vts = float(oracle.nvfp4_tensor_scale(v))
    kc, ks = oracle_cache(fmt, k, kts)
    vc, vs = oracle_cache(fmt, v, vts)
    q = (d["q"].float() * q_mul).to(qdtype)
    return q, kc, ks, kts, vc, vs, vts


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
@pytest.mark.parametrize("B,Hkv,G,T,lens", [
    (3, 2, 8, 300, [300, 1, 0]),          # full, one token, empty
    (2, 3, 5, 700, [513, 699]),           # odd group, ragged steps
    (1, 1, 16, 96, [96]),                 # the widest group
    (2, 2, 1, 1000, [1000, 33]),          # one query head per KV head
    (2, 1, 8, 4100, [4100, 4097]),        # more than one split, ragged last split
])
def test_attention_matches_oracle(fmt, B, Hkv, G, T, lens):
    q, kc, ks, kts, vc, vs, vts = cache_inputs(fmt, B, Hkv, G, T, seed=3)
    check_attention(fmt, q, kc, ks, kts, vc, vs, vts, lens, 1.0 / np.sqrt(128.0))


@pytest.mark.parametrize("qdtype,out_dtype", [(torch.float16, "f32"), (torch.bfloat16, "bf16"),
                                              (torch.float16, "bf16")])
def test_attention_dtypes(qdtype, out_dtype):
    q, kc, ks, kts, vc, vs, vts = cache_inputs("nvfp4", 2, 2, 8, 333, seed=4, qdtype=qdtype)
    check_attention("nvfp4", q, kc, ks, kts, vc, vs, vts, [333, 200], 0.0883883, out_dtype)


def test_attention_peaked_softmax_and_clamped_lengths():
    # q x 8: scores spread over tens of units, a few tokens carry the weight;
    # lengths beyond the cache clamp to it, negative ones to 0
    q, kc, ks, kts, vc, vs, vts = cache_inputs("nvfp4", 3, 2, 8, 257, seed=5, q_mul=8.0)
    check_attention("nvfp4", q, kc, ks, kts, vc, vs, vts, [257 + 40, -3, 100], 0.0883883)


def test_attention_ignores_workspace_contents():
    q, kc, ks, kts, vc, vs, vts = cache_inputs("mxfp4", 2, 2, 4, 600, seed=6)
    a, _ = check_attention("mxfp4", q, kc, ks, kts, vc, vs, vts, [600, 17], 0.1,
                           workspace_fill=0xFF)
    b, _ = check_attention("mxfp4", q, kc, ks, kts, vc, vs, vts, [600, 17], 0.1,
                           workspace_fill=0x00)
    assert torch.equal(a, b)


def test_attention_masked_tokens_with_garbage_bytes():
    # tokens past each sequence's length hold random bytes (NaN-free in the
    # table, but large): they must contribute nothing
    q, kc, ks, kts, vc, vs, vts = cache_inputs("nvfp4", 2, 2, 8, 160, seed=7)
    rng = np.random.default_rng(8)
    for arr in (kc, vc):
        arr[:, :, 70:] = rng.integers(0, 256, size=arr[:, :, 70:].shape, dtype=np.uint8)
    for arr in (ks, vs):
        arr[:, :, 70:] = 0x7E                 # 448
    check_attention("nvfp4", q, kc, ks, kts, vc, vs, vts, [70, 45], 0.0883883)


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_attention_full_kv_shape_sampled(fmt):
    # the KV workload's shape, batch 32 x 8 KV heads x 32768 tokens x 128, 64
    # query heads, in the launch configuration the benchmark times; random
    # cache bytes; sampled (sequence, query head) pairs against the oracle
    B, H, T, D, G = 32, 8, 32768, 128, 8
    kc, ks = workloads.random_cache(B, H, T, D, fmt, seed=11)
    vc, vs = workloads.random_cache(B, H, T, D, fmt, seed=12)
    kts = vts = None
    if fmt == "nvfp4":
        kts, vts = 0.0625, 0.046875
    g = torch.Generator().manual_seed(13)
    q = torch.randn((B, H * G, D), generator=g).to(torch.bfloat16)
    lens = [T] * B
    lens[3], lens[17], lens[30] = 12345, 1, 0
    note("attention full shape %s" % fmt)
    lens_d = torch.tensor(lens, dtype=torch.int32, device=DEV)
    out = fq.attention_decode(q.to(DEV), (dev_u8(kc), dev_u8(ks)), (dev_u8(vc), dev_u8(vs)),
                              lens_d, fmt, dev_scalar(kts), dev_scalar(vts), 1.0 / np.sqrt(128.0),
                              out_dtype="f32")
    torch.cuda.synchronize()
    got = out.double().cpu().numpy()
    qh = host_f32(q)
    for b, j in [(0, 0), (3, 17), (17, 40), (31, 63), (30, 5), (12, 9)]:
        h = j // G
        ref, absw, flat = oracle.attention_decode_ref(
            fmt, qh[b:b + 1, h * G:(h + 1) * G], kc[b:b + 1, h:h + 1], ks[b:b + 1, h:h + 1], kts,
            vc[b:b + 1, h:h + 1], vs[b:b + 1, h:h + 1], vts, [lens[b]], 1.0 / np.sqrt(128.0),
            with_abs=True)
        jj = j - h * G
        err = np.abs(got[b, j] - ref[0, jj])
        bound = FP16_WEIGHT_BOUND * absw[0, jj] + FP16_SUBNORMAL_BOUND * flat[0, jj]
        assert np.all(err <= bound), (b, j, float(err.max()))


@pytest.mark.parametrize("fmt,dt,D", [("nvfp4", torch.bfloat16, 128), ("nvfp4", torch.float32, 64),
                                      ("mxfp4", torch.float16, 128), ("mxfp4", torch.bfloat16, 96)])
@pytest.mark.parametrize("tn", [1, 7])
def test_kv_append_bit_exact(fmt, dt, D, tn):
    B, H, T = 3, 2, 40
    g = torch.Generator().manual_seed(21)
    x = (torch.randn((B, H, tn, D), generator=g) * 2.5).to(dt)
    rng = np.random.default_rng(22)
    codes0 = rng.integers(0, 256, size=(B, H, T, D // 2), dtype=np.uint8)
    bs = 16 if fmt == "nvfp4" else 32
    scales0 = rng.integers(0, 256, size=(B, H, T, D // bs), dtype=np.uint8)
    positions = [0, T - 3, -2]                 # start, running past the end, starting before 0
    ts = 0.0123 if fmt == "nvfp4" else None
    note("kv_append %s %s D=%d t_new=%d" % (fmt, dt, D, tn))
    cache = (dev_u8(codes0), dev_u8(scales0))
    fq.kv_append(x.to(DEV), cache, torch.tensor(positions, dtype=torch.int32, device=DEV), fmt,
                 dev_scalar(ts))
    torch.cuda.synchronize()
    want_c, want_s = oracle.kv_append_ref(fmt, codes0, scales0, host_f32(x), positions, ts)
    np.testing.assert_array_equal(np_u8(cache[0]), want_c)
    np.testing.assert_array_equal(np_u8(cache[1]), want_s)


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_decode_step_append_then_attend(fmt):
    # one decode step: the new token's K and V are appended at position
    # seq_lens[b], then the query attends over seq_lens[b] + 1 tokens
    B, Hkv, G, T = 2, 2, 8, 200
    q, kc, ks, kts, vc, vs, vts = cache_inputs(fmt, B, Hkv, G, T, seed=31)
    lens = [150, 199]
    g = torch.Generator().manual_seed(32)
    k_new = torch.randn((B, Hkv, 1, 128), generator=g).to(torch.bfloat16)
    v_new = torch.randn((B, Hkv, 1, 128), generator=g).to(torch.bfloat16)
    note("decode step %s" % fmt)
    kcache = (dev_u8(kc), dev_u8(ks))
    vcache = (dev_u8(vc), dev_u8(vs))
    pos = torch.tensor(lens, dtype=torch.int32, device=DEV)
    fq.kv_append(k_new.to(DEV), kcache, pos, fmt, dev_scalar(kts))
    fq.kv_append(v_new.to(DEV), vcache, pos, fmt, dev_scalar(vts))
    lens1 = [n + 1 for n in lens]
    out = fq.attention_decode(q.to(DEV), kcache, vcache,
                              torch.tensor(lens1, dtype=torch.int32, device=DEV), fmt,
                              dev_scalar(kts), dev_scalar(vts), 0.0883883, out_dtype="f32")
    torch.cuda.synchronize()
    kc1, ks1 = oracle.kv_append_ref(fmt, kc, ks, host_f32(k_new), lens, kts)
    vc1, vs1 = oracle.kv_append_ref(fmt, vc, vs, host_f32(v_new), lens, vts)
    np.testing.assert_array_equal(np_u8(kcache[0]), kc1)
    np.testing.assert_array_equal(np_u8(vcache[1]), vs1)
    ref, absw, flat = oracle.attention_decode_ref(fmt, host_f32(q), kc1, ks1, kts, vc1, vs1, vts,
                                                  lens1, 0.0883883, with_abs=True)
    err = np.abs(out.double().cpu().numpy() - ref)
    assert np.all(err <= FP16_WEIGHT_BOUND * absw + FP16_SUBNORMAL_BOUND * flat)
