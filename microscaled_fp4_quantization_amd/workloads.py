"""Seeded synthetic inputs for the five workloads (no quantization arithmetic).

The pages measure on LLM layers, DeepSeek-R1, Llama 3.3 70B and benchmark
suites that are not available here; these seeded tensors stand in for them
with the shapes and value distributions below.  Every draw is float32 from a
torch generator seeded with `seed` (default 0), in a fixed order, then
rounded to bfloat16 (round to nearest even) where the workload is bf16.

  tiny     X fp32 [16,256] ~ N(0,1); W fp32 [256,256] ~ N(0, 0.02^2) with
           round(0.001*65536) = 66 distinct entries multiplied by 20.
  decode   X bf16 [8,4096] ~ N(0,1); W bf16 [14336,4096] ~ N(0, 0.02^2).
  prefill  X bf16 [4096,4096] standard Student-t (3 degrees of freedom) with
           round(0.01*4096) = 41 distinct k-channels multiplied by 50;
           W as in decode.
  rotated  X bf16 [2048,8192] ~ N(0,1); W bf16 [28672,8192] ~ N(0, 0.015^2).
  kv       K and V bf16 [32, 8, 32768, 128], each N(0,1) * c[h, d] with one
           multiplier c ~ U(0.5, 4) per (head, head_dim channel), shared by
           batch and tokens; drawn c_K, K, c_V, V.

  attention  the kv workload's K and V (the cache contents) and the query of
           one decode step, Q bf16 [32, 64, 128] ~ N(0,1) (64 query heads over
           8 KV heads: grouped-query attention with 8 query heads per KV
           head), drawn after K and V.
  calibration  GPTQ calibration activations X bf16 [n_calib, k]: per-channel
           scales c ~ U(0.5, 4) times N(0,1) plus a shared rank-32 part
           (N(0,1) [n_calib, 32] @ N(0, 1/32) [32, k]), so that X^T X has
           off-diagonal structure; drawn c, Z, then the two rank-32 factors.
  random_cache  uniformly random cache bytes (codes 0..255; NVFP4 scale
           bytes uniform in [0x30, 0x50), i.e. 0.5 .. 7.5; MXFP4 scale bytes
           uniform in [120, 130), i.e. 2^-7 .. 2^2) from numpy's PCG64 with
           the given seed: the input of full-size attention checks.

Draw order inside a workload: X, then W, then outlier positions.
"""

import numpy as np
import torch

SHAPES = {
    "tiny": {"m": 16, "n": 256, "k": 256},
    "decode": {"m": 8, "n": 14336, "k": 4096},
    "prefill": {"m": 4096, "n": 14336, "k": 4096},
    "rotated": {"m": 2048, "n": 28672, "k": 8192},
    "kv": {"batch": 32, "heads": 8, "tokens": 32768, "head_dim": 128},
}


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal(shape, std, g, device):
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std


def _student_t3(shape, g, device):
    # Z / sqrt(V / 3), V a chi-square with 3 degrees of freedom (three
    # squared standard normals): the textbook construction of Student-t(3).
    z = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    v = torch.zeros(shape, device=device, dtype=torch.float32)
    for _ in range(3):
        e = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        v += e * e
    return z / torch.sqrt(v / 3.0)


def _distinct(count, population, g, device):
    return torch.randperm(population, generator=g, device=device)[:count]


def tiny(device="cpu", seed=0):
    g = _gen(device, seed)
    x = _normal((16, 256), 1.0, g, device)
    w = _normal((256, 256), 0.02, g, device)
    idx = _distinct(66, 256 * 256, g, device)
    w.view(-1)[idx] *= 20.0
    return {"x": x, "w": w}


def decode(device="cpu", seed=0, n=14336):
    g = _gen(device, seed)
    x = _normal((8, 4096), 1.0, g, device).to(torch.bfloat16)
    w = _normal((n, 4096), 0.02, g, device).to(torch.bfloat16)
    return {"x": x, "w": w}


def prefill(device="cpu", seed=0, m=4096, n=14336):
    g = _gen(device, seed)
    x = _student_t3((m, 4096), g, device)
    w = _normal((n, 4096), 0.02, g, device).to(torch.bfloat16)
    ch = _distinct(41, 4096, g, device)
    x[:, ch] *= 50.0
    return {"x": x.to(torch.bfloat16), "w": w}


def rotated(device="cpu", seed=0, m=2048, n=28672):
    g = _gen(device, seed)
    x = _normal((m, 8192), 1.0, g, device).to(torch.bfloat16)
    w = _normal((n, 8192), 0.015, g, device).to(torch.bfloat16)
    return {"x": x, "w": w}


def kv(device="cpu", seed=0, batch=32, heads=8, tokens=32768, head_dim=128):
    g = _gen(device, seed)
    out = {}
    for name in ("k", "v"):
        c = torch.rand((heads, head_dim), generator=g, device=device) * 3.5 + 0.5
        t = torch.empty((batch, heads, tokens, head_dim), device=device, dtype=torch.bfloat16)
        for b in range(batch):       # per batch entry to bound the fp32 temporary
            z = torch.randn((heads, tokens, head_dim), generator=g, device=device)
            t[b] = (z * c[:, None, :]).to(torch.bfloat16)
        out[name] = t
        out["c_" + name] = c
    return out


def attention(device="cpu", seed=0, batch=32, kv_heads=8, q_heads=64, tokens=32768,
              head_dim=128):
    out = kv(device, seed, batch, kv_heads, tokens, head_dim)
    g = _gen(device, seed + 1)
    out["q"] = torch.randn((batch, q_heads, head_dim), generator=g, device=device).to(torch.bfloat16)
    return out


def calibration(device="cpu", seed=0, n_calib=2048, k=4096, rank=32):
    g = _gen(device, seed)
    c = torch.rand((k,), generator=g, device=device) * 3.5 + 0.5
    z = torch.randn((n_calib, k), generator=g, device=device)
    a = torch.randn((n_calib, rank), generator=g, device=device)
    b = torch.randn((rank, k), generator=g, device=device) / rank ** 0.5
    return (z * c + a @ b).to(torch.bfloat16)


def random_cache(batch, heads, tokens, head_dim, fmt="nvfp4", seed=0):
    """(codes [batch, heads, tokens, head_dim/2], scales [.., head_dim/block])
    as numpy uint8 arrays of random bytes."""
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, size=(batch, heads, tokens, head_dim // 2), dtype=np.uint8)
    if fmt == "nvfp4":
        scales = rng.integers(0x30, 0x50, size=(batch, heads, tokens, head_dim // 16), dtype=np.uint8)
    else:
        scales = rng.integers(120, 130, size=(batch, heads, tokens, head_dim // 32), dtype=np.uint8)
    return codes, scales


WORKLOADS = {"tiny": tiny, "decode": decode, "prefill": prefill,
             "rotated": rotated, "kv": kv}
