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

Draw order inside a workload: X, then W, then outlier positions.
"""

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


WORKLOADS = {"tiny": tiny, "decode": decode, "prefill": prefill,
             "rotated": rotated, "kv": kv}
