"""Benchmark of the FP4 hot path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the hot path over one batch of synthetic input with
every input already resident in HBM:
  rotated_nv (default) fused blockwise Hadamard (16) + NVFP4 quantize of the
           activations X bf16 [2048, 8192] with the tensor scale computed
           from the data, then the NVFP4 W4A4 GEMM against the offline-rotated
           and quantized W [28672, 8192], bf16 out: the largest W4A4
           configuration (962 GFLOP per step).
  rotated_mx the same step in MXFP4 (Hadamard 32, E8M0 scales).
  prefill  NVFP4 quantize of X [4096, 4096] + GEMM vs W [14336, 4096].
  decode   online NVFP4 quantize of X bf16 [8, 4096] (tensor scale
           computed from the data) + NVFP4 W4A4 GEMM against a pre-quantized
           W [14336, 4096], bf16 out, as one fp4_quantize_gemm call (a single
           launch; it also writes X's codes, scales and tensor scale).
           Steps cycle over 17 distinct weight copies (over 2x the 256 MB
           last-level cache) so the weights stream from HBM as they do layer
           after layer.
  kv       NVFP4 quantize of K and V [32*8*32768, 128] bf16 with their given
           tensor scales + dequantize of both to FP8 E4M3.
  w4a16    W4A16 decode: X bf16 [8, 4096] as it is times the NVFP4 weight
           W [14336, 4096] (fp4_gemm_w4a16), bf16 out; weight copies cycled
           as for decode.
  mse      NVFP4 quantization of the weight W [14336, 4096] bf16 with the
           least-squared-error block scale (fp4_quantize_mse, tensor scale
           computed from the data): compute-bound, fp64 error sums.
  attention  one decode step over the NVFP4 KV cache of the kv workload
           ([32, 8, 32768, 128], quantized once): append the new token's K
           and V (fp4_kv_append, given tensor scales) + attention of 64 query
           heads (8 per KV head, bf16 q) over all 32768 tokens with the cache
           dequantized to FP8 (fp4_attention_decode), bf16 out.
  gptq     MR-GPTQ of the decode workload's weight W [14336, 4096] to NVFP4
           (blockwise Hadamard, 2048 calibration rows, fp4_gptq_quantize):
           the offline weight path; fp64 arithmetic (roofline "alu").
Prints one JSON line.  The step first runs untimed for --preheat-s seconds
(the GPU's clocks settle after a second or so of load), then W warm-up steps;
the timed region is K steps back to back between one pair of HIP events
(value, ms_per_step).  The dominant kernel is then timed
the same way over the K steps' launches of it alone; its algorithmic bytes
(or flops) per launch over that duration give the roofline figure.  A
separate sampling phase (at least 100 launches or 200 ms, in 10 windows of
back-to-back launches) gives the median, p10 and p90 per launch of the step,
the dominant kernel and, where the step launches it on its own, the
activation quantize (reported with its algorithmic bytes and HBM fraction).
HBM-bound workloads also report the warm figure (one weight copy, resident in
the last-level cache).  The CPU oracle is timed on a bounded sample of the
same workload on the host.
"""

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W4A4 NVFP4 GEMM TFLOPS + quantize GB/s, % of MI355X roofline"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"fp4": 10100.0, "f16": 2500.0}
FP64_FMA_PEAK_TFLOPS = 78.6    # fp64 vector with fused multiply-adds (GPTQ's products)
# fp64 vector: 78.6 TFLOP/s counts a fused multiply-add as two; one fp64
# instruction per lane and clock is 256 CUs x 64 lanes x 2.4 GHz = 39.3 T/s.
# The MSE search counts 4 operations per value and candidate (v S_b,
# x - ., d d, err + .) and issues them as 3 instructions (the first two
# fused: v S_b is exact in fp64, so one rounding of x - v S_b is what the
# definition computes; d d and the sum must round separately), so its
# operations peak at 39.3 x 4 / 3 = 52.4 T/s.
FP64_PEAK_TOPS = 39.3 * 4 / 3
MSE_CANDIDATES = 126            # positive finite E4M3 scale bytes
MSE_FLOPS_PER_VALUE = 4         # per candidate: v S_b, x - ., d d, err + .
MALL_BYTES = 256 << 20


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="rotated_nv",
                   choices=["decode", "prefill", "rotated_nv", "rotated_mx", "kv", "mse", "w4a16",
                            "attention", "gptq"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--stat-ms", type=float, default=200.0,
                   help="least GPU time of each sampling phase (median / p10 / p90)")
    p.add_argument("--no-stats", action="store_true", help="skip the sampling phases")
    p.add_argument("--preheat-s", type=float, default=1.0,
                   help="seconds of untimed steps before the warm-up steps (the clocks settle)")
    p.add_argument("--tp", type=int, default=1,
                   help="one GPU's share of a column-parallel split of the weights over TP GPUs: "
                        "n / TP weight rows (decode, prefill, rotated_nv, rotated_mx, w4a16)")
    p.add_argument("--copy-bytes", type=int, default=0,
                   help="after the timed region, copy this many bytes device to device three "
                        "times: the plain copy that scales rocprofv3 FETCH_SIZE / WRITE_SIZE")
    p.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="print the traffic entry for --workload from two rocprofv3 --pmc runs "
                        "(FETCH_SIZE, then WRITE_SIZE) of this script with --copy-bytes, and exit")
    return p.parse_args()


# Dominant kernel of each workload (name as rocprofv3 reports it) and the
# sources its code comes from: a recorded HBM traffic figure is used only
# while these files are unchanged.
DOMINANT = {
    "decode": ("gemm_nv_stream<2, 1, 1>", ["gemm_skinny.hip"]),
    "prefill": ("gemm_nv4w<", ["gemm_large.hip"]),
    "rotated_nv": ("gemm_nv4w<", ["gemm_large.hip"]),
    "rotated_mx": ("gemm_large_mx<", ["gemm_large.hip"]),
    "kv": ("blocks_kernel<0, 1, 0, false>", ["quantize.hip", "device_common.hpp"]),
    "mse": ("quantize_mse_kernel<1, true>", ["quantize.hip", "device_common.hpp"]),
    "w4a16": ("gemm_nv_stream<2, 2, 1>", ["gemm_skinny.hip"]),
    "attention": ("attn_decode_kernel<0, 1>", ["attention.hip", "device_common.hpp"]),
    "gptq": ("gemm_f64_kernel", ["gptq.hip", "quantize.hip", "device_common.hpp"]),
}
COPY_KERNEL = "copyBuffer"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def source_digest(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "microscaled_fp4_quantization_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload):
    """HBM bytes per launch of the dominant kernel from the recorded counter
    runs, each counter scaled by what it reads for the plain copy; None when
    there is no record or the kernel's sources changed since."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_digest") != source_digest(DOMINANT[workload][1]):
        return None
    fetch = rec["fetch_kib"] * rec["copy_bytes"] / rec["copy_fetch_kib"]
    write = rec["write_kib"] * rec["copy_bytes"] / rec["copy_write_kib"]
    return int(round(fetch + write))


def summarize_pmc(workload, fetch_dir, write_dir, copy_bytes):
    import csv
    import glob

    def per_dispatch(d, counter, pattern, last=0):
        rows = []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    if r["Counter_Name"].startswith(counter) and pattern in r["Kernel_Name"]:
                        rows.append((int(r["Dispatch_Id"]), float(r["Counter_Value"])))
        rows.sort()
        if last:                           # the calibration copies run last
            rows = rows[-last:]
        if not rows:
            raise SystemExit("no %s dispatches of %r under %s" % (counter, pattern, d))
        return sum(v for _, v in rows) / len(rows), len(rows)

    name, files = DOMINANT[workload]
    fk, nf = per_dispatch(fetch_dir, "FETCH_SIZE", name)
    wk, nw = per_dispatch(write_dir, "WRITE_SIZE", name)
    cf, _ = per_dispatch(fetch_dir, "FETCH_SIZE", COPY_KERNEL, last=3)
    cw, _ = per_dispatch(write_dir, "WRITE_SIZE", COPY_KERNEL, last=3)
    entry = {"kernel": name, "fetch_kib": round(fk, 1), "write_kib": round(wk, 1),
             "dispatches": [nf, nw], "copy_bytes": copy_bytes, "copy_fetch_kib": round(cf, 1),
             "copy_write_kib": round(cw, 1), "source_digest": source_digest(files)}
    print(json.dumps({workload: entry}))


class Lib:
    """Direct ctypes calls with pre-built arguments (low host overhead).  Each
    call holds the tensors its pointers come from (the `keep` default), so
    that none is freed and its memory handed out again while the call is
    still in use."""

    def __init__(self, torch, fq):
        self.torch = torch
        self.L = fq.lib()
        self.stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    @staticmethod
    def p(t):
        return None if t is None else ctypes.c_void_p(t.data_ptr())

    def check(self, st, what):
        if st != 0:
            raise RuntimeError("%s failed: %s" % (what, self.L.fp4_status_string(st).decode()))

    def quantize_call(self, fmt, x, codes, scales, ts, mode, ws, hadamard=False):
        from microscaled_fp4_quantization_amd import fp4
        fn = self.L.fp4_hadamard_quantize if hadamard else self.L.fp4_quantize
        dt = {self.torch.bfloat16: fp4.BF16, self.torch.float32: fp4.F32, self.torch.float16: fp4.F16}[x.dtype]
        need = self.L.fp4_quantize_workspace_size(fmt, mode, x.shape[0], x.shape[1])
        args = (fmt, self.p(x), dt, x.shape[0], x.shape[1], self.p(codes), self.p(scales),
                self.p(ts), mode, self.p(ws) if need else None, need, self.stream)
        return lambda keep=(x, codes, scales, ts, ws): self.check(fn(*args), "quantize")

    def gemm_call(self, fmt, a, b, c, c_dtype):
        (ac, asc, at), (bc, bsc, bt) = a, b
        m, n, k = ac.shape[0], bc.shape[0], ac.shape[1] * 2
        need = self.L.fp4_gemm_workspace_size(fmt, m, n, k)
        ws = self.torch.empty(need, dtype=self.torch.uint8, device=c.device) if need else None
        args = (fmt, m, n, k, self.p(ac), self.p(asc), self.p(at), self.p(bc), self.p(bsc),
                self.p(bt), self.p(c), c_dtype, self.p(ws), need, self.stream)
        fn = self.L.fp4_gemm
        return lambda keep=(a, b, c, ws): self.check(fn(*args), "gemm")

    def quantize_gemm_call(self, fmt, x, a, b, c, c_dtype, ws):
        from microscaled_fp4_quantization_amd import fp4
        (ac, asc, at), (bc, bsc, bt) = a, b
        m, k, n = x.shape[0], x.shape[1], bc.shape[0]
        dt = {self.torch.bfloat16: fp4.BF16, self.torch.float32: fp4.F32, self.torch.float16: fp4.F16}[x.dtype]
        need = self.L.fp4_quantize_gemm_workspace_size(fmt, m, n, k)
        args = (fmt, self.p(x), dt, m, n, k, self.p(ac), self.p(asc), self.p(at), self.p(bc),
                self.p(bsc), self.p(bt), self.p(c), c_dtype, self.p(ws) if need else None, need,
                self.stream)
        fn = self.L.fp4_quantize_gemm
        return lambda keep=(x, a, b, c, ws): self.check(fn(*args), "quantize_gemm")

    def quantize_mse_call(self, x, codes, scales, ts, mode, ws):
        from microscaled_fp4_quantization_amd import fp4
        dt = {self.torch.bfloat16: fp4.BF16, self.torch.float32: fp4.F32, self.torch.float16: fp4.F16}[x.dtype]
        need = self.L.fp4_quantize_workspace_size(fp4.NVFP4, mode, x.shape[0], x.shape[1])
        args = (self.p(x), dt, x.shape[0], x.shape[1], self.p(codes), self.p(scales), self.p(ts), mode,
                self.p(ws) if need else None, need, self.stream)
        fn = self.L.fp4_quantize_mse
        return lambda keep=(x, codes, scales, ts, ws): self.check(fn(*args), "quantize_mse")

    def w4a16_call(self, fmt, x, b, c, c_dtype):
        from microscaled_fp4_quantization_amd import fp4
        bc, bsc, bt = b
        m, k, n = x.shape[0], x.shape[1], bc.shape[0]
        dt = {self.torch.bfloat16: fp4.BF16, self.torch.float32: fp4.F32, self.torch.float16: fp4.F16}[x.dtype]
        need = self.L.fp4_gemm_w4a16_workspace_size(fmt, m, n, k)
        ws = self.torch.empty(need, dtype=self.torch.uint8, device=x.device) if need else None
        args = (fmt, self.p(x), dt, m, n, k, self.p(bc), self.p(bsc), self.p(bt), self.p(c), c_dtype,
                self.p(ws), need, self.stream)
        fn = self.L.fp4_gemm_w4a16
        return lambda keep=(x, b, c, ws): self.check(fn(*args), "gemm_w4a16")

    def kv_append_call(self, fmt, x, cache, positions, ts):
        from microscaled_fp4_quantization_amd import fp4
        codes, scales = cache
        B, H, tn, d = x.shape
        dt = {self.torch.bfloat16: fp4.BF16, self.torch.float32: fp4.F32, self.torch.float16: fp4.F16}[x.dtype]
        args = (fmt, self.p(x), dt, B, H, tn, d, self.p(positions), self.p(codes), self.p(scales),
                self.p(ts), codes.shape[2], self.stream)
        fn = self.L.fp4_kv_append
        return lambda keep=(x, cache, positions, ts): self.check(fn(*args), "kv_append")

    def attention_call(self, fmt, q, kcache, kts, vcache, vts, lens, scale, out, out_dtype, ws):
        from microscaled_fp4_quantization_amd import fp4
        B, hq, d = q.shape
        (kc, ks), (vc, vs) = kcache, vcache
        dt = {self.torch.bfloat16: fp4.BF16, self.torch.float16: fp4.F16}[q.dtype]
        args = (fmt, self.p(q), dt, B, hq, kc.shape[1], d, self.p(kc), self.p(ks), self.p(kts),
                self.p(vc), self.p(vs), self.p(vts), kc.shape[2], self.p(lens), ctypes.c_float(scale),
                self.p(out), out_dtype, self.p(ws), ws.numel(), self.stream)
        fn = self.L.fp4_attention_decode
        return lambda keep=(q, kcache, kts, vcache, vts, lens, out, ws): self.check(fn(*args), "attention_decode")

    def gptq_call(self, fmt, w, x, codes, scales, ts, ws):
        from microscaled_fp4_quantization_amd import fp4
        n, k = w.shape
        dt = {self.torch.bfloat16: fp4.BF16, self.torch.float32: fp4.F32, self.torch.float16: fp4.F16}
        args = (fmt, self.p(w), dt[w.dtype], n, k, self.p(x), dt[x.dtype], x.shape[0],
                ctypes.c_double(0.01), 1, self.p(codes), self.p(scales), self.p(ts), self.p(ws),
                ws.numel(), self.stream)
        fn = self.L.fp4_gptq_quantize
        return lambda keep=(w, x, codes, scales, ts, ws): self.check(fn(*args), "gptq_quantize")

    def dequant_call(self, fmt, codes, scales, ts, out, out_dtype):
        rows, k = codes.shape[0], codes.shape[1] * 2
        args = (fmt, self.p(codes), self.p(scales), self.p(ts), rows, k, self.p(out), out_dtype, self.stream)
        fn = self.L.fp4_dequantize
        return lambda keep=(codes, scales, ts, out): self.check(fn(*args), "dequantize")


def gemm_bytes(m, n, k, fmt, out_bytes):
    bs = 16 if fmt == "nvfp4" else 32
    return (m + n) * (k // 2 + k // bs) + m * n * out_bytes + (8 if fmt == "nvfp4" else 0)


def quant_bytes(rows, k, fmt, in_bytes):
    bs = 16 if fmt == "nvfp4" else 32
    return rows * k * in_bytes + rows * k // 2 + rows * k // bs + (4 if fmt == "nvfp4" else 0)


def setup(workload, torch, fq, lib, tp=1):
    """Returns dict with: steps (list of per-step callables split into
    pre/dominant/post), flops, bytes, dominant info, oracle sample fn."""
    from microscaled_fp4_quantization_amd import fp4, workloads
    dev = torch.device("cuda:0")
    NV, MX = fp4.NVFP4, fp4.MXFP4
    W = {}
    if workload in ("decode", "prefill"):
        m = 8 if workload == "decode" else 4096
        d = (workloads.decode(device=dev, n=14336 // tp) if workload == "decode"
             else workloads.prefill(device=dev, n=14336 // tp))
        x, w = d["x"], d["w"]
        n, k = w.shape
        wq = fq.quantize(w, "nvfp4")
        per = gemm_bytes(m, n, k, "nvfp4", 2)
        copies = 1 if workload == "prefill" else max(1, -(-2 * MALL_BYTES // (n * k // 2 + n * k // 16)))
        wqs = [wq] + [tuple(t.clone() for t in wq) for _ in range(copies - 1)]
        xc = torch.empty((m, k // 2), dtype=torch.uint8, device=dev)
        xs = torch.empty((m, k // 16), dtype=torch.uint8, device=dev)
        xt = torch.empty(1, dtype=torch.float32, device=dev)
        ws = torch.empty(1 << 16, dtype=torch.uint8, device=dev)   # quantize workspace
        c = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        if workload == "decode":
            # one call: the activations are quantized inside the GEMM launch
            gs = [lib.quantize_gemm_call(NV, x, (xc, xs, xt), wqi, c, fp4.BF16, ws) for wqi in wqs]
            pre, name = [], "fp4_quantize_gemm (NVFP4, m=%d)" % m
            per += 2 * m * k                  # the bf16 activations read
        else:
            pre = [lib.quantize_call(NV, x, xc, xs, xt, fp4.TSCALE_COMPUTE, ws)]
            gs = [lib.gemm_call(NV, (xc, xs, xt), wqi, c, fp4.BF16) for wqi in wqs]
            name = "fp4_gemm (NVFP4, m=%d)" % m
        if workload == "prefill":
            W["quant"] = dict(calls=pre, bytes=quant_bytes(m, k, "nvfp4", 2),
                              name="fp4_quantize (NVFP4, bf16 [%d, %d], tensor scale computed)" % (m, k))
        else:
            W["warm"] = [gs[0]]              # one weight copy: resident in the last-level cache
        W.update(pre=pre, dominant=gs, post=[], flops=2 * m * n * k,
                 dom_name=name,
                 dom_units=per if workload == "decode" else 2 * m * n * k,
                 dom_bound="hbm" if workload == "decode" else "mfma",
                 dom_peak=HBM_PEAK_GBS if workload == "decode" else MFMA_PEAK_TFLOPS["f16"],
                 quant_bytes=quant_bytes(m, k, "nvfp4", 2),
                 config={"workload": workload, "m": m, "n": n, "k": k, "format": "nvfp4",
                         "x_dtype": "bf16", "out_dtype": "bf16", "weight_copies": copies},
                 dtype="e2m1 x e4m3 -> f16 mfma, f32 acc",
                 host=dict(x=x.float().cpu().numpy(), w=w.float().cpu().numpy(), fmt="nvfp4",
                           hadamard=False))
    elif workload in ("rotated_nv", "rotated_mx"):
        fmt = "nvfp4" if workload == "rotated_nv" else "mxfp4"
        f = NV if fmt == "nvfp4" else MX
        d = workloads.rotated(device=dev, n=28672 // tp)
        x, w = d["x"], d["w"]
        m, k = x.shape
        n = w.shape[0]
        bs = 16 if fmt == "nvfp4" else 32
        wq = fq.hadamard_quantize(w, fmt)
        xc = torch.empty((m, k // 2), dtype=torch.uint8, device=dev)
        xs = torch.empty((m, k // bs), dtype=torch.uint8, device=dev)
        xt = torch.empty(1, dtype=torch.float32, device=dev) if fmt == "nvfp4" else None
        ws = torch.empty(1 << 16, dtype=torch.uint8, device=dev)   # quantize workspace
        c = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        q = lib.quantize_call(f, x, xc, xs, xt, fp4.TSCALE_COMPUTE, ws, hadamard=True)
        g = lib.gemm_call(f, (xc, xs, xt), wq, c, fp4.BF16)
        W["quant"] = dict(calls=[q], bytes=quant_bytes(m, k, fmt, 2),
                          name="fp4_hadamard_quantize (%s, Hadamard %d, bf16 [%d, %d]%s)" % (
                              fmt.upper(), bs, m, k,
                              ", tensor scale computed" if fmt == "nvfp4" else ""))
        W.update(pre=[q], dominant=[g], post=[], flops=2 * m * n * k,
                 dom_name="fp4_gemm (%s, m=%d)" % (fmt.upper(), m), dom_units=2 * m * n * k,
                 dom_bound="mfma",
                 dom_peak=MFMA_PEAK_TFLOPS["fp4" if fmt == "mxfp4" else "f16"],
                 quant_bytes=quant_bytes(m, k, fmt, 2),
                 config={"workload": workload, "m": m, "n": n, "k": k, "format": fmt,
                         "hadamard": bs, "x_dtype": "bf16", "out_dtype": "bf16"},
                 dtype="e2m1 x e2m1 fp4 mfma (e8m0 scales), f32 acc" if fmt == "mxfp4"
                 else "e2m1 x e4m3 -> f16 mfma, f32 acc",
                 host=dict(x=x.float().cpu().numpy(), w=w.float().cpu().numpy(), fmt=fmt,
                           hadamard=True))
    elif workload == "w4a16":
        d = workloads.decode(device=dev, n=14336 // tp)
        x, w = d["x"], d["w"]
        m, k = x.shape
        n = w.shape[0]
        wq = fq.quantize(w, "nvfp4")
        copies = max(1, -(-2 * MALL_BYTES // (n * k // 2 + n * k // 16)))
        wqs = [wq] + [tuple(t.clone() for t in wq) for _ in range(copies - 1)]
        c = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        gs = [lib.w4a16_call(NV, x, wqi, c, fp4.BF16) for wqi in wqs]
        W["warm"] = [gs[0]]
        per = (n * (k // 2 + k // 16) + 4) + 2 * m * k + 2 * m * n
        W.update(pre=[], dominant=gs, post=[], flops=2 * m * n * k,
                 dom_name="fp4_gemm_w4a16 (NVFP4 weights, bf16 X, m=%d)" % m, dom_units=per,
                 dom_bound="hbm", dom_peak=HBM_PEAK_GBS, quant_bytes=0,
                 config={"workload": "w4a16", "m": m, "n": n, "k": k, "format": "nvfp4",
                         "x_dtype": "bf16", "out_dtype": "bf16", "weight_copies": copies},
                 dtype="e2m1 x e4m3 -> f16, bf16 X -> f16 (power-of-two prescale), f16 mfma, f32 acc",
                 host=dict(x=x.float().cpu().numpy(), w=w.float().cpu().numpy(), fmt="nvfp4",
                           hadamard=False, w4a16=True))
    elif workload == "mse":
        w = workloads.decode(device=dev)["w"]
        n, k = w.shape
        codes = torch.empty((n, k // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((n, k // 16), dtype=torch.uint8, device=dev)
        ts = torch.empty(1, dtype=torch.float32, device=dev)
        ws = torch.empty(1 << 16, dtype=torch.uint8, device=dev)   # quantize workspace
        q = lib.quantize_mse_call(w, codes, scales, ts, fp4.TSCALE_COMPUTE, ws)
        nblocks = n * k // 16
        W.update(pre=[], dominant=[q], post=[], flops=0,
                 dom_name="fp4_quantize_mse (NVFP4, bf16 [%d, %d])" % (n, k),
                 dom_units=nblocks * MSE_CANDIDATES * 16 * MSE_FLOPS_PER_VALUE,
                 dom_bound="alu", dom_peak=FP64_PEAK_TOPS,
                 quant_bytes=quant_bytes(n, k, "nvfp4", 2),
                 config={"workload": "mse", "rows": n, "k": k, "format": "nvfp4",
                         "scale_rule": "least squared error", "x_dtype": "bf16"},
                 dtype="f32 quantize, f64 error sums",
                 host=dict(w=w))
    elif workload == "gptq":
        w = workloads.decode(device=dev)["w"]
        n, k = w.shape
        N = 2048
        x = workloads.calibration(device=dev, n_calib=N, k=k)
        codes = torch.empty((n, k // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((n, k // 16), dtype=torch.uint8, device=dev)
        ts = torch.empty(1, dtype=torch.float32, device=dev)
        ws = torch.empty(fq.lib().fp4_gptq_workspace_size(n, k, N), dtype=torch.uint8, device=dev)
        q = lib.gptq_call(NV, w, x, codes, scales, ts, ws)
        flops = 2 * N * k * k + 2 * k ** 3 // 3 + n * k * k
        W.update(pre=[], dominant=[q], post=[], flops=flops,
                 dom_name="fp4_gptq_quantize (NVFP4, W bf16 [%d, %d], %d calibration rows; all "
                          "its kernels)" % (n, k, N),
                 dom_units=flops, dom_bound="alu", dom_peak=FP64_FMA_PEAK_TFLOPS, quant_bytes=0,
                 config={"workload": "gptq", "rows": n, "k": k, "n_calib": N, "format": "nvfp4",
                         "hadamard": 16, "damp": 0.01, "w_dtype": "bf16", "x_dtype": "bf16"},
                 dtype="f64 (Hessian, Cholesky, inverse, error correction), f32 quantize",
                 host=dict(gptq=dict(w=w[:64].float().cpu().numpy(), x=x.float().cpu().numpy(),
                                     w_amax_rows=w.float().abs().amax().item())))
    elif workload == "attention":
        B, H, T, D, G = 32, 8, 32768, 128, 8
        d = workloads.attention(device=dev, batch=B, kv_heads=H, q_heads=H * G, tokens=T,
                                head_dim=D)
        caches, news, tss, host = [], [], [], {}
        ws = torch.empty(1 << 16, dtype=torch.uint8, device=dev)   # quantize workspace
        for name in ("k", "v"):
            x = d.pop(name)
            codes = torch.empty((B, H, T, D // 2), dtype=torch.uint8, device=dev)
            scales = torch.empty((B, H, T, D // 16), dtype=torch.uint8, device=dev)
            ts = torch.empty(1, dtype=torch.float32, device=dev)
            # the cache as it stands before the step (offline, untimed)
            lib.quantize_call(NV, x.view(-1, D), codes.view(-1, D // 2), scales.view(-1, D // 16),
                              ts, fp4.TSCALE_COMPUTE, ws)()
            news.append(x[:, :, T - 1:T, :].contiguous())        # the step's new token
            host[name] = x[0, 0].float().cpu().numpy()           # CPU-baseline sample
            caches.append((codes, scales))
            tss.append(ts)
            del x
        torch.cuda.synchronize()
        q = d["q"]
        host["q"] = q[0, :G].float().cpu().numpy()
        pos = torch.full((B,), T - 1, dtype=torch.int32, device=dev)
        lens = torch.full((B,), T, dtype=torch.int32, device=dev)
        out = torch.empty((B, H * G, D), dtype=torch.bfloat16, device=dev)
        wsa = torch.empty(max(16, fq.lib().fp4_attention_workspace_size(B, H * G, H, D, T)),
                          dtype=torch.uint8, device=dev)
        scale = 1.0 / (D ** 0.5)
        pre = [lib.kv_append_call(NV, news[0], caches[0], pos, tss[0]),
               lib.kv_append_call(NV, news[1], caches[1], pos, tss[1])]
        att = lib.attention_call(NV, q, caches[0], tss[0], caches[1], tss[1], lens, scale, out,
                                 fp4.BF16, wsa)
        attn_bytes = 2 * B * H * T * (D // 2 + D // 16) + 2 * q.numel() + 2 * out.numel() + 4 * B + 8
        append_bytes = 2 * (B * H * D * 2 + B * H * (D // 2 + D // 16)) + 4 * B + 8
        W.update(pre=pre, dominant=[att], post=[], flops=0,
                 dom_name="fp4_attention_decode (NVFP4 cache [32,8,32768,128], 64 query heads; "
                          "split kernel + merge kernel)",
                 dom_units=attn_bytes, dom_bound="hbm", dom_peak=HBM_PEAK_GBS,
                 step_bytes=attn_bytes + append_bytes, quant_bytes=0,
                 config={"workload": "attention", "batch": B, "kv_heads": H, "q_heads": H * G,
                         "tokens": T, "head_dim": D, "format": "nvfp4", "q_dtype": "bf16",
                         "out_dtype": "bf16"},
                 dtype="e2m1 x e4m3 -> fp8 e4m3 (table) -> bf16 mfma (q.K), f32 softmax, "
                       "f16 weights x f16 V mfma, f32 acc",
                 host=dict(attention=host))
    else:  # kv
        d = workloads.kv(device=dev)
        calls_q, calls_d, outs = [], [], []
        ts_list = []
        for name in ("k", "v"):
            x2 = d[name].view(-1, 128)
            rows = x2.shape[0]
            amax = torch.max(torch.abs(x2)).float()
            ts = (amax / 2688.0).reshape(1).contiguous()
            codes = torch.empty((rows, 64), dtype=torch.uint8, device=dev)
            scales = torch.empty((rows, 8), dtype=torch.uint8, device=dev)
            out = torch.empty((rows, 128), dtype=torch.uint8, device=dev)
            calls_q.append(lib.quantize_call(NV, x2, codes, scales, ts, fp4.TSCALE_GIVEN, None))
            calls_d.append(lib.dequant_call(NV, codes, scales, ts, out, fp4.E4M3))
            outs.append((codes, scales, out))
            ts_list.append(ts)
        rows = d["k"].numel() // 128
        W.update(pre=[], dominant=calls_q, post=calls_d, flops=0,
                 dom_name="fp4_quantize (NVFP4 given scale, bf16 [2^23,128])",
                 dom_units=quant_bytes(rows, 128, "nvfp4", 2), dom_bound="hbm", dom_peak=HBM_PEAK_GBS,
                 quant_bytes=quant_bytes(rows, 128, "nvfp4", 2),
                 dequant_bytes=rows * 128 * 1.5625,
                 config={"workload": "kv", "shape": [32, 8, 32768, 128], "format": "nvfp4",
                         "x_dtype": "bf16", "out_dtype": "e4m3"},
                 dtype="f32 (quantize arithmetic), e4m3 out",
                 host=dict(kv=d, ts=ts_list))
    return W


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        return 1


def cpu_baseline(workload, W, seconds):
    """The oracle timed on a bounded sample of the workload.  `cores` is the
    number of threads the sample runs on: 1 for the elementwise NumPy stages,
    NumPy's BLAS threads where the sample includes an fp64 matrix product."""
    res = _cpu_baseline(workload, W, seconds, blas_threads())
    res["host_cores"] = len(os.sched_getaffinity(0))
    res["blas_threads"] = blas_threads()
    return res


def _cpu_baseline(workload, W, seconds, cores):
    import numpy as np
    import oracle
    h = W["host"]
    if workload == "mse":
        rows = 32                        # bounded sample: the first rows of W
        x = h["w"][:rows].float().cpu().numpy()
        st = oracle.nvfp4_tensor_scale(h["w"].float().cpu().numpy())
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.nvfp4_quantize_mse(x, st)
            reps += 1
            if time.perf_counter() - t0 >= seconds:
                break
        dt = (time.perf_counter() - t0) / reps
        return {"value": rows * x.shape[1] * 2.5625 / dt / 1e9, "unit": "GB/s", "cores": 1,
                "kind": "oracle", "sample": "MSE quantize of %d of the %d W rows, %d reps" % (
                    rows, h["w"].shape[0], reps)}
    if workload == "gptq":
        # bounded sample: the full Hessian and factor, error correction of the
        # first 64 weight rows (rows are independent once the factor exists)
        g = h["gptq"]
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.gptq_quantize("nvfp4", g["w"], g["x"])
            reps += 1
            if time.perf_counter() - t0 >= seconds:
                break
        dt = (time.perf_counter() - t0) / reps
        N, k = g["x"].shape
        rows = g["w"].shape[0]
        flops = 2 * N * k * k + 2 * k ** 3 // 3 + rows * k * k
        return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
                "sample": "GPTQ of %d of the 14336 weight rows with the full %dx%d Hessian and "
                          "its factor, %d reps" % (rows, k, k, reps)}
    if workload == "attention":
        # bounded sample: one (sequence, KV head) of the 256, all 32768 tokens,
        # its 8 query heads; the cache rows quantized on the host
        a = h["attention"]
        T, D = a["k"].shape
        kc, ks, kts = oracle.nvfp4_quantize(a["k"])
        vc, vs, vts = oracle.nvfp4_quantize(a["v"])
        kc, ks = kc.reshape(1, 1, T, D // 2), ks.reshape(1, 1, T, D // 16)
        vc, vs = vc.reshape(1, 1, T, D // 2), vs.reshape(1, 1, T, D // 16)
        q = a["q"][None]
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.attention_decode_ref("nvfp4", q, kc, ks, kts, vc, vs, vts, [T], 1.0 / D ** 0.5)
            reps += 1
            if time.perf_counter() - t0 >= seconds:
                break
        dt = (time.perf_counter() - t0) / reps
        nbytes = 2 * T * (D // 2 + D // 16) + 2 * 2 * q.size
        return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
                "sample": "attention of 8 query heads over one of the 256 (sequence, KV head) "
                          "caches, 32768 tokens, %d reps" % reps}
    if workload == "kv":
        # bounded sample: the first rows of K, quantized and dequantized
        rows = 1 << 16
        x = h["kv"]["k"].view(-1, 128)[:rows].float().cpu().numpy()
        st = np.float32(h["ts"][0].item())
        reps, t0 = 0, time.perf_counter()
        while True:
            p, s, _ = oracle.nvfp4_quantize(x, st)
            oracle.dequantize("nvfp4", p, s, st, "e4m3")
            reps += 1
            if time.perf_counter() - t0 >= seconds:
                break
        dt = (time.perf_counter() - t0) / reps
        gbs = (rows * 128 * 2.5625 + rows * 128 * 1.5625) / dt / 1e9
        return {"value": gbs, "unit": "GB/s", "cores": 1, "kind": "oracle",
                "sample": "quantize + FP8 dequantize of %d of the 2^23 K rows, %d reps" % (rows, reps)}
    fmt = h["fmt"]
    x, w = h["x"], h["w"]
    if h.get("w4a16"):
        pw, sw, tw = oracle.nvfp4_quantize(w)
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.gemm_w4a16_ref(fmt, x, pw, sw, tw)
            reps += 1
            if time.perf_counter() - t0 >= seconds:
                break
        dt = (time.perf_counter() - t0) / reps
        return {"value": 2.0 * x.shape[0] * w.shape[0] * w.shape[1] / dt / 1e12, "unit": "TFLOP/s",
                "cores": cores, "kind": "oracle",
                "sample": "w4a16 step (X %dx%d, W %dx%d), %d reps" % (x.shape + w.shape + (reps,))}
    if workload in ("prefill", "rotated_nv", "rotated_mx"):
        x = x[:64]                        # bounded sample: 64 activation rows
    if workload in ("rotated_nv", "rotated_mx"):
        w = w[:4096]                      # and 4096 of the 28672 weight rows
    b = 16 if fmt == "nvfp4" else 32
    wr = oracle.hadamard_blocks(w, b) if h["hadamard"] else w
    if fmt == "nvfp4":
        pw, sw, tw = oracle.nvfp4_quantize(wr)
    else:
        (pw, sw), tw = oracle.mxfp4_quantize(wr), None
    reps, t0 = 0, time.perf_counter()
    while True:
        xr = oracle.hadamard_blocks(x, b) if h["hadamard"] else x
        if fmt == "nvfp4":
            pa, sa, ta = oracle.nvfp4_quantize(xr)
        else:
            (pa, sa), ta = oracle.mxfp4_quantize(xr), None
        oracle.gemm_ref(fmt, pa, sa, ta, pw, sw, tw)
        reps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = (time.perf_counter() - t0) / reps
    flops = 2.0 * x.shape[0] * w.shape[0] * w.shape[1]
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": "%s step (activation %squantize + GEMM reference) on X rows %d of %d and "
                      "W rows %d of %d (W quantized offline, untimed), %d reps" % (
                          workload, "Hadamard + " if h["hadamard"] else "", x.shape[0],
                          h["x"].shape[0], w.shape[0], h["w"].shape[0], reps)}


def sample(torch, fn, per_call, min_ms, cycles_per_ms, windows=10):
    """GPU time of one call of fn: the median, p10 and p90 over `windows`
    windows of back-to-back calls, each between its own HIP event pair, with
    at least 100 calls or min_ms of GPU time in all.  A GPU spin ahead of
    the windows keeps the host's enqueueing out of the measurement."""
    import math
    import numpy as np
    ev = lambda: torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0, e1 = ev(), ev()
    t0 = time.perf_counter()
    e0.record()
    for i in range(5):
        fn(i)
    e1.record()
    host_ms = (time.perf_counter() - t0) * 1e3 / 5
    torch.cuda.synchronize()
    est = max(e0.elapsed_time(e1) / 5, 1e-3)
    n = max(100, int(math.ceil(min_ms / est)))
    n = min(int(math.ceil(n / windows)) * windows, 20000)
    per = n // windows
    evs = [ev() for _ in range(windows + 1)]
    torch.cuda.synchronize()
    n_hot = int(min(10000, max(4, 40.0 / est)))
    torch.cuda._sleep(int((2.0 * host_ms * (n + n_hot) + 2.0) * cycles_per_ms))
    for i in range(n_hot):              # the GPU at full clock before the first window
        fn(i)
    evs[0].record()
    for w in range(windows):
        for i in range(w * per, (w + 1) * per):
            fn(i)
        evs[w + 1].record()
    torch.cuda.synchronize()
    v = np.array([evs[w].elapsed_time(evs[w + 1]) / (per * per_call) for w in range(windows)])
    return {"median_ms": round(float(np.median(v)), 5), "p10_ms": round(float(np.percentile(v, 10)), 5),
            "p90_ms": round(float(np.percentile(v, 90)), 5), "mean_ms": round(float(v.mean()), 5),
            "windows": windows, "calls": n}


def main():
    args = parse()
    if args.summarize_pmc:
        summarize_pmc(args.workload, args.summarize_pmc[0], args.summarize_pmc[1],
                      args.copy_bytes)
        return
    if args.gpus != 1:
        print("bench.py: this library runs on one GPU; --gpus %d is not supported (the "
              "multi-GPU sharding of the path is not built)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    import microscaled_fp4_quantization_amd as fq
    torch.cuda.set_device(0)
    lib = Lib(torch, fq)
    if args.tp != 1 and args.workload not in ("decode", "prefill", "rotated_nv", "rotated_mx", "w4a16"):
        print("bench.py: --tp applies to the GEMM workloads only", file=sys.stderr)
        sys.exit(2)
    W = setup(args.workload, torch, fq, lib, tp=args.tp)
    if args.tp != 1:
        W["config"]["tp_share"] = "1/%d of the weight rows (one GPU of a column-parallel split)" % args.tp
    pre, dom, post = W["pre"], W["dominant"], W["post"]
    ndom = len(dom)

    def step(i):
        for f in pre:
            f()
        if args.workload == "kv":
            for f in dom:
                f()
        else:
            dom[i % ndom]()
        for f in post:
            f()

    def dominant(i):
        # the dominant kernel's launches of step i, alone
        if args.workload == "kv":
            for f in dom:
                f()
        else:
            dom[i % ndom]()
    launches_per_step = len(dom) if args.workload == "kv" else 1

    # Pre-heat: the GPU's clocks settle only after a second or so of load
    # (the first steps of a process run up to ~10 % slower), so the step runs
    # untimed for --preheat-s seconds before the W warm-up steps.
    t_end = time.perf_counter() + args.preheat_s
    i = 0
    while time.perf_counter() < t_end:
        for _ in range(64):
            step(i)
            i += 1
        torch.cuda.synchronize()
    w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0.record()
    for i in range(args.warmup):
        step(i)
    w1.record()
    torch.cuda.synchronize()
    est_step_ms = max(w0.elapsed_time(w1) / max(1, args.warmup), 1e-3)
    # Steps run untimed right before each timed region, after its GPU spin:
    # ~40 ms of the step's own work.  After any idle stretch (the spin, a host
    # pause) the GPU runs the next ~20 ms of load up to 25 % slower before its
    # clocks settle; the timed steps start after that.
    n_hot = int(min(10000, max(4, 40.0 / est_step_ms)))
    # Host cost of enqueuing one step (the GPU may be faster than the host).
    t0 = time.perf_counter()
    for i in range(min(args.warmup, 20)):
        step(i)
    host_step = (time.perf_counter() - t0) / max(1, min(args.warmup, 20))
    torch.cuda.synchronize()
    # Calibrate a GPU spin that outlasts enqueuing all K steps, so the timed
    # steps run back to back on the GPU and the events measure GPU time only.
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    torch.cuda._sleep(1 << 20)
    c1.record()
    torch.cuda.synchronize()
    ms_per_cycle = c0.elapsed_time(c1) / float(1 << 20)
    spin_ms = 2.0 * host_step * 1e3 * (args.steps + n_hot + 4) + 2.0
    spin_cycles = int(spin_ms / ms_per_cycle)
    # Timed region: K whole steps back to back, one event pair around them.
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    torch.cuda._sleep(spin_cycles)
    for i in range(n_hot):
        step(i)
    start.record()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    end.record()
    enqueue_s = time.perf_counter() - t0
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # The dominant kernel's launch duration: the same K steps' launches of it
    # back to back between one event pair on the bench stream (an event pair
    # around each single launch would add its own dispatch and timestamp
    # cost, several microseconds, to a kernel this short).
    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    torch.cuda._sleep(spin_cycles)
    for i in range(n_hot):
        step(i)
    d0.record()
    for i in range(args.steps):
        dominant(i)
    d1.record()
    torch.cuda.synchronize()
    dom_avg = d0.elapsed_time(d1) / (args.steps * launches_per_step)
    stats = {}
    if not args.no_stats:
        stats["step"] = sample(torch, step, 1, args.stat_ms, 1.0 / ms_per_cycle)
        stats["dominant"] = sample(torch, dominant, launches_per_step, args.stat_ms,
                                   1.0 / ms_per_cycle)
        if "quant" in W:
            qc = W["quant"]["calls"]
            stats["quantize"] = sample(torch, lambda i: qc[i % len(qc)](), 1, args.stat_ms,
                                       1.0 / ms_per_cycle)
        if "warm" in W:
            wc = W["warm"]
            stats["warm"] = sample(torch, lambda i: wc[i % len(wc)](), 1, args.stat_ms,
                                   1.0 / ms_per_cycle)
    if args.copy_bytes:
        # the plain copy of known size that calibrates the HBM byte counters
        src = torch.empty(args.copy_bytes, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    ms_total = start.elapsed_time(end)
    ms_step = ms_total / args.steps
    gpu_fed = enqueue_s * 1e3 < spin_ms     # host stayed ahead of the GPU

    if W["dom_bound"] == "hbm":
        achieved = W["dom_units"] / (dom_avg * 1e-3) / 1e9
        unit = "GB/s"
    elif W["dom_bound"] == "alu":
        achieved = W["dom_units"] / (dom_avg * 1e-3) / 1e12
        unit = "T fp64 operations/s" if args.workload == "mse" else "TFLOP/s (fp64)"
    else:
        achieved = W["dom_units"] / (dom_avg * 1e-3) / 1e12
        unit = "TFLOP/s"
    if args.workload == "kv":
        value = 2 * (W["quant_bytes"] + W["dequant_bytes"]) / (ms_step * 1e-3) / 1e9
        vunit = "GB/s"
    elif args.workload == "mse":
        value = W["quant_bytes"] / (ms_step * 1e-3) / 1e9
        vunit = "GB/s"
    elif args.workload == "attention":
        value = W["step_bytes"] / (ms_step * 1e-3) / 1e9
        vunit = "GB/s"
    elif args.workload == "gptq":
        value = W["flops"] / (ms_step * 1e-3) / 1e12
        vunit = "TFLOP/s (fp64)"
    else:
        value = W["flops"] / (ms_step * 1e-3) / 1e12
        vunit = "TFLOP/s"
    out = {
        "metric": METRIC, "value": round(value, 3), "unit": vunit, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "preheat_s": args.preheat_s,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": W["dtype"], "data": "synthetic (seeded, see workloads.py)",
        "config": W["config"],
        "roofline": {"bound": W["dom_bound"], "achieved": round(achieved, 2),
                     "peak": W["dom_peak"], "unit": unit,
                     "frac": round(achieved / W["dom_peak"], 4),
                     "traffic": recorded_traffic(args.workload),
                     "kernel": W["dom_name"], "avg_ms": round(dom_avg, 5),
                     "timing": "HIP events around the %d back-to-back launches of it "
                               "that the %d timed steps make" % (args.steps * launches_per_step,
                                                                  args.steps),
                     "units_per_launch": W["dom_units"]},
        "host_wall_s": round(wall, 4),
        "host_enqueue_ms_per_step": round(enqueue_s * 1e3 / args.steps, 4),
        "gpu_fed_by_host": bool(gpu_fed),
    }
    if W["dom_bound"] == "mfma":
        rf = out["roofline"]
        rf["frac_fp4"] = round(achieved / MFMA_PEAK_TFLOPS["fp4"], 4)
        if W["config"].get("format") == "nvfp4":
            rf["peak_unit_used"] = "f16 matrix cores"
            rf["note"] = ("NVFP4 runs as exact fp16 products (E2M1 x E4M3 is exact in fp16; the "
                          "scaled FP4 MFMA takes only E8M0 scales per 32 values) on the f16 matrix "
                          "cores: frac is against their %.0f TFLOP/s; against the FP4 peak the "
                          "ceiling is %.3f" % (MFMA_PEAK_TFLOPS["f16"],
                                               MFMA_PEAK_TFLOPS["f16"] / MFMA_PEAK_TFLOPS["fp4"]))
    if stats:
        out["stats"] = stats
    if "quant" in W:
        qb = W["quant"]["bytes"]
        q = {"kernel": W["quant"]["name"], "bytes_per_launch": qb,
             "bytes_rule": "input read once + codes + scales (+4 B tensor scale)"}
        if "quantize" in stats:
            qms = stats["quantize"]["median_ms"]
            q.update({"median_ms": qms, "achieved_gbs": round(qb / (qms * 1e-3) / 1e9, 1),
                      "peak_gbs": HBM_PEAK_GBS,
                      "frac": round(qb / (qms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                      "timing": "median over windows of back-to-back launches of it alone "
                                "(all its kernels)"})
        out["quantize"] = q
    elif args.workload == "decode":
        out["quantize"] = {"kernel": "inside the fp4_quantize_gemm launch (not timed alone)",
                           "bytes_per_launch": W["quant_bytes"]}
    elif args.workload == "kv" and "dominant" in stats:
        qms = stats["dominant"]["median_ms"]
        out["quantize"] = {"kernel": W["dom_name"], "bytes_per_launch": W["dom_units"],
                           "median_ms": qms,
                           "achieved_gbs": round(W["dom_units"] / (qms * 1e-3) / 1e9, 1),
                           "peak_gbs": HBM_PEAK_GBS,
                           "frac": round(W["dom_units"] / (qms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                           "timing": "median over windows of back-to-back launches of it alone"}
    if "warm" in stats and W["dom_bound"] == "hbm":
        wms = stats["warm"]["median_ms"]
        out["warm"] = {"median_ms": wms,
                       "achieved_gbs": round(W["dom_units"] / (wms * 1e-3) / 1e9, 1),
                       "frac": round(W["dom_units"] / (wms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                       "note": "one weight copy, resident in the 256 MB last-level cache: not an "
                               "HBM figure"}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.workload, W, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
