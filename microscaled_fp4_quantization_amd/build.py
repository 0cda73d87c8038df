"""Build libfp4.so (the HIP kernels + C ABI) in-tree for gfx950 with hipcc.

Usage: python -m microscaled_fp4_quantization_amd.build
"""

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfp4.so")

SOURCES = [
    "fp4_api.cpp",
    "quantize.hip",
    "dequantize.hip",
    "gemm_simple.hip",
    "gemm_skinny.hip",
    "gemm_mx_stream.hip",
    "gemm_large.hip",
    "gemm.hip",
    "attention.hip",
    "gptq.hip",
]

# -ffp-contract=off: every a*b and a+b rounds on its own (no fused
# multiply-add), which the bit-exact quantization relies on.  Packed fp32
# instructions are switched off.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


# Scratch (bytes per lane) the main-loop kernels may use, from the compiler's
# resource report.  The large GEMMs keep their operands in registers; when a
# code change makes the compiler leave a k-step rolled, their fragment arrays
# go to scratch (1.5-1.7 KiB per lane) and the kernel runs ~70x slower with
# correct results, so the build refuses it.  (The MXFP4 kernel spills ~116
# bytes in its epilogue only.)
SCRATCH_LIMITS = {"gemm_nv4w": 32, "gemm_large_mx": 128}


def hipcc():
    return os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


def _check_scratch(src, report):
    name = None
    for line in report.splitlines():
        if "Function Name:" in line:
            name = line.split("Function Name:")[1].strip().split()[0]
        elif "ScratchSize [bytes/lane]:" in line and name:
            size = int(line.split("ScratchSize [bytes/lane]:")[1].split()[0])
            for kernel, limit in SCRATCH_LIMITS.items():
                if kernel in name and size > limit:
                    raise RuntimeError("%s: %s uses %d bytes of scratch per lane (limit %d): "
                                       "its main loop no longer stays in registers" % (src, name, size, limit))


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + FLAGS + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if src == "gemm_large.hip":
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    if src == "gemm_large.hip":
        _check_scratch(src, r.stderr)
    return obj


def build(verbose=True):
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
