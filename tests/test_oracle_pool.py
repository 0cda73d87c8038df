"""The whole-tensor checker (oracle_pool) finds a planted difference in any
row and agrees with a direct oracle run (CPU only)."""

import numpy as np
import torch

import oracle
from oracle_pool import OracleRun


def _bf16_bits(x):
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_whole_tensor_check_finds_planted_differences():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((300, 256)) * 0.7).astype(np.float32)
    bits = _bf16_bits(x)
    xw = (bits.astype(np.uint32) << 16).view(np.float32)
    for fmt, had in (("nvfp4", 16), ("mxfp4", 0)):
        xr = oracle.hadamard_blocks(xw, had) if had else xw
        if fmt == "nvfp4":
            p, s, st = oracle.nvfp4_quantize(xr)
        else:
            (p, s), st = oracle.mxfp4_quantize(xr), None
        e8 = oracle.dequantize(fmt, p, s, st, "e4m3")
        with OracleRun(bits, "bf16", p, s, deq=e8, deq_dtype="e4m3", chunk_rows=37, workers=2) as run:
            if fmt == "nvfp4":
                assert np.float32(oracle.nvfp4_tensor_scale_from_amax(np.float32(run.amax(had)))) == st
            assert run.check(fmt, st, had) is None
        for what, arr in (("codes", p), ("scales", s), ("dequantized e4m3", e8)):
            bad = arr.copy()
            bad[211, 3] ^= 1
            args = dict(codes=p, scales=s, deq=e8)
            args["deq" if what.startswith("deq") else what] = bad
            with OracleRun(bits, "bf16", args["codes"], args["scales"], deq=args["deq"],
                           deq_dtype="e4m3", chunk_rows=37, workers=2) as run:
                assert run.check(fmt, st, had) == (what, 211)
