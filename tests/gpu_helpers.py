"""Helpers for the GPU parity tests: device selection, exact host copies and
the comparison metrics.  Inputs are generated once and fed unchanged to both
the HIP library and the CPU oracle."""

import sys

import numpy as np
import pytest
import torch

DEV = "cuda:0"


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def note(msg):
    """Name the case before a GPU step (flushed), so a failing run says which."""
    print("[gpu] " + msg, flush=True)
    sys.stdout.flush()


def host_f32(t):
    """Exact fp32 numpy copy of a CPU/GPU tensor (bf16/fp16 widen exactly)."""
    return t.detach().to("cpu").to(torch.float32).numpy()


def np_u8(t):
    return t.detach().cpu().numpy()


def rel_fro(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return np.linalg.norm(got - ref) / (den if den > 0 else 1.0)


def bf16_round_f64(ref):
    """float64 -> nearest bf16 value (via fp32; the double rounding cannot
    matter at the tolerance these tests use), back as float64."""
    t = torch.from_numpy(np.asarray(ref, dtype=np.float64)).to(torch.bfloat16)
    return t.to(torch.float64).numpy()
