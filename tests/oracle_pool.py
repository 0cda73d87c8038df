"""Whole-tensor oracle checks spread over host processes (test infrastructure).

The CPU oracle is plain single-threaded NumPy; a full-size tensor (2^30
values of a KV-cache tensor, the 28672 x 8192 rotated weight) would take it
minutes.  Rows are independent once the tensor scale is fixed, so the rows
are cut into chunks and each chunk is checked by the oracle in its own
process ("spawn": the workers import NumPy and the oracle only and never
touch the GPU).  Inputs and the GPU's results are handed over as .npy files
under a temporary directory and memory-mapped by the workers.

Bit-for-bit comparisons only: a worker returns the first row of its chunk
whose codes, scale bytes or dequantized bytes differ, or None.
"""

import multiprocessing as mp
import os
import shutil
import tempfile

import numpy as np


def _workers():
    # the GPU machine grants one GPU's share of the host: at most 16 threads
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _widen(bits, dtype):
    """Stored 16-bit input bits -> exact float32 (bf16 or f16)."""
    if dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float32)
    return np.asarray(bits, dtype=np.float32)


def _first_bad(a, b):
    bad = np.nonzero(np.any(np.asarray(a) != np.asarray(b), axis=1))[0]
    return None if bad.size == 0 else int(bad[0])


def _chunk_amax(args):
    d, r0, r1, dtype, had = args
    import oracle
    x = _widen(np.load(os.path.join(d, "x.npy"), mmap_mode="r")[r0:r1], dtype)
    if had:
        x = oracle.hadamard_blocks(x, had)
    return float(np.max(np.abs(x))) if x.size else 0.0


def _chunk_check(args):
    d, r0, r1, dtype, had, fmt, s_t, deq = args
    import oracle
    x = _widen(np.load(os.path.join(d, "x.npy"), mmap_mode="r")[r0:r1], dtype)
    if had:
        x = oracle.hadamard_blocks(x, had)
    if fmt == "nvfp4":
        p, s, _ = oracle.nvfp4_quantize(x, np.float32(s_t))
    else:
        p, s = oracle.mxfp4_quantize(x)
    codes = np.load(os.path.join(d, "codes.npy"), mmap_mode="r")[r0:r1]
    scales = np.load(os.path.join(d, "scales.npy"), mmap_mode="r")[r0:r1]
    for name, got, exp in (("scales", scales, s), ("codes", codes, p)):
        r = _first_bad(got, exp)
        if r is not None:
            return (name, r0 + r)
    if deq:
        y = np.load(os.path.join(d, "deq.npy"), mmap_mode="r")[r0:r1]
        e = oracle.dequantize(fmt, p, s, None if fmt == "mxfp4" else np.float32(s_t), deq)
        r = _first_bad(y, e)
        if r is not None:
            return ("dequantized " + deq, r0 + r)
    return None


class OracleRun:
    """Hands host copies of a quantization's input and the GPU's outputs to
    worker processes and checks every row against the oracle."""

    def __init__(self, x_bits, dtype, codes, scales, deq=None, deq_dtype=None, chunk_rows=None,
                 workers=None):
        self.dir = tempfile.mkdtemp(prefix="fp4_oracle_", dir="/dev/shm" if os.path.isdir("/dev/shm") else None)
        self.rows, self.k = x_bits.shape
        self.dtype = dtype
        self.deq_dtype = deq_dtype
        np.save(os.path.join(self.dir, "x.npy"), x_bits)
        np.save(os.path.join(self.dir, "codes.npy"), codes)
        np.save(os.path.join(self.dir, "scales.npy"), scales)
        if deq is not None:
            np.save(os.path.join(self.dir, "deq.npy"), deq)
        # about 4 Mi values per chunk: ~100 MB of NumPy temporaries per worker
        self.chunk = chunk_rows or max(1, (4 << 20) // self.k)
        self.workers = workers or _workers()
        self.pool = None

    def _ranges(self):
        return [(r, min(r + self.chunk, self.rows)) for r in range(0, self.rows, self.chunk)]

    def amax(self, hadamard=0):
        """max |x| (after the blockwise rotation when hadamard > 0), exact."""
        jobs = [(self.dir, r0, r1, self.dtype, hadamard) for r0, r1 in self._ranges()]
        return max(self._pool().map(_chunk_amax, jobs, chunksize=1))

    def check(self, fmt, s_t=None, hadamard=0):
        """First mismatch (what, row) over all rows, or None."""
        jobs = [(self.dir, r0, r1, self.dtype, hadamard, fmt, s_t, self.deq_dtype)
                for r0, r1 in self._ranges()]
        first = None
        for res in self._pool().imap(_chunk_check, jobs, chunksize=1):
            if res is not None and first is None:
                first = res
        return first

    def _pool(self):
        if self.pool is None:
            self.pool = mp.get_context("spawn").Pool(self.workers)
        return self.pool

    def close(self):
        if self.pool is not None:
            self.pool.terminate()
            self.pool.join()
            self.pool = None
        shutil.rmtree(self.dir, ignore_errors=True)

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
