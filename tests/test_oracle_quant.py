"""Pins for the oracle's NVFP4 / MXFP4 quantize and dequantize (CPU only).

Hand-derived golden tensors, exact-rational property checks, brute-force
searches and invariants -- none of them re-computes the oracle's formulas.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle.formats import E2M1_MAGNITUDES


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def _num(v):
    if isinstance(v, str):
        if v == "-0.0":
            return -0.0
        if "^" in v:            # forms like "6*2^-127", "-6*2^-127", "2^-128"
            sign = -1.0 if v.startswith("-") else 1.0
            v = v.lstrip("-")
            mult, _, exp = v.rpartition("2^")
            m = float(mult.rstrip("*")) if mult else 1.0
            return sign * math.ldexp(m, int(exp))
        return float(v)
    return float(v)


def _hex(rows):
    return np.array([[int(b, 16) for b in r] for r in rows], dtype=np.uint8)


# --- golden ----------------------------------------------------------------

def test_nvfp4_worked_examples(golden_dir):
    g = _load(golden_dir, "nvfp4_worked.json")
    for case in g["cases"]:
        x = np.array([[_num(v) for v in r] for r in case["x"]], dtype=np.float32)
        packed, sb, s_t = oracle.nvfp4_quantize(x)
        assert s_t == np.float32(case["tensor_scale"]), case["name"]
        assert np.array_equal(sb, _hex(case["scales"])), case["name"]
        assert np.array_equal(packed, _hex(case["packed"])), case["name"]


def test_mxfp4_worked_example(golden_dir):
    g = _load(golden_dir, "mxfp4_worked.json")
    k = g["k"]
    x = np.zeros((len(g["x_rows"]), k), dtype=np.float32)
    for r, row in enumerate(g["x_rows"]):
        for i, v in row["nonzero"].items():
            x[r, int(i)] = _num(v)
    packed, sc = oracle.mxfp4_quantize(x)
    assert np.array_equal(sc, _hex(g["scales"]))
    exp = np.zeros((x.shape[0], k // 2), dtype=np.uint8)
    for r, row in enumerate(g["packed_nonzero"]):
        for i, b in row.items():
            exp[r, int(i)] = int(b, 16)
    assert np.array_equal(packed, exp)


def _codes_to_packed(rows):
    c = np.array(rows, dtype=np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def test_dequantize_worked_examples(golden_dir):
    g = _load(golden_dir, "dequant_worked.json")
    nv = g["nvfp4"]
    packed = _codes_to_packed(nv["codes_rows"])
    sb = _hex(nv["scales"])
    y = oracle.dequantize("nvfp4", packed, sb, np.float32(nv["tensor_scale"]), "f32")
    exp = np.zeros_like(y)
    for r, row in enumerate(nv["expected_f32_nonzero"]):
        for i, v in row.items():
            exp[r, int(i)] = _num(v)
    assert np.array_equal(y, exp)
    y8 = oracle.dequantize("nvfp4", packed, sb, np.float32(nv["tensor_scale"]), "e4m3")
    exp8 = np.zeros_like(y8)
    for r, row in enumerate(nv["expected_e4m3_nonzero"]):
        for i, v in row.items():
            exp8[r, int(i)] = int(v, 16)
    assert np.array_equal(y8, exp8)
    # bf16 output: every value above is exact in bf16
    yb = oracle.dequantize("nvfp4", packed, sb, np.float32(nv["tensor_scale"]), "bf16")
    yb_f = (yb.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(yb_f, exp)

    mx = g["mxfp4"]
    packed = _codes_to_packed(mx["codes_rows"])
    y = oracle.dequantize("mxfp4", packed, _hex(mx["scales"]), None, "f32")
    exp = np.zeros_like(y)
    for r, row in enumerate(mx["expected_f32_nonzero"]):
        for i, v in row.items():
            exp[r, int(i)] = _num(v)
    assert np.array_equal(y, exp)


# --- exact-rational properties --------------------------------------------

E4M3_GRID = [Fraction(float(v)) for v in oracle.e4m3_decode(np.arange(127))]
E2M1_MAGS = [Fraction(m) for m in E2M1_MAGNITUDES]


def _nearest_set(val, grid):
    """Indices of the grid points nearest to a rational value."""
    d = [abs(val - g) for g in grid]
    best = min(d)
    return [i for i, x in enumerate(d) if x == best]


def _f32_ulp(v):
    v = abs(float(v))
    if v == 0:
        return Fraction(2) ** -149
    return Fraction(float(np.spacing(np.float32(v))))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_nvfp4_properties_exact(seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_t(3, size=(3, 64)) * rng.choice([0.01, 1, 30], size=(3, 1))).astype(np.float32)
    x[1, 16:32] = 0.0                  # one all-zero block
    packed, sb, s_t = oracle.nvfp4_quantize(x)
    A = Fraction(float(np.max(np.abs(x))))
    # tensor scale: within one fp32 rounding of A / (6 * 448)
    assert abs(Fraction(float(s_t)) - A / 2688) <= _f32_ulp(s_t) / 2
    codes = oracle.unpack_nibbles(packed)
    st = Fraction(float(s_t))
    found_max_block = False
    for r in range(x.shape[0]):
        for b in range(x.shape[1] // 16):
            blk = x[r, 16 * b:16 * b + 16]
            a_b = Fraction(float(np.max(np.abs(blk))))
            ideal = a_b / (6 * st)
            code = int(sb[r, b])
            # the scale is a nearest E4M3 value to amax/(6 s_t), up to the
            # single fp32 rounding of that ratio
            lo = ideal - _f32_ulp(float(ideal)) / 2
            hi = ideal + _f32_ulp(float(ideal)) / 2
            ok = set(_nearest_set(lo, E4M3_GRID)) | set(_nearest_set(hi, E4M3_GRID)) | set(_nearest_set(ideal, E4M3_GRID))
            assert code in ok
            if a_b == A:
                assert code == 0x7E
                found_max_block = True
            S = E4M3_GRID[code] * st
            for i, xv in enumerate(blk.tolist()):
                c = int(codes[r, 16 * b + i])
                assert (c >> 3) == (1 if math.copysign(1, xv) < 0 else 0)
                if S == 0:
                    assert c & 7 == 0
                    continue
                t = abs(Fraction(xv)) / S
                # nearest E2M1 magnitude of |x|/S, allowing the two fp32
                # roundings (reciprocal, product) to move a value across a
                # tie by a few ulps; saturating above 6
                eps = t * Fraction(1, 2 ** 21)
                cand = set()
                for tv in (t - eps, t, t + eps):
                    cand |= set(_nearest_set(min(tv, Fraction(6)), E2M1_MAGS))
                assert (c & 7) in cand, (r, b, i, xv, float(t), c)
            # a block with a normal E4M3 scale maps its max element to +-6
            if code >= 8 and a_b > 0:
                imax = int(np.argmax(np.abs(blk)))
                assert int(codes[r, 16 * b + imax]) & 7 == 7
    assert found_max_block
    assert sb[1, 1] == 0 and np.all(codes[1, 16:32] & 7 == 0)


def test_mxfp4_scale_brute_force():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((4, 256)) * np.exp2(rng.integers(-40, 40, size=(4, 1)))).astype(np.float32)
    x[0, :32] = np.float32(0.09375)          # amax exactly 6 * 2^-6
    x[0, 32:64] = np.float32(6.0)            # amax exactly 6 * 2^0
    x[0, 64:96] = np.float32(6.0000005)      # just above -> next power
    packed, sc = oracle.mxfp4_quantize(x)
    codes = oracle.unpack_nibbles(packed)
    for r in range(4):
        for b in range(8):
            blk = x[r, 32 * b:32 * b + 32].astype(np.float64)
            a_b = float(np.max(np.abs(blk)))
            kk = next(k for k in range(-127, 128) if a_b <= 6 * math.ldexp(1.0, k))
            assert int(sc[r, b]) == kk + 127
            q = blk / math.ldexp(1.0, kk)        # exact
            assert np.max(np.abs(q)) <= 6.0       # never clips
            mx = int(codes[r, 32 * b + int(np.argmax(np.abs(blk)))]) & 7
            assert mx in (5, 6, 7)                # block max maps to 3, 4 or 6
            for i, qv in enumerate(q.tolist()):
                c = int(codes[r, 32 * b + i])
                assert (c & 7) in _nearest_set(Fraction(abs(qv)), E2M1_MAGS)
                if (c & 7) in (1, 3, 5) and len(_nearest_set(Fraction(abs(qv)), E2M1_MAGS)) > 1:
                    pytest.fail("tie not resolved to the even code")
    assert sc[0, 0] == 121 and sc[0, 1] == 127 and sc[0, 2] == 128


# --- invariants ------------------------------------------------------------

def _data(seed, rows=4, k=128):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((rows, k)) * 3).astype(np.float32)


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_sign_symmetry(fmt):
    x = _data(5)
    q = oracle.nvfp4_quantize if fmt == "nvfp4" else oracle.mxfp4_quantize
    a, b = q(x)[:2], q(-x)[:2]
    assert np.array_equal(a[1], b[1])
    assert np.array_equal(oracle.unpack_nibbles(a[0]) ^ 8, oracle.unpack_nibbles(b[0]))


@pytest.mark.parametrize("j", [-20, -3, 1, 7, 30])
def test_power_of_two_equivariance(j):
    x = _data(6)
    p0, s0, t0 = oracle.nvfp4_quantize(x)
    p1, s1, t1 = oracle.nvfp4_quantize(x * np.float32(2.0 ** j))
    assert np.array_equal(p0, p1) and np.array_equal(s0, s1)
    assert t1 == np.float32(t0 * np.float32(2.0 ** j))
    m0, c0 = oracle.mxfp4_quantize(x)
    m1, c1 = oracle.mxfp4_quantize(x * np.float32(2.0 ** j))
    assert np.array_equal(m0, m1)
    assert np.array_equal(c1.astype(int), c0.astype(int) + j)


def test_exact_round_trip():
    # x = v * S with S a representable block scale is recovered exactly
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 16, size=(3, 64)).astype(np.uint8)
    codes[:, ::16] = 7                                   # each block max = 6
    v = oracle.e2m1_decode(codes)
    sb = rng.integers(0x20, 0x7E, size=(3, 4)).astype(np.uint8)
    sb[0, 0] = 0x7E                                      # forces s_t = 1
    S = np.repeat(oracle.e4m3_decode(sb), 16, axis=1)
    x = (v * S).astype(np.float32)
    packed, sb2, s_t = oracle.nvfp4_quantize(x)
    assert s_t == 1.0
    assert np.array_equal(sb2, sb)
    assert np.array_equal(oracle.unpack_nibbles(packed) & 7, codes & 7)
    y = oracle.dequantize("nvfp4", packed, sb2, s_t, "f32")
    assert np.array_equal(np.abs(y), np.abs(x))
    # MXFP4 round trip with power-of-two scales
    ksc = rng.integers(100, 150, size=(3, 2)).astype(np.uint8)
    xm = (v * np.repeat(oracle.e8m0_decode(ksc), 32, axis=1)).astype(np.float32)
    pm, scm = oracle.mxfp4_quantize(xm)
    assert np.array_equal(scm.astype(int), ksc.astype(int) - 0)  # block max 6 -> k exact
    assert np.array_equal(np.abs(oracle.dequantize("mxfp4", pm, scm)), np.abs(xm))


def test_zero_tensor():
    x = np.zeros((2, 64), dtype=np.float32)
    x[1, 5] = -0.0
    p, s, t = oracle.nvfp4_quantize(x)
    assert t == 1.0 and not s.any()
    assert oracle.unpack_nibbles(p)[1, 5] == 8 and (oracle.unpack_nibbles(p) & 7).sum() == 0
    pm, sm = oracle.mxfp4_quantize(x)
    assert not sm.any() and oracle.unpack_nibbles(pm)[1, 5] == 8


def test_given_tensor_scale_used_as_is():
    x = _data(8)
    p, s, t = oracle.nvfp4_quantize(x, tensor_scale=np.float32(0.25))
    assert t == np.float32(0.25)
    # a tensor scale far too small saturates the block scales at 448
    p, s, t = oracle.nvfp4_quantize(x, tensor_scale=np.float32(1e-6))
    assert np.all(s == 0x7E)


def test_dequantize_error_bound():
    # |x - deq(x)| is at most half an E2M1 step times the block scale, plus
    # the saturation of the top step (6 -> at most a_b/S <= 6.x)
    x = _data(9, rows=8, k=256)
    p, sb, st = oracle.nvfp4_quantize(x)
    y = oracle.dequantize("nvfp4", p, sb, st, "f32").astype(np.float64)
    S = np.repeat(oracle.e4m3_decode(sb).astype(np.float64) * float(st), 16, axis=1)
    err = np.abs(x - y) / S
    assert np.all(err <= 1.0 + 1e-5)           # largest half-step is 1 (4..6)
    pm, sm = oracle.mxfp4_quantize(x)
    ym = oracle.dequantize("mxfp4", pm, sm, None, "f32").astype(np.float64)
    Sm = np.repeat(oracle.e8m0_decode(sm), 32, axis=1)
    assert np.all(np.abs(x - ym) / Sm <= 1.0)


def test_nvfp4_more_accurate_than_mxfp4_on_gaussian():
    # finer (E4M3, 16-element) scaling fits better than power-of-two scales
    # on 32 (pimento.cloud, section on the formats) -- a soft ordering
    x = np.random.default_rng(10).standard_normal((64, 1024)).astype(np.float32)
    p, s, t = oracle.nvfp4_quantize(x)
    e_nv = np.linalg.norm(x - oracle.dequantize("nvfp4", p, s, t)) / np.linalg.norm(x)
    pm, sm = oracle.mxfp4_quantize(x)
    e_mx = np.linalg.norm(x - oracle.dequantize("mxfp4", pm, sm)) / np.linalg.norm(x)
    assert e_nv < e_mx


def _scale_of(case):
    """Tensor scale of a rounding case: a sum of terms like "1", "2^-8",
    "3*2^-11", or the fp32 bit pattern in hex."""
    if "tensor_scale_bits" in case:
        return np.array([int(case["tensor_scale_bits"], 16)], dtype=np.uint32).view(np.float32)[0]
    if "tensor_scale" not in case:
        return None
    total = sum(_num(term) for term in case["tensor_scale"].split("+"))
    s = np.float32(total)
    assert float(s) == total          # every scale in the file is exact in fp32
    return s


def rounding_case_inputs(case):
    """(packed codes [1, k/2], scale bytes [1, k/block], tensor scale) of a
    case in dequant_rounding_worked.json."""
    packed = _codes_to_packed([case["codes"]])
    scales = _hex([case["scales"]])
    return packed, scales, _scale_of(case)


def rounding_case_expected(case):
    k = len(case["codes"])
    exp = np.zeros((1, k), dtype=np.uint16)
    for i, v in case["expected"].items():
        exp[0, int(i)] = int(v, 16)
    return exp


def test_dequantize_rounding_worked(golden_dir):
    # bf16 / f16 output rounding: ties to even, f16 overflow to infinity at
    # 65520, f16 subnormals, bf16 of fp32 subnormals (hand-derived)
    g = _load(golden_dir, "dequant_rounding_worked.json")
    for case in g["cases"]:
        packed, scales, ts = rounding_case_inputs(case)
        y = oracle.dequantize(case["fmt"], packed, scales, ts, case["out"])
        assert y.dtype == np.uint16, case["name"]
        assert np.array_equal(y, rounding_case_expected(case)), (case["name"], y)
