"""Pins for the oracle's FP4 KV cache append and decode attention (CPU only).

hyper.ai story on the NVFP4 KV cache: new K/V vectors go into the cache in
NVFP4, the cache is dequantized to FP8 before attention.  Each case below
has its answer fixed by hand or by the mathematics of softmax attention
(exact rows, means, 3:1 weights, head mapping, FP8 ties, saturation), so
that a dropped FP8 rounding, a wrong GQA index, a masking slip or a mixed-up
K/V operand fails one of them.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle.attention import attention_decode_ref, kv_append_ref, kv_fp8_values

E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
ONE_E4M3 = 0x38        # exponent 7, mantissa 0: 1.0
E4M3_1_125 = 0x39      # 1.125


def _pack(nibbles):
    n = np.asarray(nibbles, dtype=np.uint8)
    return (n[..., 0::2] | (n[..., 1::2] << 4)).astype(np.uint8)


def _nv_cache(nibbles, sbyte=ONE_E4M3):
    """nibbles [B, H, T, D] -> (codes, scales) with one scale byte for all."""
    nib = np.asarray(nibbles, dtype=np.uint8)
    codes = _pack(nib)
    scales = np.full(nib.shape[:-1] + (nib.shape[-1] // 16,), sbyte, dtype=np.uint8)
    return codes, scales


def _attend(k_nib, v_nib, q, seq_lens, scale, k_sb=ONE_E4M3, v_sb=ONE_E4M3, ts=1.0):
    kc, ks = _nv_cache(k_nib, k_sb)
    vc, vs = _nv_cache(v_nib, v_sb)
    return attention_decode_ref("nvfp4", np.asarray(q, dtype=np.float32), kc, ks, ts,
                                vc, vs, ts, seq_lens, scale)


def test_single_token_returns_its_value_row():
    # seq_len 1: the softmax weight is exactly 1, so out = V[0] (scale byte
    # 1.0, tensor scale 1: the FP8 values are the E2M1 values themselves)
    v_row = [1, 2, 3, 4, 5, 6, 7, 9, 10, 11, 12, 13, 14, 15, 0, 8]
    want = [0.5, 1, 1.5, 2, 3, 4, 6, -0.5, -1, -1.5, -2, -3, -4, -6, 0, -0.0]
    rng = np.random.default_rng(3)
    k = rng.integers(0, 16, size=(1, 1, 4, 16))
    v = np.zeros((1, 1, 4, 16), dtype=np.uint8)
    v[0, 0, 0] = v_row
    v[0, 0, 1:] = 7
    out = _attend(k, v, rng.standard_normal((1, 1, 16)), [1], 0.25)
    np.testing.assert_array_equal(out[0, 0], want)


def test_fp8_rounding_of_the_cache_is_applied():
    # E2M1 x E4M3 1.125: 1.5 -> 1.6875, 3 -> 3.375, 6 -> 6.75 are E4M3 ties
    # (between 1.625/1.75, 3.25/3.5, 6.5/7) and go to the even mantissa:
    # 1.75, 3.5, 7.  0.5 -> 0.5625 is exact.  Without the FP8 step the
    # output would hold the unrounded products.
    v = np.zeros((1, 1, 1, 16), dtype=np.uint8)
    v[0, 0, 0, :4] = [3, 5, 7, 1]
    v[0, 0, 0, 4:8] = [11, 13, 15, 9]
    k = np.zeros((1, 1, 1, 16), dtype=np.uint8)
    out = _attend(k, v, np.ones((1, 1, 16)), [1], 1.0, v_sb=E4M3_1_125)
    np.testing.assert_array_equal(out[0, 0, :8], [1.75, 3.5, 7.0, 0.5625,
                                                  -1.75, -3.5, -7.0, -0.5625])
    np.testing.assert_array_equal(out[0, 0, 8:], 0.0)


def test_equal_scores_give_the_mean_and_masked_tokens_do_not_count():
    # K = 0: every score is 0, the weights are 1/L, out = mean of V[:L].
    # Token t holds E2M1 code t % 8 in every channel; L = 8 -> mean
    # (0 + .5 + 1 + 1.5 + 2 + 3 + 4 + 6) / 8 = 2.25.  Tokens 8.. hold 6.0 and
    # must not enter.
    T = 12
    v = np.zeros((1, 1, T, 16), dtype=np.uint8)
    for t in range(T):
        v[0, 0, t] = t % 8 if t < 8 else 7
    k = np.zeros((1, 1, T, 16), dtype=np.uint8)
    out = _attend(k, v, np.ones((1, 1, 16)), [8], 0.125)
    np.testing.assert_allclose(out[0, 0], 2.25, rtol=0, atol=1e-15)


def test_two_tokens_with_three_to_one_weights():
    # K0 = e_0, K1 = 0, q = e_0: scores scale and 0; scale = ln 3 gives
    # weights 3/4 and 1/4, so out = 0.75 * 2 + 0.25 * 6 = 3.
    k = np.zeros((1, 1, 2, 16), dtype=np.uint8)
    k[0, 0, 0, 0] = 2                       # 1.0
    v = np.zeros((1, 1, 2, 16), dtype=np.uint8)
    v[0, 0, 0] = 4                          # 2.0
    v[0, 0, 1] = 7                          # 6.0
    q = np.zeros((1, 1, 16))
    q[0, 0, 0] = 1.0
    out = _attend(k, v, q, [2], math.log(3.0))
    np.testing.assert_allclose(out[0, 0], 3.0, rtol=1e-6)


def test_query_head_j_reads_kv_head_j_div_g():
    # 3 KV heads x G = 2: V of kv head h is constant E2M1[h + 2] = 1, 1.5, 2;
    # query heads 0..5 must see 1, 1, 1.5, 1.5, 2, 2 (head j // 2), not
    # j % 3.
    rng = np.random.default_rng(5)
    Hkv, G, T = 3, 2, 5
    k = rng.integers(0, 16, size=(1, Hkv, T, 16))
    v = np.zeros((1, Hkv, T, 16), dtype=np.uint8)
    for h in range(Hkv):
        v[0, h] = h + 2
    out = _attend(k, v, rng.standard_normal((1, Hkv * G, 16)), [T], 0.3)
    want = [1.0, 1.0, 1.5, 1.5, 2.0, 2.0]
    for j in range(Hkv * G):
        np.testing.assert_allclose(out[0, j], want[j], rtol=0, atol=1e-15)


def test_one_dominant_key_selects_its_value():
    # token 5's key is 6 e_0, the others 0.5 e_0; q = e_0, scale 20: score
    # gap 20 * 5.5 = 110, the other weights are below 8 e^-110.  V of token t
    # is E2M1[t % 8] (token 5: 3.0); K and V swapped would give 6 or 0.5.
    T = 8
    k = np.zeros((1, 1, T, 16), dtype=np.uint8)
    k[0, 0, :, 0] = 1
    k[0, 0, 5, 0] = 7
    v = np.zeros((1, 1, T, 16), dtype=np.uint8)
    for t in range(T):
        v[0, 0, t] = t % 8
    q = np.zeros((1, 1, 16))
    q[0, 0, 0] = 1.0
    out = _attend(k, v, q, [T], 20.0)
    np.testing.assert_allclose(out[0, 0], 3.0, rtol=1e-40, atol=0)


def test_per_sequence_lengths_and_empty_sequence():
    # sequence 0 has no tokens -> zeros; sequence 1 one token -> its row;
    # sequence 2 with K = 0 over 4 tokens -> the mean.
    T = 4
    k = np.zeros((3, 1, T, 16), dtype=np.uint8)
    v = np.zeros((3, 1, T, 16), dtype=np.uint8)
    v[:, 0, 0] = 4                       # 2.0
    v[:, 0, 1] = 7                       # 6.0
    v[:, 0, 2] = 2                       # 1.0
    v[:, 0, 3] = 3                       # 1.5
    out = _attend(k, v, np.ones((3, 1, 16)), [0, 1, 4], 1.0)
    np.testing.assert_array_equal(out[0, 0], 0.0)
    np.testing.assert_array_equal(out[1, 0], 2.0)
    np.testing.assert_allclose(out[2, 0], (2 + 6 + 1 + 1.5) / 4, rtol=0, atol=1e-15)


def test_scaling_q_and_softmax_scale_inversely_changes_nothing():
    rng = np.random.default_rng(9)
    k = rng.integers(0, 16, size=(2, 2, 7, 32))
    v = rng.integers(0, 16, size=(2, 2, 7, 32))
    q = rng.standard_normal((2, 4, 32)).astype(np.float32)
    a = _attend(k, v, q, [7, 3], 0.5)
    b = _attend(k, v, 2 * q, [7, 3], 0.25)
    np.testing.assert_array_equal(a, b)


def test_tensor_scale_enters_before_the_fp8_rounding():
    # E2M1 1.5 x E4M3 1.0 x tensor scale 1.125 = 1.6875 -> FP8 tie -> 1.75
    v = np.zeros((1, 1, 1, 16), dtype=np.uint8)
    v[0, 0, 0, 0] = 3
    out = _attend(np.zeros_like(v), v, np.ones((1, 1, 16)), [1], 1.0, ts=1.125)
    assert out[0, 0, 0] == 1.75


def test_mxfp4_cache_values_and_fp8_saturation():
    # E8M0 127 (1.0): E2M1 values as they are; E8M0 135 (2^8): 6 * 256 = 1536
    # saturates to the FP8 maximum 448, 0.5 * 256 = 128 is exact.
    nib = np.zeros((1, 1, 2, 32), dtype=np.uint8)
    nib[0, 0, 0, :4] = [7, 1, 13, 0]
    nib[0, 0, 1, :4] = [7, 1, 15, 0]
    codes = _pack(nib)
    scales = np.array([[[[127], [135]]]], dtype=np.uint8)
    vals = kv_fp8_values("mxfp4", codes, scales)
    np.testing.assert_array_equal(vals[0, 0, 0, :4], [6.0, 0.5, -3.0, 0.0])
    np.testing.assert_array_equal(vals[0, 0, 1, :4], [448.0, 128.0, -448.0, 0.0])
    out = attention_decode_ref("mxfp4", np.ones((1, 1, 32), dtype=np.float32),
                               np.zeros_like(codes), np.full_like(scales, 127), None,
                               codes, scales, None, [1], 1.0)
    np.testing.assert_array_equal(out[0, 0, :4], [6.0, 0.5, -3.0, 0.0])


def test_abs_weighted_sum_bounds_the_output():
    rng = np.random.default_rng(11)
    k = rng.integers(0, 16, size=(2, 2, 9, 16))
    v = rng.integers(0, 16, size=(2, 2, 9, 16))
    kc, ks = _nv_cache(k)
    vc, vs = _nv_cache(v)
    out, absw, flat = attention_decode_ref("nvfp4", rng.standard_normal((2, 4, 16)), kc, ks, 1.0,
                                           vc, vs, 1.0, [9, 4], 0.4, with_abs=True)
    assert np.all(np.abs(out) <= absw + 1e-12)
    assert np.all(absw <= 6.0 + 1e-12)
    # max_t p_t sum_t |V_t| >= sum_t p_t |V_t| >= |out|
    assert np.all(absw <= flat + 1e-12)


def _golden():
    here = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
    with open(os.path.join(here, "kv_append_worked.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("case", [0, 1])
def test_append_writes_the_hand_worked_row_at_its_positions(case):
    g = _golden()
    c = g["nvfp4"][case]
    row = np.array(g["row"], dtype=np.float32)
    B, H, Tn, T_max = 2, 1, 3, 8
    new = np.zeros((B, H, Tn, 16), dtype=np.float32)
    new[:] = row
    base_codes = np.full((B, H, T_max, 8), 0x5A, dtype=np.uint8)
    base_scales = np.full((B, H, T_max, 1), 0x11, dtype=np.uint8)
    codes, scales = kv_append_ref("nvfp4", base_codes, base_scales, new, [3, 6],
                                  tensor_scale=c["tensor_scale"])
    want_c = np.frombuffer(bytes.fromhex(c["codes_hex"]), dtype=np.uint8)
    want_s = int(c["scale_hex"], 16)
    written = {(0, 3), (0, 4), (0, 5), (1, 6), (1, 7)}       # (1, 8) is past the cache
    for b in range(B):
        for p in range(T_max):
            if (b, p) in written:
                np.testing.assert_array_equal(codes[b, 0, p], want_c)
                assert scales[b, 0, p, 0] == want_s
            else:
                np.testing.assert_array_equal(codes[b, 0, p], 0x5A)
                assert scales[b, 0, p, 0] == 0x11


def test_append_mxfp4_hand_worked_row():
    g = _golden()
    row = np.concatenate([np.array(g["row"], dtype=np.float32), np.zeros(16, np.float32)])
    new = row.reshape(1, 1, 1, 32)
    codes, scales = kv_append_ref("mxfp4", np.zeros((1, 1, 4, 16), np.uint8),
                                  np.zeros((1, 1, 4, 1), np.uint8), new, [2])
    np.testing.assert_array_equal(codes[0, 0, 2],
                                  np.frombuffer(bytes.fromhex(g["mxfp4"]["codes_hex"]), np.uint8))
    assert scales[0, 0, 2, 0] == int(g["mxfp4"]["scale_hex"], 16)
    np.testing.assert_array_equal(codes[0, 0, [0, 1, 3]], 0)


def test_append_negative_positions_are_dropped():
    new = np.ones((1, 1, 3, 16), dtype=np.float32)
    codes, scales = kv_append_ref("nvfp4", np.zeros((1, 1, 4, 8), np.uint8),
                                  np.zeros((1, 1, 4, 1), np.uint8), new, [-2],
                                  tensor_scale=1.0)
    # rows land at -2, -1 (dropped) and 0
    assert scales[0, 0, 0, 0] != 0
    np.testing.assert_array_equal(scales[0, 0, 1:], 0)
