"""Pins of the oracle's exact roundings and its INT2 codec.

Everything here is checked against something other than the oracle itself:
torch's own bf16 conversion, an enumeration of all fp16 values, exact rational
arithmetic (``fractions.Fraction``) and brute-force nearest-level search.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

from oracle import qevict_oracle as O

ALL_FP16 = np.unique(np.arange(65536, dtype=np.uint16).view(np.float16).astype(np.float64))
ALL_FP16 = ALL_FP16[np.isfinite(ALL_FP16)]


def test_to_bf16_matches_torch_on_fp32_values():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-30, 1e-3, 1.0, 1e3, 1e30)])
    x = x.astype(np.float32).astype(np.float64)        # single rounding fp32 -> bf16 in torch
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.to_bf16(x), ref)


def test_to_bf16_ties_to_even():
    # 1 + 2**-8 lies half way between bf16 neighbours 1 and 1 + 2**-7: even mantissa wins
    assert O.to_bf16(1.0 + 2.0 ** -8) == 1.0
    assert O.to_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6


@pytest.mark.parametrize("seed", range(3))
def test_directed_fp16_rounding_against_enumeration(seed):
    rng = np.random.default_rng(seed)
    x = np.concatenate([rng.uniform(-70000.0, 70000.0, 3000) / 10 ** rng.integers(0, 9, 3000),
                        ALL_FP16[rng.integers(0, ALL_FP16.size, 500)]])
    x = x[np.abs(x) < 65504]
    i = np.searchsorted(ALL_FP16, x, side="right") - 1
    np.testing.assert_array_equal(O.rd_fp16(x), ALL_FP16[i])
    j = np.searchsorted(ALL_FP16, x, side="left")
    np.testing.assert_array_equal(O.ru_fp16(x), ALL_FP16[j])


def test_fp16_range_error():
    with pytest.raises(O.RangeError):
        O.ru_fp16(np.array([65505.0]))
    with pytest.raises(O.RangeError):
        O.rd_fp16(np.array([-65520.0]))


def _bf16_group(rng, n, scale=1.0):
    x = rng.standard_normal(n) * scale
    return O.to_bf16(x)


@settings(max_examples=300, deadline=None)
@given(st.integers(0, 2 ** 31 - 1), st.sampled_from([1e-6, 1e-3, 0.5, 1.0, 10.0, 300.0]),
       st.sampled_from([4, 16, 32, 64, 128]), st.sampled_from([2, 4]))
def test_group_quantization_exact_definition(seed, scale, n, bits):
    rng = np.random.default_rng(seed)
    x = _bf16_group(rng, n, scale)
    L = 2 ** bits - 1
    codes, off, scl = O.quantize_groups(x[None, :], axis=1, bits=bits)
    codes, off, scl = codes[0], float(off[0]), float(scl[0])
    mn, mx = Fraction(float(x.min())), Fraction(float(x.max()))
    # off is the largest fp16 value <= min; scl the smallest fp16 value >= (max - off) / L
    i = np.searchsorted(ALL_FP16, float(x.min()), side="right") - 1
    assert off == ALL_FP16[i] and Fraction(off) <= mn
    target = (mx - Fraction(off)) / L
    cand = [f for f in ALL_FP16[np.searchsorted(ALL_FP16, float(target)) - 2:][:6] if Fraction(f) >= target]
    assert scl == min(cand)
    # nearest level, ties to the upper level, found by brute force in exact arithmetic
    for xi, c in zip(x, codes):
        if scl == 0:
            assert c == 0
            continue
        dist = [abs(Fraction(float(xi)) - (Fraction(off) + k * Fraction(scl))) for k in range(L + 1)]
        best = min(dist)
        assert c == max(k for k in range(L + 1) if dist[k] == best)
    # round-trip bound |x - x_hat| <= scl / 2, exact
    xh = O.dequantize(codes[None, :], np.array([off]), np.array([scl]), axis=1)[0]
    for xi, yi in zip(x, xh):
        assert abs(Fraction(float(xi)) - Fraction(float(yi))) <= Fraction(scl) / 2


def test_exactly_recoverable_group():
    off, s = -1.5, 0.75          # fp16 and bf16 exact
    x = np.array([off + k * s for k in (0, 1, 2, 3, 3, 0, 2, 1)])
    codes, o, sc = O.quantize_groups(x[None], axis=1)
    assert o[0] == off and sc[0] == s
    np.testing.assert_array_equal(codes[0], [0, 1, 2, 3, 3, 0, 2, 1])
    np.testing.assert_array_equal(O.dequantize(codes, o, sc, axis=1)[0], x)


def test_int4_exactly_recoverable_group_uses_all_sixteen_levels():
    off, s = -3.0, 0.25
    ks = [0, 15, 7, 8, 1, 14, 3, 12, 5, 10, 2, 13, 4, 11, 6, 9]
    x = np.array([off + k * s for k in ks])
    codes, o, sc = O.quantize_groups(x[None], axis=1, bits=4)
    assert o[0] == off and sc[0] == s
    np.testing.assert_array_equal(codes[0], ks)
    np.testing.assert_array_equal(O.dequantize(codes, o, sc, axis=1)[0], x)


def test_int4_midpoints_round_up_and_error_shrinks():
    """Half-way values take the upper of the 16 levels; on the same group the INT4
    reconstruction error bound scl/2 is a fifth of the INT2 one (range / 15 vs / 3)."""
    x = np.array([[0.0, 0.5, 1.5, 13.5, 14.5, 15.0, 7.0]])
    codes, o, sc = O.quantize_groups(x, axis=1, bits=4)
    assert o[0] == 0.0 and sc[0] == 1.0
    np.testing.assert_array_equal(codes[0], [0, 1, 2, 14, 15, 15, 7])
    rng = np.random.default_rng(9)
    y = O.to_bf16(rng.standard_normal((64, 32)))
    _, _, s2 = O.quantize_groups(y, axis=1, bits=2)
    _, _, s4 = O.quantize_groups(y, axis=1, bits=4)
    assert np.all(s4 * 5 <= s2 * (1 + 2.0 ** -9)) and np.all(s4 * 5 >= s2 * (1 - 2.0 ** -9))


def test_midpoints_round_up():
    """A value half way between two levels takes the upper level."""
    x = np.array([[0.0, 0.5, 1.5, 2.5, 3.0, 1.0]])
    codes, o, sc = O.quantize_groups(x, axis=1)
    assert o[0] == 0.0 and sc[0] == 1.0
    np.testing.assert_array_equal(codes[0], [0, 1, 2, 3, 3, 1])


def test_constant_group_gives_zero_codes():
    x = np.full((1, 16), 0.625)
    codes, o, sc = O.quantize_groups(x, axis=1)
    assert sc[0] == 0 and o[0] == 0.625 and not codes.any()
    # a constant below the fp16 normal range: off rounds down, codes recover within scl/2
    y = np.full((1, 8), O.to_bf16(1.234e-6))
    codes, o, sc = O.quantize_groups(y, axis=1)
    assert o[0] <= y[0, 0] and sc[0] > 0
    assert np.all(np.abs(O.dequantize(codes, o, sc, axis=1) - y) <= sc[0] / 2)


def test_window_quantization_axes():
    rng = np.random.default_rng(5)
    H, W, d = 2, 16, 8
    k = O.to_bf16(rng.standard_normal((H, W, d)))
    v = O.to_bf16(rng.standard_normal((H, W, d)))
    k[1, :, 3] *= 10
    led = O.quantize_window(k, v, start_pos=20)
    assert led.k_off.shape == (H, d) and led.v_off.shape == (H, W)
    # K groups are channels across tokens, V groups tokens across channels
    for h in range(H):
        for c in range(d):
            _, o, s = O.quantize_groups(k[h, :, c][None], axis=1)
            assert o[0] == led.k_off[h, c] and s[0] == led.k_scl[h, c]
        for i in range(W):
            _, o, s = O.quantize_groups(v[h, i][None], axis=1)
            assert o[0] == led.v_off[h, i] and s[0] == led.v_scl[h, i]
    assert np.all(np.abs(led.k_hat() - k) <= led.k_scl[:, None, :] / 2)
    assert np.all(np.abs(led.v_hat() - v) <= led.v_scl[:, :, None] / 2)


def test_pack_codes_bit_layout():
    codes = np.array([[1, 2, 3, 0, 3, 3, 3, 3]], dtype=np.uint8)
    packed = O.pack_codes(codes)
    assert packed.tolist() == [[0b00111001, 0xFF]]


def test_pack_codes_int4_bit_layout():
    codes = np.array([[1, 15, 0, 9]], dtype=np.uint8)
    assert O.pack_codes(codes, 4).tolist() == [[0xF1, 0x90]]


def test_canonical_bytes_int4_sizes():
    rng = np.random.default_rng(3)
    H, W, d = 2, 16, 64
    k = O.to_bf16(rng.standard_normal((H, W, d)))
    v = O.to_bf16(rng.standard_normal((H, W, d)))
    led = O.quantize_window(k, v, 0, bits=4)
    assert led.k_codes.max() > 3 and led.k_codes.max() <= 15
    blob = O.canonical_ledger_bytes(led)
    per_head = 2 * W * d // 2 + 4 * d + 4 * W
    assert len(blob) == H * per_head
    # the first K code byte holds tokens 0's channels 0 and 1, low nibble first
    assert blob[0] == int(led.k_codes[0, 0, 0]) | (int(led.k_codes[0, 0, 1]) << 4)


def test_canonical_bytes_layout_sizes():
    rng = np.random.default_rng(2)
    H, W, d = 3, 16, 64
    k = O.to_bf16(rng.standard_normal((H, W, d)))
    v = O.to_bf16(rng.standard_normal((H, W, d)))
    led = O.quantize_window(k, v, 0)
    blob = O.canonical_ledger_bytes(led)
    per_head = 2 * W * d // 4 + 4 * d + 4 * W
    assert len(blob) == H * per_head
    # head 1's K offsets sit after its two code blocks
    base = per_head + 2 * W * d // 4
    np.testing.assert_array_equal(np.frombuffer(blob[base:base + 2 * d], np.float16), led.k_off[1].astype(np.float16))


def test_range_error_on_huge_values():
    k = np.zeros((1, 4, 4))
    k[0, 0, 0] = 70000.0
    with pytest.raises(O.RangeError):
        O.quantize_window(k, np.zeros((1, 4, 4)), 0)
    with pytest.raises(ValueError):
        O.quantize_groups(np.zeros((1, 4)), axis=1, bits=3)
