"""Pins for the oracle's MXFP4 codec and Smooth-QK calibration (CPU only).

Each test checks the oracle against something other than itself: the
hand-written tables under tests/golden/, an independent threshold
formulation of round-to-nearest-even, closed forms of the two scale rules,
exact round trips, and hand-computed calibration factors.
"""

import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import mx, smooth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def _threshold_code(z):
    """Independent RNE formulation: count the midpoints passed, with the
    inclusive/exclusive side of each midpoint chosen by its even neighbour."""
    z = np.asarray(z, dtype=np.float64)
    return ((z > 0.25).astype(int) + (z >= 0.75) + (z > 1.25) + (z >= 1.75)
            + (z > 2.5) + (z >= 3.5) + (z > 5.0)).astype(np.uint8)


def test_e2m1_code_table_golden():
    for code, val in _table("e2m1_codes.txt"):
        got = mx.e2m1_decode(np.uint8(int(code)))
        assert got == float(val)
        assert np.signbit(got) == (int(code) >= 8)


def test_e2m1_rounding_golden():
    rows = _table("e2m1_rounding.txt")
    z = np.array([float(r[0]) for r in rows])
    want = np.array([int(r[1]) for r in rows], dtype=np.uint8)
    np.testing.assert_array_equal(mx.e2m1_round_magnitude(z), want)


def test_e2m1_rounding_exhaustive_bf16():
    """Every finite bf16 magnitude, at unit scale, against the threshold form."""
    bits = np.arange(0, 0x7F80, dtype=np.uint16)          # +0 .. largest finite
    z = mx.bf16_bits_to_f64(bits)
    np.testing.assert_array_equal(mx.e2m1_round_magnitude(z), _threshold_code(z))


@settings(max_examples=300, deadline=None)
@given(st.lists(st.floats(min_value=0.0, max_value=16.0, allow_nan=False, width=32),
                min_size=1, max_size=64))
def test_e2m1_rounding_property(vals):
    z = np.array(vals, dtype=np.float64)
    np.testing.assert_array_equal(mx.e2m1_round_magnitude(z), _threshold_code(z))


def test_scale_rules_golden():
    for amax, e_ocp, e_uos in _table("scale_rules.txt"):
        a = np.float64(float(amax))
        assert int(mx.e8m0_exponent(a, mx.RULE_OCP)) == int(e_ocp), amax
        assert int(mx.e8m0_exponent(a, mx.RULE_UOS, 7.25)) == int(e_uos), amax


def test_scale_rules_closed_form_all_bf16():
    bits = np.arange(1, 0x7F80, dtype=np.uint16)
    amax = mx.bf16_bits_to_f64(bits)
    e_o = mx.e8m0_exponent(amax, mx.RULE_OCP)
    e_u = mx.e8m0_exponent(amax, mx.RULE_UOS, 7.25)
    # Away from the clamp the ratios lie in the closed-form intervals.
    free = (e_o > -127) & (e_u > -127)
    r_o = amax[free] / np.ldexp(1.0, e_o[free])
    r_u = amax[free] / np.ldexp(1.0, e_u[free])
    assert ((r_o >= 4.0) & (r_o < 8.0)).all()
    assert ((r_u > 3.625) & (r_u <= 7.25)).all()
    # The rules differ exactly where the OCP ratio exceeds 7.25.
    differ = e_o[free] != e_u[free]
    np.testing.assert_array_equal(differ, r_o > 7.25)
    assert (e_u[free][differ] == e_o[free][differ] + 1).all()
    # Inside the clamp region the exponent is the minimum.
    assert (e_o[~free] == -127).all() or (e_u[~free] == -127).all()


@pytest.mark.parametrize("rule", [mx.RULE_OCP, mx.RULE_UOS])
def test_round_trip_representable_blocks(rule):
    """Blocks of grid values times 2^e whose maximum implies e come back bit-exact."""
    rng = np.random.default_rng(7)
    for e in (-127, -100, -3, 0, 5, 120):
        codes = rng.integers(0, 16, size=(50, 32)).astype(np.uint8)
        codes[:, 0] = rng.choice([6, 7, 14, 15], size=50)   # |max| = 4 or 6
        vals = np.ldexp(mx.e2m1_decode(codes), e)
        got_codes, sb = mx.quantize_blocks(vals, rule, 7.25)
        # A zero that came in with either sign keeps that sign.
        np.testing.assert_array_equal(got_codes, codes)
        np.testing.assert_array_equal(sb.astype(int) - 127, e)
        np.testing.assert_array_equal(mx.dequantize_blocks(got_codes, sb), vals)


def test_zero_block_sign_and_saturation():
    y = np.zeros((1, 32))
    y[0, 3] = -0.0
    codes, sb = mx.quantize_blocks(y)
    assert sb[0, 0] == 0
    assert codes[0, 3] == 8 and (np.delete(codes[0], 3) == 0).all()
    # amax = 7.9 with OCP: e = 0, 7.9 and 6.5 saturate to 6, a tiny negative
    # value rounds to -0.
    y = np.zeros((1, 32))
    y[0, 0], y[0, 1], y[0, 2] = 7.9, -6.5, -0.01
    codes, sb = mx.quantize_blocks(y, mx.RULE_OCP)
    assert sb[0, 0] == 127
    assert codes[0, 0] == 7 and codes[0, 1] == 15 and codes[0, 2] == 8
    # The same block under UOS moves to e = 1 and stops clipping.
    codes, sb = mx.quantize_blocks(y, mx.RULE_UOS, 7.25)
    assert sb[0, 0] == 128
    assert mx.e2m1_decode(codes[0, 0]) * 2 == 8.0 and mx.e2m1_decode(codes[0, 1]) * 2 == -6.0


def test_quantize_error_bound_random():
    """|x - x_hat| <= half the local grid gap (times the scale) below 6*2^e."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((200, 128)) * np.exp(rng.uniform(-8, 8, size=(200, 1)))
    codes, sb = mx.quantize(x, axis=1)
    xh = mx.dequantize(codes, sb, axis=1)
    e = np.repeat(sb.astype(np.int64) - 127, 32, axis=1)
    z = np.abs(x) / np.ldexp(1.0, e)
    gap = np.where(z < 2, 0.5, np.where(z < 4, 1.0, 2.0))
    ok = np.abs(x - xh) <= np.ldexp(gap / 2, e) + 0.0
    sat = z > 6
    assert ok[~sat].all()
    assert (np.abs(xh[sat]) == np.ldexp(6.0, e[sat])).all()


def _block_max(a):
    return np.abs(a).reshape(a.shape[0], -1, 32).max(axis=-1)


@pytest.mark.parametrize("rule, frac", [(mx.RULE_OCP, 0.25), (mx.RULE_UOS, 1.0 / 3.625)])
def test_dual_residual_error_bounds(rule, frac):
    """One MXFP4 stage leaves at most frac of its block maximum: under OCP the
    maximum maps into [4, 8), so the rounding gap (at most 1 scale unit below
    6) and the clipping above 6 (under 2 units, only when the maximum passes
    6) are at most a quarter of it; under UOS the maximum maps into
    (3.625, 7.25] and the worst case is a gap of 1 against 3.625.  The second
    stage then leaves at most frac of the residual's maximum, so the pair
    leaves at most frac^2 of the block maximum.  A sign slip in the residual
    (x + dequant) or a dropped second term fails these bounds."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((300, 128)) * np.exp(rng.uniform(-6, 6, size=(300, 1)))
    x[::7, 5] *= 40.0                                    # outlier channels
    x = x.astype(np.float32).astype(np.float64)          # values an fp32 kernel sees
    c1, s1, c2, s2 = mx.quantize_dual(x, axis=1, rule=rule)
    d1 = mx.dequantize(c1, s1, axis=1)
    d2 = mx.dequantize(c2, s2, axis=1)
    a = np.repeat(_block_max(x), 32, axis=1)
    r = x - d1
    ar = np.repeat(_block_max(r), 32, axis=1)
    assert (np.abs(r) <= frac * a * (1 + 1e-12)).all()
    assert (np.abs(x - d1 - d2) <= frac * ar * (1 + 1e-12)).all()
    assert (np.abs(x - d1 - d2) <= frac * frac * a * (1 + 1e-12)).all()
    # The residual is exact in float32: rebuilding it there changes nothing.
    r32 = (x.astype(np.float32) - d1.astype(np.float32)).astype(np.float64)
    np.testing.assert_array_equal(r32, r)


def test_dual_residual_of_representable_blocks_is_zero():
    """A block already on the MXFP4 grid leaves a zero residual: codes 0 and
    scale byte 0 (the all-zero block)."""
    rng = np.random.default_rng(12)
    codes = rng.integers(0, 16, size=(40, 64)).astype(np.uint8)
    codes[:, 0] = 7
    codes[:, 32] = 15
    e = rng.integers(-60, 60, size=(40, 2))
    vals = mx.dequantize(codes, (e + 127).astype(np.uint8), axis=1)
    c1, s1, c2, s2 = mx.quantize_dual(vals, axis=1)
    np.testing.assert_array_equal(mx.dequantize(c1, s1, axis=1), vals)
    assert (s2 == 0).all() and (c2 == 0).all()


def test_dual_residual_cuts_logit_error():
    """The split query's logits against random keys are much closer to the
    exact ones than the single MXFP4 query's (the page reports 60% -> 1% on
    its queries; these synthetic ones only need a large cut)."""
    rng = np.random.default_rng(13)
    q = rng.standard_normal((64, 128))
    q[:, rng.choice(128, 4, replace=False)] *= 20.0      # outlier channels
    k = rng.standard_normal((4096, 128))
    exact = q @ k.T
    c1, s1, c2, s2 = mx.quantize_dual(q, axis=1)
    d1 = mx.dequantize(c1, s1, axis=1)
    d2 = mx.dequantize(c2, s2, axis=1)
    err1 = np.abs(d1 @ k.T - exact).mean() / np.abs(exact).mean()
    err2 = np.abs((d1 + d2) @ k.T - exact).mean() / np.abs(exact).mean()
    assert err2 < err1 / 5          # measured 2.5% against 16.8%
    assert err2 < 0.05


def test_pack_unpack_and_padding():
    rng = np.random.default_rng(1)
    c = rng.integers(0, 16, size=(3, 64)).astype(np.uint8)
    p = mx.pack_nibbles(c)
    assert p.shape == (3, 32)
    assert p[0, 0] == (c[0, 0] | (c[0, 1] << 4))
    np.testing.assert_array_equal(mx.unpack_nibbles(p), c)
    x = rng.standard_normal((5, 40))
    codes, sb = mx.quantize(x, axis=1)
    assert codes.shape == (5, 64) and sb.shape == (5, 2)
    assert (codes[:, 40:] == 0).all()
    np.testing.assert_array_equal(mx.dequantize(codes, sb, axis=1, n=40).shape, (5, 40))


def test_smooth_calibration_hand_case():
    # Two query heads share one KV head; channel maxima chosen by hand.
    q = np.zeros((2, 4, 5))
    k = np.zeros((1, 4, 5))
    q[0, 1, 0], q[1, 2, 0], k[0, 3, 0] = 1.0, -0.5, 16.0     # s = sqrt(16/1) = 4
    q[0, 0, 1], k[0, 0, 1] = 4.0, 1.0                        # s = sqrt(1/4) = 1/2
    q[1, 0, 2], k[0, 0, 2] = 1.0, 2.0 ** 20                  # s = 2^10 -> clamp 2^8
    q[0, 0, 3] = 3.0                                         # kmax = 0 -> s = 1
    k[0, 0, 4] = 2.0                                         # q max 0 -> s = 1
    qs, ks = smooth.calibrate(q, k)
    assert qs.shape == (2, 5) and ks.shape == (1, 5)
    assert qs.dtype == np.float32 and ks.dtype == np.float32
    np.testing.assert_array_equal(qs[0, :4], [4.0, 0.5, 256.0, 1.0])
    np.testing.assert_array_equal(qs[1], qs[0])
    np.testing.assert_array_equal(ks[0, :4], [0.25, 2.0, 1.0 / 256.0, 1.0])
    assert qs[0, 4] == 1.0 and ks[0, 4] == 1.0
    assert qs[0, 0] * ks[0, 0] == 1.0
    # s = sqrt(2) is stored as float32(sqrt 2) and float32(1/sqrt 2).
    q2 = np.ones((1, 1, 1)); k2 = np.full((1, 1, 1), 2.0)
    qs2, ks2 = smooth.calibrate(q2, k2)
    assert qs2[0, 0] == np.float32(np.sqrt(2.0)) and ks2[0, 0] == np.float32(1 / np.sqrt(2.0))


def test_smooth_apply_is_float32_multiply():
    x = np.array([[[[1.0 + 2 ** -7, 3.0]]]], dtype=np.float32)  # [B=1, H=1, S=1, D=2]
    f = np.array([[np.float32(1.0 / 3.0), 2.0]], dtype=np.float32)
    y = smooth.apply(x[0], f)
    assert y.dtype == np.float32
    assert y[0, 0, 0] == np.float32(np.float32(1.0 + 2 ** -7) * np.float32(1.0 / 3.0))
    assert y[0, 0, 1] == 6.0


def test_bf16_bits_decode_hand_values_and_formula():
    """bf16_bits_to_f64 on hand-decoded patterns, then on every finite
    pattern against sign * 2^(E-127) * (1 + M/128) (2^-126 * M/128 for E = 0)."""
    hand = {0x0000: 0.0, 0x3F80: 1.0, 0xBF80: -1.0, 0x4000: 2.0, 0x3FC0: 1.5, 0x4049: 3.140625,
            0x0001: 2.0 ** -133, 0x0080: 2.0 ** -126, 0x7F7F: (2 - 2 ** -7) * 2.0 ** 127, 0xC2F7: -123.5}
    got = mx.bf16_bits_to_f64(np.array(list(hand), dtype=np.uint16))
    np.testing.assert_array_equal(got, np.array(list(hand.values())))
    assert np.signbit(mx.bf16_bits_to_f64(np.uint16(0x8000)))
    bits = np.concatenate([np.arange(0, 0x7F80), np.arange(0x8000, 0xFF80)]).astype(np.uint16)
    b = bits.astype(np.int64)
    sign = np.where(b >> 15, -1.0, 1.0)
    ex, man = (b >> 7) & 0xFF, b & 0x7F
    want = sign * np.where(ex == 0, np.ldexp(man / 128.0, -126), np.ldexp(1.0 + man / 128.0, ex - 127))
    np.testing.assert_array_equal(mx.bf16_bits_to_f64(bits), want)
