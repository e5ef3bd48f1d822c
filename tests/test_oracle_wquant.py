"""Pins of the oracle's INT4 group-128 weight quantizer on hand-computed groups.

The quantizer follows the "GLM-5.3-W4A8" card, section 量化方式: symmetric
INT4 with one scale per 128 weights, the scale of each group picked by the
smallest squared error over 11 shrink ratios 1.00, 0.97, ..., 0.70.  The
pages' error figures (0.103 / 0.124) only bound the quantizer's average
behaviour; the groups below fix its three discrete rules, each with a
literal expected result worked out by hand in the comments:
  * the quotient w / s is rounded half to even (not half away from zero);
  * codes are clamped to [-8, 7] (uint4b8 stores q + 8 in 0..15, so -8 is
    a legal code and a quotient of -10 becomes -8);
  * when ratios tie on the squared error, the larger ratio is kept.
A quantizer that broke any one rule fails at least one test.
"""
import numpy as np

import oracle


def _group(values):
    g = np.zeros(128, np.float32)
    g[:len(values)] = np.asarray(values, np.float32)
    return g


def test_half_integer_quotients_round_half_to_even():
    # amax = 7, so the round-to-nearest scale is 7 / 7 = 1 exactly and the
    # quotients are the values themselves: 0.5, 1.5, 2.5, ... are exact ties
    half = [0.5, 1.5, 2.5, 3.5, 4.5, 5.5, 6.5, -0.5, -1.5, -2.5, -3.5, -4.5, -5.5, -6.5]
    W = _group([7.0] + half)[None, :]
    q, s = oracle.quantize_int4_g128(W, mse_clip=False)
    assert s[0, 0] == np.float32(1.0)
    # half to even: 0.5 -> 0, 1.5 -> 2, 2.5 -> 2, 3.5 -> 4, 4.5 -> 4, 5.5 -> 6, 6.5 -> 6
    # (half away from zero would give 1 2 3 4 5 6 7)
    want = [7, 0, 2, 2, 4, 4, 6, 6, 0, -2, -2, -4, -4, -6, -6]
    assert q[0, :15].tolist() == want
    assert not q[0, 15:].any()


def test_half_integer_quotients_with_the_clip_search():
    # 120 integers -7..7 (eight of each) and eight half-integers, amax 7.
    # Ratio 1.00: scale 1, the integers are exact, each half-integer is off by
    # 0.5: SSE = 8 * 0.25 = 2.0.  Ratio 0.97 (scale 0.97): the integers already
    # cost 8 * 2 * (0.21^2 + 0.18^2 + 0.15^2 + 0.12^2 + 0.09^2 + 0.06^2 + 0.03^2)
    # = 2.016 before the half-integers, SSE 3.47 in all; every smaller ratio
    # is worse still (9.1 .. 65).  So the scale is 1 and the half-integers
    # round half to even.
    ints = np.tile(np.arange(-7, 8, dtype=np.float32), 8)
    half = np.float32([0.5, 1.5, 2.5, 3.5, -0.5, -1.5, -2.5, -3.5])
    W = np.concatenate([ints, half])[None, :]
    q, s = oracle.quantize_int4_g128(W, mse_clip=True)
    assert s[0, 0] == np.float32(1.0)
    assert np.array_equal(q[0, :120], ints.astype(np.int8))
    assert q[0, 120:].tolist() == [0, 2, 2, 4, 0, -2, -2, -4]


def test_clamp_at_minus_eight_decides_the_ratio():
    # w = [-8, 0.8 * (-7, -6, ..., 7, -7, ...)]: amax 8, scale r * 8 / 7.
    # Ratio 0.70: scale 0.8, every multiple of 0.8 is exact (q = -7..7) and
    # -8 / 0.8 = -10 is clamped to -8, reconstructed as -6.4: SSE = 1.6^2 = 2.56.
    # Ratio 0.73 (scale 0.8343): -8 -> -9.59 -> clamp -8 -> -6.67 (1.76) plus
    # the multiples of 0.8, which are no longer exact: SSE 4.56.  Ratios 0.76
    # .. 1.00: 8.6 .. 14.  So ratio 0.70 wins, with the -8 code.
    # Clamping to [-7, 7] instead would keep ratio 0.70 but give q = -7.
    mult = np.resize(np.arange(-7, 8, dtype=np.float32), 127)
    W = np.concatenate([np.float32([-8.0]), mult * np.float32(0.8)])[None, :]
    q, s = oracle.quantize_int4_g128(W, mse_clip=True)
    assert s[0, 0] == np.float32(0.8)
    assert q[0, 0] == -8
    assert np.array_equal(q[0, 1:], mult.astype(np.int8))
    words = oracle.int4_pack(q)
    assert (int(words[0, 0]) & 0xF) == 0          # uint4b8 nibble of -8 is 0


def test_ratio_ties_keep_the_larger_ratio():
    # An all-zero group counts as amax 1; every ratio then gives q = 0 and a
    # squared error of exactly 0, an 11-way tie.  Keeping the larger ratio
    # gives the scale 1.00 * 1 / 7; keeping the smaller would give 0.70 / 7.
    W = np.zeros((1, 256), np.float32)
    W[0, 128:] = np.tile(np.arange(-7, 8, dtype=np.float32), 9)[:128]   # a second, exact group
    q, s = oracle.quantize_int4_g128(W, mse_clip=True)
    assert s[0, 0] == np.float32(1.0 / 7.0)
    assert s[0, 0] != np.float32(0.7 / 7.0)
    assert not q[0, :128].any()
    # the exact group: ratio 1.00 reconstructs it with error 0; no other ratio does
    assert s[0, 1] == np.float32(1.0)
    assert np.array_equal(q[0, 128:], W[0, 128:].astype(np.int8))


def test_round_to_nearest_scale_is_amax_over_seven():
    # without the clip search the scale is fl32(amax / 7); 3.5 / 7 = 0.5 exactly
    W = _group([3.5, -1.75, 0.25, 0.75, 1.25])[None, :]
    q, s = oracle.quantize_int4_g128(W, mse_clip=False)
    assert s[0, 0] == np.float32(0.5)
    # quotients 7, -3.5, 0.5, 1.5, 2.5 -> 7, -4, 0, 2, 2 (half to even)
    assert q[0, :5].tolist() == [7, -4, 0, 2, 2]
