"""Pins of the oracle's FP8 E4M3FN codec (OCP 8-bit floating point, E4M3).

Checked against things fixed outside the oracle: the format's closed-form
values, torch's own float8_e4m3fn conversion (an independent implementation),
and an exhaustive nearest-value search.
"""
import math

import numpy as np
import pytest
import torch

import oracle

pytestmark = []


def _closed_form_code(v: float) -> int:
    """E4M3 code of an exactly representable normal value, by its fields."""
    s = 0x80 if v < 0 else 0
    a = abs(v)
    e = math.floor(math.log2(a))
    m = a / 2.0 ** e - 1.0
    assert (m * 8) == int(m * 8)
    return s | ((e + 7) << 3) | int(m * 8)


def test_decode_landmarks():
    d = oracle.e4m3_decode
    assert d(0x38) == 1.0
    assert d(0x7E) == 448.0
    assert d(0xFE) == -448.0
    assert d(0x01) == 2.0 ** -9          # smallest subnormal
    assert d(0x08) == 2.0 ** -6          # smallest normal
    assert d(0x07) == 7 * 2.0 ** -9      # largest subnormal
    assert d(0x80) == 0.0 and math.copysign(1, d(0x80)) == -1
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    pos = oracle.e4m3_decode(np.arange(0x7F))
    assert np.all(np.diff(pos) > 0)      # codes 0..0x7E increase
    assert np.array_equal(oracle.e4m3_decode(np.arange(0x80, 0xFF)), -pos)


def test_decode_matches_torch_all_codes():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = oracle.e4m3_decode(np.arange(256))
    same = (ref == ours) | (np.isnan(ref) & np.isnan(ours))
    assert same.all()


def test_encode_roundtrips_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = oracle.e4m3_decode(codes).astype(np.float32)
    back = oracle.e4m3_encode(vals)
    # +0 and -0 keep their own codes
    assert np.array_equal(back, codes)


def test_encode_midpoints_go_to_even_code():
    pos = oracle.e4m3_decode(np.arange(0x7F))
    for c in range(0x7E):
        mid = np.float32((pos[c] + pos[c + 1]) / 2)   # exact in fp32 (few significant bits)
        assert float(mid) == (pos[c] + pos[c + 1]) / 2
        even = c if c % 2 == 0 else c + 1
        assert oracle.e4m3_encode(mid) == even
        assert oracle.e4m3_encode(-mid) == (even | 0x80)
        lo = np.nextafter(mid, np.float32(0))
        hi = np.nextafter(mid, np.float32(np.inf))
        assert oracle.e4m3_encode(lo) == c
        assert oracle.e4m3_encode(hi) == c + 1


@pytest.mark.parametrize("v,code", [
    (0.5 * 2 ** -9, 0x00),    # tie between 0 and the smallest subnormal -> 0
    (1.5 * 2 ** -9, 0x02),    # tie between codes 1 and 2 -> 2
    (2.5 * 2 ** -9, 0x02),    # tie between codes 2 and 3 -> 2
    (3.5 * 2 ** -9, 0x04),    # tie between codes 3 and 4 -> 4
    (0.75 * 2 ** -9, 0x01),
    (-1e-30, 0x80),           # negative underflow keeps the sign
    (-0.0, 0x80),
    (0.0, 0x00),
    (448.0, 0x7E), (460.0, 0x7E), (464.0, 0x7E), (1e30, 0x7E), (-500.0, 0xFE),
    (float("inf"), 0x7E), (float("-inf"), 0xFE),
])
def test_encode_special_values(v, code):
    assert oracle.e4m3_encode(np.float32(v)) == code


def test_encode_matches_torch(rng):
    # torch's cast is RNE and keeps the sign of zero; it turns |v| > 464 into
    # NaN where the method saturates, so compare on |v| <= 464.
    parts = [
        rng.standard_normal(200_000).astype(np.float32) * np.float32(50),
        (rng.standard_normal(100_000) * 2.0 ** -8).astype(np.float32),     # subnormal range
        rng.uniform(-464, 464, 100_000).astype(np.float32),
        np.exp(rng.uniform(-30, 6.1, 100_000)).astype(np.float32) * rng.choice([-1, 1], 100_000),
    ]
    v = np.concatenate(parts).astype(np.float32)
    v = v[np.abs(v) <= 464]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode(v), ref)


def test_encode_brute_force_nearest(rng):
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    fv = oracle.e4m3_decode(finite)
    v = np.concatenate([rng.uniform(-450, 450, 3000),
                        rng.uniform(-0.05, 0.05, 3000)]).astype(np.float32)
    for x in v:
        x64 = float(x)
        if abs(x64) >= 448:
            want = 0x7E | (0x80 if x64 < 0 else 0)
        else:
            dist = np.abs(fv - x64)
            best = finite[dist == dist.min()]
            # candidates: equal-distance codes; prefer the sign of x, then the even mantissa
            best = [c for c in best if (c >= 0x80) == (np.signbit(x))] or list(best)
            even = [c for c in best if (c & 1) == 0]
            want = (even or best)[0]
        assert oracle.e4m3_encode(x) == want, x


def test_int4_values_exact_in_e4m3():
    # every INT4 value -8..7 is an exact E4M3 number: closed-form fields
    for q in range(-8, 8):
        code = int(oracle.e4m3_encode(np.float32(q)))
        if q == 0:
            assert code == 0
        else:
            assert code == _closed_form_code(float(q))
        assert oracle.e4m3_decode(code) == q


def test_low_bytes_are_linear():
    # a byte u in 0..15 read as E4M3 is u * 2^-9 (subnormals, then the first
    # normal binade, share the spacing 2^-9)
    for u in range(16):
        assert oracle.e4m3_decode(u) == u * 2.0 ** -9
