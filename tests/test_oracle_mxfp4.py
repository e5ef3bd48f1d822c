"""Pins of the MXFP4 group-32 oracle against the format's definition, brute force and the pages' figure.

The format is the OCP microscaling one: E2M1 elements (value fixed by the
sign, 2 exponent bits with bias 1 and 1 mantissa bit) sharing one E8M0 scale
per 32 elements.  The error figure is the "GLM-5.3-W4A8" card's (section
量化方式).
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import mxfp4_oracle as mx

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")))


def e2m1_from_bits(c: int) -> float:
    """Value of a 4-bit E2M1 code from its fields: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0."""
    s, e, m = (c >> 3) & 1, (c >> 1) & 3, c & 1
    mag = m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)
    return -mag if s else mag


def test_e2m1_decode_matches_field_definition():
    got = mx.e2m1_decode(np.arange(16))
    want = np.array([e2m1_from_bits(c) for c in range(16)])
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.arange(16) >= 8)        # code 8 is -0
    assert got.max() == 6.0 and got.min() == -6.0


def test_e2m1_encode_round_trip_all_codes():
    assert np.array_equal(mx.e2m1_encode(mx.e2m1_decode(np.arange(16))), np.arange(16))


@pytest.mark.parametrize("v,code", [
    (0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6),   # ties go to the even code
    (0.2499, 0), (0.2501, 1), (4.9, 6), (5.1, 7), (6.0, 7), (7.9, 7), (1e9, 7),  # nearest, then saturation
    (-0.25, 8), (-5.0, 14), (-100.0, 15), (-1e-30, 8),
])
def test_e2m1_encode_ties_and_saturation(v, code):
    assert int(mx.e2m1_encode(v)) == code


def test_e2m1_encode_is_nearest_by_brute_force():
    v = np.linspace(-7.0, 7.0, 14001)
    codes = mx.e2m1_encode(v)
    table = np.array([e2m1_from_bits(c) for c in range(16)])
    err = np.abs(np.clip(v, -6, 6)[:, None] - table[None, :])
    best = err.min(axis=1)
    assert np.array_equal(np.abs(np.clip(v, -6, 6) - table[codes]), best)


def test_e8m0_decode_matches_torch():
    b = torch.arange(0, 255, dtype=torch.uint8)          # 255 is NaN in E8M0
    want = b.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    vals = np.zeros((255, 2), dtype=np.uint8)
    vals[:, 0] = 2                                        # code 2 = 1.0, code 0 = 0
    got = mx.dequant_mxfp4(np.repeat(mx.fp4_pack(vals), 16, axis=1), b.numpy()[:, None])
    assert np.array_equal(got[:, 0], want)


@pytest.mark.parametrize("amax,X", [(6.0, 0), (4.0, 0), (7.99, 0), (8.0, 1), (3.99, -1), (0.0, -2),
                                    (1.0, -2), (2.0 ** -130, -127), (2.0 ** 140, 127)])
def test_block_exponent_rule(amax, X):
    assert int(mx.mx_block_exponent(amax)) == X


def test_block_scale_puts_amax_in_top_binade():
    rng = np.random.Generator(np.random.PCG64(1))
    W = (rng.standard_normal((64, 256)) * np.exp2(rng.integers(-20, 20, (64, 1)))).astype(np.float32)
    codes, scales = mx.quantize_mxfp4(W)
    B = np.abs(W.astype(np.float64)).reshape(64, 8, 32).max(axis=2)
    r = B / np.exp2(scales.astype(np.float64) - 127)
    assert ((r >= 4) & (r < 8)).all()


def test_exactly_representable_blocks_are_recovered():
    rng = np.random.Generator(np.random.PCG64(2))
    codes = rng.integers(0, 16, (16, 128)).astype(np.uint8)
    codes[:, ::32] = 7                                    # every block holds a 6 so the rule picks X = x0
    x0 = rng.integers(-30, 30, (16, 4))
    W = mx.e2m1_decode(codes) * np.repeat(np.exp2(x0), 32, axis=1)
    q, s = mx.quantize_mxfp4(W.astype(np.float32))
    assert np.array_equal(s, (x0 + 127).astype(np.uint8))
    assert np.array_equal(mx.e2m1_decode(q), mx.e2m1_decode(codes))   # +0 and -0 may swap only where equal
    assert np.array_equal(mx.dequant_mxfp4(mx.fp4_pack(q), s), W)


def test_zero_block():
    q, s = mx.quantize_mxfp4(np.zeros((2, 64), dtype=np.float32))
    assert (s == 125).all() and (mx.e2m1_decode(q) == 0).all()     # amax 0 counts as 1: X = -2


def test_element_error_bound():
    # inside the block's range each element is off by at most half a step of its binade
    rng = np.random.Generator(np.random.PCG64(3))
    W = rng.standard_normal((32, 512)).astype(np.float32)
    q, s = mx.quantize_mxfp4(W)
    scale = np.repeat(np.exp2(s.astype(np.float64) - 127), 32, axis=1)
    x = W.astype(np.float64) / scale
    err = np.abs(x - mx.e2m1_decode(q))
    step = np.where(np.abs(x) < 2, 0.5, np.where(np.abs(x) < 4, 1.0, 2.0))
    assert (err <= step / 2 + np.maximum(np.abs(x) - 6, 0)).all()


def test_pack_layout():
    assert np.array_equal(mx.fp4_pack(np.array([1, 2, 15, 0])), np.array([0x21, 0x0F], dtype=np.uint8))
    rng = np.random.Generator(np.random.PCG64(4))
    c = rng.integers(0, 16, (3, 5, 64)).astype(np.uint8)
    assert np.array_equal(mx.fp4_unpack(mx.fp4_pack(c)), c)


def test_reconstruction_error_envelope():
    # the card: 0.113 relative L2 for MXFP4 group 32 (INT4 group 128: 0.103 / 0.124)
    rng = np.random.Generator(np.random.PCG64(0))
    W = rng.standard_normal((512, 4096)).astype(np.float32)
    q, s = mx.quantize_mxfp4(W)
    e = oracle.relative_l2(W, mx.dequant_mxfp4(mx.fp4_pack(q), s))
    assert abs(e - GOLDEN["mxfp4_g32_rel_l2"]["value"]) < 0.004


def _brute_gemm(a_codes, a_scale, a_rows, offsets, w_packed, w_scale):
    """Pure-Python loops over tiny inputs, decoding each element from its bit fields."""
    e4m3 = oracle.e4m3_decode(np.arange(256))
    M, N, K = int(offsets[-1]), w_packed.shape[1], 2 * w_packed.shape[2]
    out = np.zeros((M, N))
    for e in range(len(offsets) - 1):
        for p in range(offsets[e], offsets[e + 1]):
            r = a_rows[p] if a_rows is not None else p
            for n in range(N):
                acc = 0.0
                for k in range(K):
                    byte = int(w_packed[e, n, k // 2])
                    c = byte & 15 if k % 2 == 0 else byte >> 4
                    w = e2m1_from_bits(c) * 2.0 ** (int(w_scale[e, n, k // 32]) - 127)
                    acc += float(e4m3[a_codes[r, k]]) * w
                out[p, n] = acc * float(a_scale[r])
    return out.astype(np.float32)


def test_grouped_gemm_brute_force():
    rng = np.random.Generator(np.random.PCG64(5))
    E, N, K, T = 3, 5, 64, 6
    a_codes = rng.integers(0, 256, (T, K)).astype(np.uint8)
    a_codes[(a_codes & 0x7F) == 0x7F] = 0                  # E4M3 NaN codes are never produced
    a_scale = rng.uniform(0.01, 1, T).astype(np.float32)
    offsets = np.array([0, 3, 3, 7])                       # an empty expert in the middle
    a_rows = np.array([0, 5, 2, 1, 1, 4, 3])
    w = rng.integers(0, 256, (E, N, K // 2)).astype(np.uint8)
    s = rng.integers(117, 137, (E, N, K // 32)).astype(np.uint8)
    got = mx.grouped_gemm_mxfp4(a_codes, a_scale, a_rows, offsets, w, s)
    want = _brute_gemm(a_codes, a_scale, a_rows, offsets, w, s)
    np.testing.assert_allclose(got, want, rtol=1e-6, atol=1e-30)


def test_layer_equals_int4_layer_on_shared_grid():
    # weights drawn from {0, +-1, +-2, +-3, +-4, +-6}: exact both as INT4 (scale 1) and as MXFP4 (scale 2^0),
    # so the two layers must agree (up to fp64 summation order)
    rng = np.random.Generator(np.random.PCG64(6))
    E, H, I, T, k = 4, 256, 128, 9, 2
    grid = np.array([0, 1, 2, 3, 4, 6, -1, -2, -3, -4, -6])

    def make(N, K):
        Wv = grid[rng.integers(0, grid.size, (E, N, K))].astype(np.float64)
        codes = mx.e2m1_encode(Wv)
        packed_fp4 = mx.fp4_pack(codes)
        s_fp4 = np.full((E, N, K // 32), 127, dtype=np.uint8)
        words = oracle.int4_pack(Wv.astype(np.int64))               # signed values; the packer adds the bias
        s_i4 = np.ones((E, N, K // 128), dtype=np.float32)
        assert np.array_equal(mx.dequant_mxfp4(packed_fp4, s_fp4), oracle.dequant_weights(words, s_i4))
        return packed_fp4, s_fp4, words, s_i4

    w13, s13, w13i, s13i = make(2 * I, H)
    w2, s2, w2i, s2i = make(H, I)
    x = oracle.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    a = mx.moe_layer_mxfp4(x, logits, w13, s13, w2, s2, k)
    b = oracle.moe_layer(x, logits, w13i, s13i, w2i, s2i, k)
    np.testing.assert_allclose(a["h"], b["h"], rtol=1e-6)
    np.testing.assert_allclose(a["y"], b["y"], rtol=1e-5, atol=1e-6)


def test_grid_is_exhaustive_over_sign_and_magnitude():
    # every (sign, magnitude) pair appears once in the 16 codes
    vals = mx.e2m1_decode(np.arange(16))
    pairs = {(bool(np.signbit(v)), abs(v)) for v in vals}
    assert len(pairs) == 16 and set(itertools.chain([0.0], mx.E2M1_MAGNITUDES)) == {abs(v) for v in vals}
