"""Pins of the oracle's per-token dynamic FP8 quantization (amax / 448)."""
import numpy as np
import torch

import oracle


def _x(rng, M=64, K=512):
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[3, 17] = 300.0       # an outlier
    x[5] *= 1e-3           # a small row
    return x


def test_matches_torch_division_and_cast(rng):
    x = _x(rng)
    codes, scale = oracle.quant_rows(x)
    xt = torch.from_numpy(x)
    amax = xt.abs().amax(dim=1)
    sc = amax / 448.0
    assert np.array_equal(sc.numpy(), scale)
    ref = (xt / sc[:, None]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ref, codes)


def test_every_row_reaches_full_scale(rng):
    x = _x(rng)
    codes, scale = oracle.quant_rows(x)
    mag = codes & 0x7F
    assert np.all(mag.max(axis=1) == 0x7E)


def test_sign_symmetry(rng):
    x = _x(rng)
    c1, s1 = oracle.quant_rows(x)
    c2, s2 = oracle.quant_rows(-x)
    assert np.array_equal(s1, s2)
    assert np.array_equal(c2, c1 ^ 0x80)


def test_power_of_two_scaling(rng):
    x = _x(rng)
    c1, s1 = oracle.quant_rows(x)
    for m in (-7, 3, 20):
        f = np.float32(2.0 ** m)
        c2, s2 = oracle.quant_rows(x * f)
        assert np.array_equal(c1, c2)
        assert np.array_equal(s2, s1 * f)


def test_error_bound(rng):
    x = _x(rng)
    codes, scale = oracle.quant_rows(x)
    q = x.astype(np.float64) / scale.astype(np.float64)[:, None]
    d = oracle.e4m3_decode(codes)
    a = np.abs(d)
    # half a unit in the last place of E4M3 at the decoded magnitude
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    half_ulp = 2.0 ** (e - 4)
    # the fp32 quotient adds at most 2^-24 relative before the FP8 rounding
    assert np.all(np.abs(q - d) <= half_ulp * (1 + 2.0 ** -20) + np.abs(q) * 2.0 ** -23)


def test_zero_row_scale_one():
    x = np.zeros((2, 128), np.float32)
    x[1, :] = -0.0
    codes, scale = oracle.quant_rows(x)
    assert np.array_equal(scale, [1.0, 1.0])
    assert np.all(codes[0] == 0x00) and np.all(codes[1] == 0x80)


def test_bf16_widening_matches_torch(rng):
    x = rng.standard_normal(10_000).astype(np.float32) * 30
    t = torch.from_numpy(x).to(torch.bfloat16)
    bits = t.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_bits_to_f32(bits), t.to(torch.float32).numpy())


def test_bf16_rounding_matches_torch(rng):
    y = (rng.standard_normal(10_000) * 1e3).astype(np.float32)
    ref = torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f32_to_bf16_bits(y), ref)


def test_quant_act_path(rng):
    x = (rng.standard_normal((8, 256)) * 5).astype(np.float32)
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    c1, s1 = oracle.quant_act(bits)
    c2, s2 = oracle.quant_rows(torch.from_numpy(x).to(torch.bfloat16).float().numpy())
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
