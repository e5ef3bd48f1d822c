"""Pins of the per-channel INT4 x per-token INT8 oracle (no GPU).

Each check compares the oracle with something other than itself: torch's
rounding, exact round trips, closed forms, an fp64 BLAS product of the
dequantized operands, or a brute-force token loop.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle


def _act(rng, M, K):
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, rng.choice(K, max(1, K // 100), replace=False)] *= 20.0
    return x


def test_quant_rows_i8_matches_torch_rounding(rng):
    x = _act(rng, 64, 512)
    codes, scale = oracle.quant_rows_i8(x)
    rowsum = oracle.code_row_sums(codes)
    t = torch.from_numpy(x)
    s = (t.abs().amax(dim=1) / 127.0)                          # fp32, as torch computes it
    ref = torch.clamp(torch.round(t / s[:, None]), -127, 127).to(torch.int8).numpy()
    assert np.array_equal(scale, s.numpy())
    assert np.array_equal(codes, ref)
    assert np.array_equal(rowsum, codes.astype(np.int64).sum(axis=1))


def test_quant_rows_i8_invariants(rng):
    x = _act(rng, 32, 256)
    codes, scale = oracle.quant_rows_i8(x)
    assert np.all(np.abs(codes).max(axis=1) == 127)           # the largest element lands on +-127
    c_neg, s_neg = oracle.quant_rows_i8(-x)
    assert np.array_equal(c_neg, -codes) and np.array_equal(s_neg, scale)
    c_2, s_2 = oracle.quant_rows_i8(x * np.float32(2.0 ** 5))
    assert np.array_equal(c_2, codes) and np.array_equal(s_2, scale * np.float32(2.0 ** 5))
    err = np.abs(x.astype(np.float64) - codes * scale.astype(np.float64)[:, None])
    assert np.all(err <= 0.5 * scale.astype(np.float64)[:, None] * (1 + 1e-6))


def test_quant_rows_i8_zero_row():
    codes, scale = oracle.quant_rows_i8(np.zeros((2, 128), np.float32))
    rowsum = oracle.code_row_sums(codes)
    assert np.all(codes == 0) and np.all(scale == 1.0) and np.all(rowsum == 0)


def test_quantize_int4_channel_round_trip(rng):
    N, K = 16, 256
    q = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    q[:, 0] = 7
    s = (2.0 ** rng.integers(-12, -4, size=N)).astype(np.float32)   # powers of two: s * 7 / 7 is exact
    W = (q * s[:, None]).astype(np.float32)
    q2, s2 = oracle.quantize_int4_channel(W)
    assert np.array_equal(s2, s) and np.array_equal(q2, q)


def test_quantize_int4_channel_closed_form():
    W = np.array([[7.0, -3.5, 2.5, 0.0] * 32], np.float32)          # amax 7 -> scale 1, ties to even
    q, s = oracle.quantize_int4_channel(W)
    assert s[0] == 1.0
    assert list(q[0, :4]) == [7, -4, 2, 0]
    qz, sz = oracle.quantize_int4_channel(np.zeros((1, 128), np.float32))
    assert sz[0] == np.float32(1.0 / 7.0) and np.all(qz == 0)


def _problem(rng, E, N, K, counts, gather):
    T = 11
    R = int(np.sum(counts))
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    x = _act(rng, T if gather else R, K)
    codes, scale = oracle.quant_rows_i8(x)
    rows = rng.integers(0, T, size=R).astype(np.int32) if gather else None
    q = rng.integers(-8, 8, size=(E, N, K)).astype(np.int8)
    words = np.stack([oracle.int4_pack(q[e]) for e in range(E)])
    ws = rng.lognormal(-4, 0.5, size=(E, N)).astype(np.float32)
    return codes, scale, rows, offsets, q, words, ws


def test_grouped_gemm_i8_matches_dequantized_blas(rng):
    codes, scale, rows, offsets, q, words, ws = _problem(rng, 3, 64, 256, [5, 0, 9], gather=True)
    got = oracle.grouped_gemm_i8(codes, scale, rows, offsets, words, ws)
    for e in range(3):
        r0, r1 = offsets[e], offsets[e + 1]
        if r0 == r1:
            continue
        A = codes[rows[r0:r1]].astype(np.float64) * scale[rows[r0:r1]].astype(np.float64)[:, None]
        W = q[e].astype(np.float64) * ws[e].astype(np.float64)[:, None]
        want = A @ W.T
        assert np.allclose(got[r0:r1], want, rtol=2 ** -23, atol=0)


def test_grouped_gemm_i8_integer_sums_are_exact(rng):
    # extreme codes (127 against -8 everywhere) at a long K: each sum is checked
    # against Python integers, so no rounding anywhere can hide
    K = 8192
    codes = np.full((3, K), 127, np.int8)
    codes[1] = -127
    codes[2] = rng.integers(-127, 128, size=K).astype(np.int8)
    q = np.full((1, 2, K), -8, np.int8)
    q[0, 1] = rng.integers(-8, 8, size=K)
    words = np.stack([oracle.int4_pack(q[0])])
    got = oracle.grouped_gemm_i8(codes, np.ones(3, np.float32), None, np.array([0, 3]), words,
                                 np.ones((1, 2), np.float32))
    for r in range(3):
        for n in range(2):
            exact = sum(int(a) * int(b) for a, b in zip(codes[r].tolist(), q[0, n].tolist()))
            assert got[r, n] == np.float32(exact)
    assert got[0, 0] == np.float32(-127 * 8 * K)


def test_grouped_gemm_i8_linear_in_scales_and_dense_case(rng):
    codes, scale, rows, offsets, q, words, ws = _problem(rng, 1, 32, 128, [7], gather=False)
    a = oracle.grouped_gemm_i8(codes, scale, None, offsets, words, ws)
    b = oracle.grouped_gemm_i8(codes, scale, None, offsets, words, ws * np.float32(2.0))
    assert np.array_equal(b, a * np.float32(2.0))
    dense = (codes.astype(np.int64) @ q[0].astype(np.int64).T).astype(np.float64)
    want = (dense * scale.astype(np.float64)[:, None] * ws[0].astype(np.float64)[None, :]).astype(np.float32)
    assert np.array_equal(a, want)


def test_moe_layer_i8_brute_force_tiny(rng):
    T, H, I, E, k = 6, 256, 128, 4, 2
    x = rng.standard_normal((T, H)).astype(np.float32)
    xb = oracle.f32_to_bf16_bits(x)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    q13 = rng.integers(-8, 8, size=(E, 2 * I, H)).astype(np.int8)
    q2 = rng.integers(-8, 8, size=(E, H, I)).astype(np.int8)
    w13 = np.stack([oracle.int4_pack(q13[e]) for e in range(E)])
    w2 = np.stack([oracle.int4_pack(q2[e]) for e in range(E)])
    s13 = rng.lognormal(-4, 0.5, size=(E, 2 * I)).astype(np.float32)
    s2 = rng.lognormal(-4, 0.5, size=(E, H)).astype(np.float32)
    res = oracle.moe_layer_i8(xb, logits, w13, s13, w2, s2, k)
    qx, sx = oracle.quant_act_i8(xb)
    ids, w = oracle.route(logits, k)
    for t in range(T):
        y = np.zeros(H)
        for j in range(k):
            e = ids[t, j]
            h = (qx[t].astype(np.float64) * float(sx[t])) @ (q13[e].astype(np.float64) * s13[e][:, None]).T
            a = oracle.swiglu_f32(h.astype(np.float32)[None, :])
            qa, sa = oracle.quant_rows_i8(a)
            o = (qa[0].astype(np.float64) * float(sa[0])) @ (q2[e].astype(np.float64) * s2[e][:, None]).T
            y += float(w[t, j]) * o.astype(np.float32).astype(np.float64)
        assert np.allclose(res["y"][t], y, rtol=1e-5, atol=1e-6 * np.abs(y).max())
