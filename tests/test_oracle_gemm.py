"""Pins of the oracle's grouped W4A8 GEMM."""
from fractions import Fraction

import numpy as np
import torch

import oracle


def _torch_dec(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64)


def _problem(rng, E, N, K, counts, gather_from=None):
    q = rng.integers(-8, 8, size=(E, N, K))
    w = oracle.int4_pack(q)
    s = rng.lognormal(-4, 0.5, size=(E, N, K // 128)).astype(np.float32)
    M = int(sum(counts))
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    src = M if gather_from is None else gather_from
    a = rng.integers(0, 256, size=(src, K)).astype(np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x38                 # no NaN codes
    sa = rng.lognormal(-2, 1, size=src).astype(np.float32)
    rows = None if gather_from is None else rng.integers(0, src, size=M).astype(np.int32)
    return q, w, s, offsets, a, sa, rows


def test_exact_rational_brute_force(rng):
    E, N, K = 3, 5, 256
    q, w, s, offsets, a, sa, rows = _problem(rng, E, N, K, [2, 0, 3], gather_from=4)
    out = oracle.grouped_gemm(a, sa, rows, offsets, w, s)
    dec = _torch_dec(a).numpy()
    for e in range(E):
        for p in range(offsets[e], offsets[e + 1]):
            r = rows[p]
            for n in range(N):
                tot = Fraction(0)
                for g in range(K // 128):
                    part = Fraction(0)
                    for kk in range(g * 128, (g + 1) * 128):
                        part += Fraction(float(dec[r, kk])) * int(q[e, n, kk])
                    tot += Fraction(float(s[e, n, g])) * part
                exact = tot * Fraction(float(sa[r]))
                got = Fraction(float(out[p, n]))
                assert abs(got - exact) <= abs(exact) * Fraction(1, 2 ** 23) + Fraction(1, 2 ** 140)


def test_identity_weights_return_activations(rng):
    # q = identity on the first 128 columns, unit scales, unit row scale
    K = N = 256
    q = np.zeros((1, N, K), int)
    q[0, np.arange(N), np.arange(K)] = 1
    w = oracle.int4_pack(q)
    s = np.ones((1, N, K // 128), np.float32)
    a = rng.integers(0, 0x7F, size=(6, K)).astype(np.uint8) | (rng.integers(0, 2, (6, K)) * 0x80).astype(np.uint8)
    sa = np.ones(6, np.float32)
    out = oracle.grouped_gemm(a, sa, None, np.array([0, 6], np.int32), w, s)
    assert np.array_equal(out, _torch_dec(a).numpy().astype(np.float32))


def test_scale_one_integer_sums(rng):
    # activation codes chosen as exact small integers, unit scales: every
    # output is an integer sum computed here with Python integers
    K, N, M = 384, 7, 5
    vals = rng.integers(-16, 17, size=(M, K))
    codes = oracle.e4m3_encode(vals.astype(np.float32))
    q = rng.integers(-8, 8, size=(1, N, K))
    out = oracle.grouped_gemm(codes, np.ones(M, np.float32), None, np.array([0, M], np.int32),
                              oracle.int4_pack(q), np.ones((1, N, K // 128), np.float32))
    want = np.array([[sum(int(vals[m, kk]) * int(q[0, n, kk]) for kk in range(K)) for n in range(N)]
                     for m in range(M)], dtype=np.float64)
    assert np.array_equal(out.astype(np.float64), want)


def test_single_expert_is_dense_matmul(rng):
    # E = 1, every row routed to it: a dense W4A8 GEMM
    N, K, M = 64, 512, 24
    q, w, s, offsets, a, sa, rows = _problem(rng, 1, N, K, [M])
    A = _torch_dec(a) * torch.from_numpy(sa).double()[:, None]
    W = torch.from_numpy(q[0]).double() * torch.from_numpy(np.repeat(s[0], 128, axis=1)).double()
    ref = torch.matmul(A, W.T).float().numpy()
    out = oracle.grouped_gemm(a, sa, None, offsets, w, s)
    assert np.allclose(out, ref, rtol=1e-6, atol=0)


def test_exact_group_variant_agrees(rng):
    q, w, s, offsets, a, sa, rows = _problem(rng, 4, 16, 256, [3, 0, 5, 2], gather_from=7)
    o1 = oracle.grouped_gemm(a, sa, rows, offsets, w, s).astype(np.float64)
    o2 = oracle.grouped_gemm_exact_groups(a, sa, rows, offsets, w, s).astype(np.float64)
    assert np.all(np.abs(o1 - o2) <= np.abs(o1) * 2.0 ** -22)


def test_linear_in_weight_scale(rng):
    q, w, s, offsets, a, sa, rows = _problem(rng, 2, 8, 256, [3, 4])
    o1 = oracle.grouped_gemm(a, sa, None, offsets, w, s)
    s2 = s.copy()
    s2[1, 5, :] *= 2
    o2 = oracle.grouped_gemm(a, sa, None, offsets, w, s2)
    assert np.array_equal(o2[3:, 5], 2 * o1[3:, 5])
    mask = np.ones_like(o1, bool)
    mask[3:, 5] = False
    assert np.array_equal(o1[mask], o2[mask])


def test_rows_follow_expert_ranges(rng):
    # swapping two experts' weights moves results between the row ranges
    q, w, s, offsets, a, sa, rows = _problem(rng, 2, 8, 128, [3, 3])
    o1 = oracle.grouped_gemm(a, sa, None, offsets, w, s)
    o_sw = oracle.grouped_gemm(a, sa, None, offsets, w[::-1].copy(), s[::-1].copy())
    o_e0 = oracle.grouped_gemm(a, sa, None, np.array([0, 6, 6], np.int32), w, s)
    o_e1 = oracle.grouped_gemm(a, sa, None, np.array([0, 0, 6], np.int32), w, s)
    assert np.array_equal(o1[:3], o_e0[:3]) and np.array_equal(o1[3:], o_e1[3:])
    assert np.array_equal(o_sw[:3], o_e1[:3]) and np.array_equal(o_sw[3:], o_e0[3:])


def test_gather_equals_materialized_rows(rng):
    q, w, s, offsets, a, sa, rows = _problem(rng, 3, 16, 256, [2, 4, 1], gather_from=5)
    o1 = oracle.grouped_gemm(a, sa, rows, offsets, w, s)
    o2 = oracle.grouped_gemm(a[rows], sa[rows], None, offsets, w, s)
    assert np.array_equal(o1, o2)
