"""Pins of the oracle's SwiGLU step and routing-weighted combine."""
import math

import numpy as np
from scipy.special import expit

import oracle


def test_silu_closed_form():
    I = 6
    gate = np.array([0.0, 1.0, -1.0, 30.0, -30.0, 2.5], np.float32)
    up = np.array([3.0, 1.0, 1.0, 1.0, 1.0, -2.0], np.float32)
    a = oracle.swiglu_f32(np.concatenate([gate, up])[None, :])[0]
    want = [0.0, 1 / (1 + math.exp(-1)), -1 / (1 + math.e), 30.0, -30 * math.exp(-30) / (1 + math.exp(-30)),
            -2 * 2.5 / (1 + math.exp(-2.5))]
    assert a.shape == (I,)
    assert np.allclose(a, np.array(want, np.float32), rtol=2 ** -23, atol=0)
    assert a[0] == 0.0


def test_silu_matches_scipy(rng):
    h = (rng.standard_normal((16, 256)) * 4).astype(np.float32)
    a = oracle.swiglu_f32(h)
    g, u = h[:, :128].astype(np.float64), h[:, 128:].astype(np.float64)
    ref = (g * expit(g) * u).astype(np.float32)
    assert np.allclose(a, ref, rtol=2 ** -22, atol=1e-30)


def test_swiglu_gate_is_first_half(rng):
    # the gate half goes through silu, the up half is linear
    h = (rng.standard_normal((4, 256))).astype(np.float32)
    h2 = h.copy()
    h2[:, 128:] *= 2
    assert np.array_equal(oracle.swiglu_f32(h2), (oracle.swiglu_f32(h) * 2))


def test_swiglu_quantizes_per_row(rng):
    h = (rng.standard_normal((8, 256)) * 3).astype(np.float32)
    qa, sa = oracle.swiglu(h)
    c2, s2 = oracle.quant_rows(oracle.swiglu_f32(h))
    assert np.array_equal(qa, c2) and np.array_equal(sa, s2)


def test_unpermute_brute_force(rng):
    T, k, H = 9, 3, 40
    o = rng.standard_normal((T * k, H)).astype(np.float32)
    inv = rng.permutation(T * k).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    y = oracle.unpermute(o, inv, w)
    for t in range(T):
        for hh in range(H):
            acc = 0.0
            for j in range(k):
                acc += float(w[t, j]) * float(o[inv[t * k + j], hh])
            assert abs(float(y[t, hh]) - acc) <= abs(acc) * 2 ** -23 + 1e-30


def test_unpermute_one_hot():
    o = np.arange(12, dtype=np.float32).reshape(4, 3)
    inv = np.array([2, 0, 3, 1], np.int32)
    w = np.array([[1.0, 0.0], [0.0, 1.0]], np.float32)
    y = oracle.unpermute(o, inv, w)
    assert np.array_equal(y, np.stack([o[2], o[1]]))
