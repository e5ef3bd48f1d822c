"""Pins of the oracle's top-k softmax routing."""
import itertools

import numpy as np
import pytest
from scipy.special import softmax

import oracle


def test_brute_force_subsets(rng):
    # the chosen set is the k-subset with the largest sum of logits (distinct
    # logits); found here by enumerating every subset
    T, E, k = 40, 7, 3
    logits = rng.standard_normal((T, E)).astype(np.float32)
    ids, w = oracle.route(logits, k)
    for t in range(T):
        best = max(itertools.combinations(range(E), k), key=lambda s: sum(float(logits[t, i]) for i in s))
        assert set(ids[t]) == set(best)
        vals = logits[t, ids[t]]
        assert np.all(np.diff(vals) < 0)          # descending


def test_python_sort_order(rng):
    T, E, k = 50, 64, 8
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[:, 10] = logits[:, 3]                  # forced ties
    ids, _ = oracle.route(logits, k)
    for t in range(T):
        want = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))[:k]
        assert list(ids[t]) == want


def test_all_equal_logits():
    ids, w = oracle.route(np.zeros((3, 16), np.float32), 4)
    assert np.array_equal(ids, np.tile(np.arange(4), (3, 1)))
    assert np.allclose(w, 0.25, rtol=0, atol=0)


def test_k_equals_E_is_softmax(rng):
    logits = rng.standard_normal((20, 12)).astype(np.float32) * 3
    ids, w = oracle.route(logits, 12, renormalize=True)
    p = softmax(logits.astype(np.float64), axis=1)
    for t in range(20):
        assert np.allclose(w[t], p[t, ids[t]], rtol=1e-6, atol=0)
    assert np.allclose(w.sum(1), 1.0, atol=1e-6)


def test_no_renormalize_is_softmax_entries(rng):
    logits = rng.standard_normal((20, 32)).astype(np.float32)
    ids, w = oracle.route(logits, 4, renormalize=False)
    p = softmax(logits.astype(np.float64), axis=1)
    assert np.allclose(w, np.take_along_axis(p, ids.astype(int), 1), rtol=1e-6, atol=0)


def test_renormalized_sum_and_shift_invariance(rng):
    logits = rng.standard_normal((30, 256)).astype(np.float32)
    ids, w = oracle.route(logits, 8)
    assert np.allclose(w.sum(1), 1.0, atol=1e-6)
    ids2, w2 = oracle.route(logits + np.float32(4.0), 8)
    assert np.array_equal(ids, ids2)
    assert np.allclose(w, w2, rtol=1e-5)


def test_signed_zero_is_a_tie():
    logits = np.array([[-0.0, 0.0, -1.0]], np.float32)
    ids, _ = oracle.route(logits, 2)
    assert list(ids[0]) == [0, 1]


def test_bad_k():
    with pytest.raises(ValueError):
        oracle.route(np.zeros((2, 4), np.float32), 5)
