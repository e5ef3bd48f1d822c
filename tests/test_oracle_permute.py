"""Pins of the oracle's expert permutation (stable counting sort)."""
import numpy as np

import oracle


def _brute(ids, E):
    T, k = ids.shape
    rows = []
    for e in range(E):                    # experts in order
        for f in range(T * k):            # routed index order inside an expert
            if ids.reshape(-1)[f] == e:
                rows.append(f)
    offsets = [0]
    for e in range(E):
        offsets.append(offsets[-1] + int((ids == e).sum()))
    row_token = [f // k for f in rows]
    inv_pos = [0] * (T * k)
    for p, f in enumerate(rows):
        inv_pos[f] = p
    return np.array(offsets), np.array(row_token), np.array(inv_pos)


def test_against_brute_force(rng):
    for T, E, k in [(16, 8, 2), (33, 5, 3), (7, 64, 8), (1, 4, 4)]:
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        got = oracle.permute(ids, E)
        want = _brute(ids, E)
        for g, w in zip(got, want):
            assert np.array_equal(g, w)


def test_repeated_ids_are_stable(rng):
    # ids need not be distinct per token for the permutation to be defined
    ids = rng.integers(0, 3, size=(20, 4)).astype(np.int32)
    got = oracle.permute(ids, 3)
    want = _brute(ids, 3)
    for g, w in zip(got, want):
        assert np.array_equal(g, w)


def test_invariants(rng):
    T, E, k = 300, 256, 8
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    offsets, row_token, inv_pos = oracle.permute(ids, E)
    R = T * k
    assert offsets[0] == 0 and offsets[-1] == R
    assert np.all(np.diff(offsets) >= 0)
    assert np.array_equal(np.sort(inv_pos), np.arange(R))        # a permutation
    flat = ids.reshape(-1)
    for f in range(R):
        p = inv_pos[f]
        e = flat[f]
        assert offsets[e] <= p < offsets[e + 1]
        assert row_token[p] == f // k
    empty = np.setdiff1d(np.arange(E), flat)
    for e in empty:
        assert offsets[e] == offsets[e + 1]
