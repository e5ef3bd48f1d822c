"""Pins of the oracle's INT4 uint4b8 packing (8 nibbles per int32, along K)."""
import numpy as np
import pytest

import oracle


def test_known_words():
    # q = -8..-1 stores nibbles 0..7; q = 0..7 stores nibbles 8..15
    assert oracle.int4_pack(np.arange(-8, 0)).view(np.uint32)[0] == 0x76543210
    assert oracle.int4_pack(np.arange(0, 8)).view(np.uint32)[0] == 0xFEDCBA98
    assert oracle.int4_pack(np.full(8, -8)).view(np.uint32)[0] == 0x00000000
    assert oracle.int4_pack(np.zeros(8, int)).view(np.uint32)[0] == 0x88888888
    assert oracle.int4_pack(np.full(8, 7)).view(np.uint32)[0] == 0xFFFFFFFF
    # first element of the row goes to the lowest nibble
    q = np.array([7, -8, -8, -8, -8, -8, -8, -8])
    assert oracle.int4_pack(q).view(np.uint32)[0] == 0x0000000F


def test_roundtrip_q(rng):
    q = rng.integers(-8, 8, size=(5, 3, 256))
    w = oracle.int4_pack(q)
    assert w.shape == (5, 3, 32) and w.dtype == np.int32
    assert np.array_equal(oracle.int4_unpack(w), q)


def test_roundtrip_words(rng):
    w = rng.integers(0, 2**32, size=(4, 96), dtype=np.uint32).view(np.int32)
    assert np.array_equal(oracle.int4_pack(oracle.int4_unpack(w)), w)


def test_uniform_words_give_uniform_int4(rng):
    w = rng.integers(0, 2**32, size=(256, 512), dtype=np.uint32).view(np.int32)
    q = oracle.int4_unpack(w)
    counts = np.bincount((q.reshape(-1) + 8), minlength=16)
    assert q.min() == -8 and q.max() == 7
    expected = q.size / 16
    assert np.all(np.abs(counts - expected) < 6 * np.sqrt(expected))


def test_dequant_is_exact_product(rng):
    q = rng.integers(-8, 8, size=(4, 256))
    s = rng.lognormal(-4, 0.5, size=(4, 2)).astype(np.float32)
    W = oracle.dequant_weights(oracle.int4_pack(q), s)
    for n in range(4):
        for kk in (0, 127, 128, 255):
            assert W[n, kk] == q[n, kk] * float(s[n, kk // 128])


def test_rejects_out_of_range():
    with pytest.raises(ValueError):
        oracle.int4_pack(np.array([8, 0, 0, 0, 0, 0, 0, 0]))
    with pytest.raises(ValueError):
        oracle.int4_pack(np.zeros(7, int))
