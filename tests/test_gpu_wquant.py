"""GPU parity of the INT4 group-128 weight quantizer (RTN and the 11-ratio MSE clip search).

Both sides decide the codes from the exact quotient w / s and the clip ratio
from fp64 sums of squared errors, so scales and packed words are compared
bit for bit.  The only allowed difference is a ratio choice between two
candidates whose squared errors agree to 1e-12 (the two sides add the 128
terms in different orders); the tests count such groups and expect none on
these inputs.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_util import host, say, to_dev
from quantized_grouped_gemm_token_amd import ops

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert ops.w4a8_moe_device_supported(), "the current device is not a gfx950"
    yield
    torch.cuda.synchronize()


def _group_sse(W, s):
    """Squared reconstruction error of each group [N, G] for the scales s [N, G]."""
    N, K = W.shape
    Wg = np.asarray(W, np.float64).reshape(N, K // 128, 128)
    s64 = np.asarray(s, np.float32).astype(np.float64)[..., None]
    q = np.clip(np.rint(Wg / s64), -8, 7)
    return ((Wg - q * s64) ** 2).sum(axis=2)


def _check(W, mse_clip=True):
    W = np.ascontiguousarray(W, np.float32)
    N, K = W.shape
    say(f"quantize_weights N={N} K={K} mse_clip={mse_clip}")
    words, scales = ops.w4a8_moe_quantize_weights(to_dev(W), mse_clip=mse_clip)
    words, scales = host(words), host(scales)
    q_ref, s_ref = oracle.quantize_int4_g128(W, mse_clip=mse_clip)
    words_ref = oracle.int4_pack(q_ref)
    differ = scales.view(np.uint32) != s_ref.view(np.uint32)
    if differ.any():
        # a different ratio is acceptable only as a tie of the two squared errors
        e_gpu = _group_sse(W, scales)
        e_ref = _group_sse(W, s_ref)
        rel = np.abs(e_gpu - e_ref)[differ] / np.maximum(e_ref[differ], 1e-300)
        assert rel.max() <= 1e-12, f"{differ.sum()} groups chose a worse ratio (rel {rel.max():.3e})"
    same = ~np.repeat(differ, 16, axis=1)
    assert np.array_equal(words[same], words_ref[same]), "packed words differ where the scales agree"
    return int(differ.sum()), words, scales


@pytest.mark.parametrize("N,K", [(8, 128), (96, 640), (256, 2048)])
@pytest.mark.parametrize("mse_clip", [True, False])
def test_quantize_gaussian(N, K, mse_clip, rng):
    W = rng.standard_normal((N, K)).astype(np.float32) * np.float32(0.02)
    n_tie, _, _ = _check(W, mse_clip)
    assert n_tie == 0


def test_quantize_special_groups(rng):
    K = 128 * 6
    W = rng.standard_normal((4, K)).astype(np.float32)
    W[0, 0:128] = 0.0                                         # all zero: scale 1/7, codes 8
    W[0, 128:256] = 3.0                                       # constant
    W[0, 256:384] = 0.0
    W[0, 300] = -5.0                                          # one spike
    W[1, 0:128] = np.float32(1e-30) * rng.standard_normal(128).astype(np.float32)  # tiny values
    W[1, 128:256] = np.float32(1e30) * rng.standard_normal(128).astype(np.float32)  # huge values
    # exact half-integer quotients at r = 1 (amax 7 -> scale 1): ties to even
    W[2, 0:128] = np.resize(np.arange(-14, 15, dtype=np.float32) * np.float32(0.5), 128)
    W[2, 0] = np.float32(7.0)
    W[3, :] = np.repeat(np.float32([1, -1, 2, -2, 0.5, -0.5]), 128)
    _, words, scales = _check(W)
    assert scales[0, 0] == np.float32(1.0 / 7.0)
    assert np.all(oracle.int4_unpack(words[0, :16]) == 0)


def test_quantize_expert_shape_and_error_envelope():
    """A [E, N, K] expert stack as the layer stores it, and the reconstruction
    error against the pages' group-128 figures (about 0.10 with the clip search)."""
    g = np.random.Generator(np.random.PCG64(2024))
    W = (g.standard_normal((2, 512, 2048)) * 0.02).astype(np.float32)
    say("quantize_weights E=2 N=512 K=2048")
    words, scales = ops.w4a8_moe_quantize_weights(to_dev(W))
    assert tuple(words.shape) == (2, 512, 256) and tuple(scales.shape) == (2, 512, 16)
    words, scales = host(words), host(scales)
    for e in range(2):
        q_ref, s_ref = oracle.quantize_int4_g128(W[e])
        assert np.array_equal(scales[e].view(np.uint32), s_ref.view(np.uint32))
        assert np.array_equal(words[e], oracle.int4_pack(q_ref))
    err = oracle.relative_l2(W.reshape(-1, 2048), oracle.dequant_weights(words.reshape(-1, 256),
                                                                          scales.reshape(-1, 16)))
    assert 0.09 <= err <= 0.11, err


def test_quantize_empty():
    w = torch.empty((0, 256), dtype=torch.float32, device="cuda:0")
    words, scales = ops.w4a8_moe_quantize_weights(w)
    assert words.shape == (0, 32) and scales.shape == (0, 2)


def test_quantize_hand_computed_groups():
    """The groups whose results are worked out by hand in test_oracle_wquant.py
    (ties to even, the -8 clamp deciding the ratio, ties keeping the larger
    ratio), checked on the GPU against the literal results."""
    ints = np.tile(np.arange(-7, 8, dtype=np.float32), 8)
    half = np.float32([0.5, 1.5, 2.5, 3.5, -0.5, -1.5, -2.5, -3.5])
    mult = np.resize(np.arange(-7, 8, dtype=np.float32), 127)
    W = np.zeros((2, 256), np.float32)
    W[0, :128] = np.concatenate([ints, half])                           # ratio 1.00, half to even
    W[0, 128:] = np.concatenate([np.float32([-8.0]), mult * np.float32(0.8)])   # ratio 0.70, -10 -> -8
    W[1, 128:] = np.tile(np.arange(-7, 8, dtype=np.float32), 9)[:128]   # exact at ratio 1.00
    # W[1, :128] stays zero: an 11-way tie, kept at ratio 1.00
    say("quantize_weights hand-computed groups")
    words, scales = ops.w4a8_moe_quantize_weights(to_dev(W), mse_clip=True)
    words, scales = host(words), host(scales)
    assert scales.tolist() == [[np.float32(1.0), np.float32(0.8)], [np.float32(1.0 / 7.0), np.float32(1.0)]]
    q = oracle.int4_unpack(words)
    assert np.array_equal(q[0, :120], ints.astype(np.int8))
    assert q[0, 120:128].tolist() == [0, 2, 2, 4, 0, -2, -2, -4]
    assert q[0, 128] == -8 and np.array_equal(q[0, 129:], mult.astype(np.int8))
    assert not q[1, :128].any() and np.array_equal(q[1, 128:], W[1, 128:].astype(np.int8))
    # round to nearest without the clip search: scale fl32(amax / 7)
    Wr = np.zeros((1, 128), np.float32)
    Wr[0, :15] = [7.0, 0.5, 1.5, 2.5, 3.5, 4.5, 5.5, 6.5, -0.5, -1.5, -2.5, -3.5, -4.5, -5.5, -6.5]
    words, scales = ops.w4a8_moe_quantize_weights(to_dev(Wr), mse_clip=False)
    assert host(scales)[0, 0] == np.float32(1.0)
    assert oracle.int4_unpack(host(words))[0, :15].tolist() == [7, 0, 2, 2, 4, 4, 6, 6, 0, -2, -2, -4, -4, -6, -6]
