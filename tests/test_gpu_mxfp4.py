"""GPU parity of the MXFP4 group-32 weight form, called through the C-ABI.

The quantizer's codes and scale bytes are compared bit for bit.  GEMM
products are exact on both sides (E4M3 x E2M1 x a power of two); only the
matrix core's fp32 summation differs from the oracle's fp64 one, so the
outputs are held to the float bar with the tight Frobenius bound, and to
exact equality where every partial sum is an fp32 integer.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_util import (GEMM_FRO_TIGHT, assert_float_parity, bf16_to_dev, check_layer_output, check_requant,
                      edge_shape_maxrel, host, near_midpoint, say, to_dev)
from oracle import mxfp4_oracle as mx
from quantized_grouped_gemm_token_amd import ops, workloads
from quantized_grouped_gemm_token_amd.layer import W4A8MoEMxfp4

pytestmark = pytest.mark.gpu

ALGOS = (ops.W4A8_GG_STREAM, ops.W4A8_GG_TILED)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert ops.w4a8_moe_device_supported(), "the current device is not a gfx950"
    yield
    torch.cuda.synchronize()


# ------------------------------------------------------------------ offline quantizer
@pytest.mark.parametrize("N,K", [(1, 32), (64, 128), (300, 2048), (7, 6144)])
def test_quantize_weights_mxfp4(N, K, rng):
    W = (rng.standard_normal((N, K)) * np.exp2(rng.integers(-20, 20, size=(N, 1)))).astype(np.float32)
    if N >= 7:
        W[0, :32] = 0.0                                            # all-zero block
        W[1, :32] = np.float32([6, 5, 3.5, 2.5, 1.75, 1.25, 0.75, 0.25] * 4)   # every tie, scale 2^0
        W[1, 32:64] = -W[1, :32]
        W[2, :32] = -0.0                                           # negative zeros keep their sign
        W[3, :32] = np.float32(1e-40) * np.arange(32)              # subnormal block
        W[4, :32] = np.float32(3e38) * np.linspace(-1, 1, 32)      # near the top of fp32
        W[5, :32] = np.float32(7.9)                                # saturates at 6 after scaling by 2^0
        W[6, :32] = rng.standard_normal(32).astype(np.float32) * np.float32(2.0 ** -60)
    say(f"quantize_weights_mxfp4 N={N} K={K}")
    packed, scales = ops.w4a8_moe_quantize_weights_mxfp4(to_dev(W))
    codes_ref, s_ref = mx.quantize_mxfp4(W)
    assert np.array_equal(host(scales), s_ref)
    assert np.array_equal(host(packed), mx.fp4_pack(codes_ref))


# ------------------------------------------------------------------ layout step
@pytest.mark.parametrize("E,N,K", [(1, 16, 128), (3, 64, 384), (2, 4096, 6144)])
def test_prepack_mxfp4(E, N, K, rng):
    w = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    s = rng.integers(0, 256, size=(E, N, K // 32), dtype=np.uint8)
    say(f"prepack_mxfp4 E={E} N={N} K={K}")
    wb, sb = ops.w4a8_moe_prepack_mxfp4(to_dev(w), to_dev(s))
    G = K // 128
    # GEMM storage: [E][N/16][G][16][64] weight bytes, [E][G][N][4] scale bytes
    assert np.array_equal(host(wb), w.reshape(E, N // 16, 16, G, 64).transpose(0, 1, 3, 2, 4))
    assert np.array_equal(host(sb), s.reshape(E, N, G, 4).transpose(0, 2, 1, 3))


# ------------------------------------------------------------------ steps 4 and 6
def _prepacked(w, s):
    return ops.w4a8_moe_prepack_mxfp4(to_dev(w), to_dev(s))


def _problem(rng, E, N, K, counts, src_rows=None, scale_lo=118, scale_hi=136):
    w = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    s = rng.integers(scale_lo, scale_hi, size=(E, N, K // 32)).astype(np.uint8)
    M = int(np.sum(counts))
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    src = M if src_rows is None else src_rows
    x = rng.standard_normal((src, K)).astype(np.float32) * np.exp2(rng.integers(-3, 3, size=(src, 1)))
    a, sa = oracle.quant_rows(x.astype(np.float32))
    rows = None if src_rows is None else rng.integers(0, src, size=M).astype(np.int32)
    return w, s, offsets, a, sa, rows


def _gemm(w, s, offsets, a, sa, rows, algo):
    M = int(offsets[-1])
    wb, sb = _prepacked(w, s)
    out = ops.w4a8_moe_grouped_gemm_mxfp4_prepacked(to_dev(a), to_dev(sa), None if rows is None else to_dev(rows),
                                          to_dev(offsets), wb, sb, M, algo=algo)
    return host(out)


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("E,N,K,counts,gather", [
    (4, 256, 256, [3, 0, 17, 1], True),
    (3, 128, 384, [70, 1, 129], False),            # odd group count
    (5, 192, 128, [0, 0, 0, 5, 0], True),
    (2, 64, 1024, [300, 33], True),
    (8, 512, 640, [16, 16, 16, 16, 0, 15, 17, 1], False),
    (3, 320, 256, [200, 241, 0], True),            # partial tiles; N not a multiple of 256
    (1, 768, 6144, [130], False),                  # a wide tile half past N, long K
    (4, 256, 256, [128, 129, 257, 513], False),    # square tiles of equal height: 1, 2 and 3 per expert
])
def test_grouped_gemm_mxfp4(E, N, K, counts, gather, algo, rng):
    w, s, offsets, a, sa, rows = _problem(rng, E, N, K, counts, src_rows=40 if gather else None)
    want = mx.grouped_gemm_mxfp4(a, sa, rows, offsets, w, s)
    say(f"grouped_gemm_mxfp4 E={E} N={N} K={K} counts={counts} gather={gather} algo={algo}")
    got = _gemm(w, s, offsets, a, sa, rows, algo)
    assert_float_parity(got, want, "grouped_gemm_mxfp4", fro_tight=GEMM_FRO_TIGHT, maxrel=edge_shape_maxrel(N))


@pytest.mark.parametrize("algo", ALGOS)
def test_grouped_gemm_mxfp4_exact_integers(algo, rng):
    # integer activations, scale bytes 127 and 128 (x1, x2) and unit token
    # scales: every output is a multiple of 1/2 far below 2^23, which fp32
    # holds, so any misplaced K element, nibble or scale byte changes it
    E, N, K, M = 2, 128, 512, 24
    vals = rng.integers(-16, 17, size=(M, K)).astype(np.float32)
    codes = oracle.e4m3_encode(vals)
    w = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    s = rng.integers(127, 129, size=(E, N, K // 32)).astype(np.uint8)
    offsets = np.array([0, 10, M], np.int32)
    ones = np.ones(M, np.float32)
    want = mx.grouped_gemm_mxfp4(codes, ones, None, offsets, w, s)
    say(f"grouped_gemm_mxfp4 exact integers algo={algo}")
    assert np.array_equal(_gemm(w, s, offsets, codes, ones, None, algo), want)


# ------------------------------------------------------- steps 4 + 5, fused
@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("E,I,K,counts,gather", [
    (4, 128, 256, [3, 0, 17, 1], True),
    (3, 256, 384, [70, 1, 129], False),
    (2, 384, 1024, [300, 33], True),                  # N = 768: a wide tile half past N
])
def test_grouped_gemm_swiglu_mxfp4(E, I, K, counts, gather, algo, rng):
    w, s, offsets, a, sa, rows = _problem(rng, E, 2 * I, K, counts, src_rows=40 if gather else None,
                                          scale_lo=120, scale_hi=128)
    M = int(offsets[-1])
    want = oracle.swiglu_f32(mx.grouped_gemm_mxfp4(a, sa, rows, offsets, w, s))
    say(f"grouped_gemm_swiglu_mxfp4 E={E} I={I} K={K} counts={counts} algo={algo}")
    wb, sb = _prepacked(w, s)
    act, pmax = ops.w4a8_moe_grouped_gemm_swiglu_mxfp4_prepacked(to_dev(a), to_dev(sa), None if rows is None else to_dev(rows),
                                                       to_dev(offsets), wb, sb, M, algo=algo)
    act, pmax = host(act), host(pmax)
    assert_float_parity(act, want, "grouped_gemm_swiglu_mxfp4", fro_tight=GEMM_FRO_TIGHT, maxrel=edge_shape_maxrel(I))
    row = np.abs(act).max(axis=1)
    assert pmax.shape == (M, I // 64)
    assert np.array_equal(pmax.max(axis=1), row)
    assert np.all(pmax <= row[:, None])
    # the fused path's codes against the unfused one's on the same inputs
    out = ops.w4a8_moe_grouped_gemm_mxfp4_prepacked(to_dev(a), to_dev(sa), None if rows is None else to_dev(rows),
                                          to_dev(offsets), wb, sb, M, algo=algo)
    q_ref, s_ref = ops.w4a8_moe_swiglu(out)
    q, sq = ops.w4a8_moe_requant(to_dev(act), to_dev(pmax))
    q, sq, q_ref, s_ref = host(q), host(sq), host(q_ref), host(s_ref)
    assert np.allclose(sq, s_ref, rtol=1e-5, atol=0)
    diff = q != q_ref
    assert np.all(near_midpoint(want, s_ref, rel=1e-4)[diff]), f"{int(diff.sum())} codes differ off a midpoint"


# ------------------------------------------------------------------ the layer
def _layer_vs_oracle(wl, algo, fused):
    sh = wl.shape
    w13, s13, w2, s2 = workloads.mxfp4_weights(wl)
    res = mx.moe_layer_mxfp4(wl.x_bf16, wl.logits, w13, s13, w2, s2, k=sh.k)
    say(f"layer_mxfp4 {sh.name} algo={algo} fused={fused}")
    moe = W4A8MoEMxfp4(to_dev(w13), to_dev(s13), to_dev(w2), to_dev(s2), k=sh.k, fused=fused)
    y = host(moe(bf16_to_dev(wl.x_bf16), to_dev(wl.logits), algo=algo))
    b = moe.buffers(sh.T)
    assert np.array_equal(host(b["qx"]), res["qx"])
    assert np.array_equal(host(b["ids"]), res["ids"])
    for name in ("offsets", "row_token", "inv_pos"):
        assert np.array_equal(host(b[name]), res[name]), name
    if fused:
        act = host(b["act"])
        assert_float_parity(act, res["a_f32"], "MXFP4 gate/up + SwiGLU", fro_tight=GEMM_FRO_TIGHT)
        assert np.array_equal(host(b["pmax"]).max(axis=1), np.abs(act).max(axis=1)), "row maxima of act"
    else:
        assert_float_parity(host(b["h"]), res["h"], "MXFP4 gate/up", fro_tight=GEMM_FRO_TIGHT)
    # the re-quantized codes: exact on the GPU's own act (recomputed from its h on the unfused
    # path), and where they differ from the independent run, explained by the act difference
    act_gpu = host(b["act"]) if fused else oracle.swiglu_f32(host(b["h"]))
    qa_gpu, sa_gpu = host(b["qa"]), host(b["sa"])
    flipped = check_requant(act_gpu, qa_gpu, sa_gpu, res["qa"], act_exact=fused)
    token_flipped = flipped.any(axis=1)[res["inv_pos"]].reshape(sh.T, sh.k).any(axis=1)
    o_same = mx.grouped_gemm_mxfp4(qa_gpu, sa_gpu, None, res["offsets"], w2, s2)
    y_same = oracle.unpermute(o_same, res["inv_pos"], res["w"])
    maxrel_bar = edge_shape_maxrel(sh.H) if sh.name.startswith("custom") else 1e-2
    r = check_layer_output(y, res["y"], y_same, token_flipped, "MXFP4 layer output", maxrel=maxrel_bar)
    say(f"layer output vs oracle: {r}; {int(flipped.sum())} codes differ from the independent run")


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("algo", ALGOS)
def test_layer_mxfp4_tiny(algo, fused):
    _layer_vs_oracle(workloads.make_config(0), algo, fused)


@pytest.mark.parametrize("T,H,I,E,k", [(64, 1024, 256, 16, 4), (37, 384, 256, 5, 3), (1, 256, 128, 8, 8),
                                       (200, 256, 128, 4, 2)])
@pytest.mark.parametrize("algo", ALGOS)
def test_layer_mxfp4_shapes(T, H, I, E, k, algo):
    _layer_vs_oracle(workloads.make_custom(T, H, I, E, k, seed=T * 1000 + E + 7), algo, fused=True)
