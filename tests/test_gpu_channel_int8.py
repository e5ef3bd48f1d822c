"""GPU parity of the per-channel INT4 x per-token INT8 variant, called through the C-ABI.

Integer steps are compared bit for bit (codes, row sums, packed weights).
The GEMM's integer sums are exact on both sides, so its outputs may differ
only by the fp32 rounding of the two scale products (relative 1e-6).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_util import (assert_float_parity, bf16_to_dev, check_layer_output, check_requant, host, prepack_int4, say,
                      to_dev)
from quantized_grouped_gemm_token_amd import ops, workloads
from quantized_grouped_gemm_token_amd.layer import W4A8MoEChannel

pytestmark = pytest.mark.gpu

ALGOS = (ops.W4A8_GG_STREAM, ops.W4A8_GG_TILED)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert ops.w4a8_moe_device_supported(), "the current device is not a gfx950"
    yield
    torch.cuda.synchronize()


def _bf16(x32):
    return oracle.f32_to_bf16_bits(np.asarray(x32, np.float32))


# ------------------------------------------------------------------ step 1
@pytest.mark.parametrize("T,H", [(1, 128), (37, 512), (256, 6144), (3, 16384), (2, 17408), (1100, 6144), (1030, 2176)])
def test_quant_act_i8(T, H, rng):
    x = rng.standard_normal((T, H)).astype(np.float32)
    x[:, rng.choice(H, max(1, H // 100), replace=False)] *= 20.0
    if T > 2:
        x[1] = 0.0                                           # all-zero row
        x[2, :] = np.resize(np.arange(-126, 128, dtype=np.float32) + np.float32(0.5), H)
        x[2, 0] = 127.0                                      # scale 1: exact half-integer quotients
    xb = _bf16(x)
    say(f"quant_act_i8 T={T} H={H}")
    qx, sx, rs = ops.w4a8_moe_quant_act_i8(bf16_to_dev(xb))
    c_ref, s_ref = oracle.quant_act_i8(xb)
    r_ref = oracle.code_row_sums(c_ref)
    assert np.array_equal(host(sx).view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(host(qx), c_ref)
    assert np.array_equal(host(rs), r_ref)


# ------------------------------------------------------------------ steps 4 and 6
def _problem(rng, E, N, K, counts, gather):
    T = 23
    R = int(np.sum(counts))
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    src = T if gather else R
    x = rng.standard_normal((src, K)).astype(np.float32)
    x[:, rng.choice(K, max(1, K // 64), replace=False)] *= 15.0
    codes, scale = oracle.quant_rows_i8(x)
    rowsum = oracle.code_row_sums(codes)
    rows = rng.integers(0, T, size=R).astype(np.int32) if gather else None
    words = rng.integers(0, 2**32, size=(E, N, K // 8), dtype=np.uint32).view(np.int32)
    ws = rng.lognormal(-4, 0.5, size=(E, N)).astype(np.float32)
    return codes, scale, rowsum, rows, offsets, words, ws


def _gemm(codes, scale, rowsum, rows, offsets, words, ws, algo):
    R = int(offsets[-1])
    out = ops.w4a8_moe_grouped_gemm_i8_prepacked(to_dev(codes), to_dev(scale), to_dev(rowsum),
                                       to_dev(rows) if rows is not None else None, to_dev(offsets),
                                       prepack_int4(words)[0], to_dev(ws), M_total=R, algo=algo)
    return host(out)


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("E,N,K,counts,gather", [
    (4, 64, 128, [3, 0, 17, 1], True),
    (3, 192, 384, [40, 1, 300], True),             # odd group count, ragged tiles
    (2, 512, 2048, [257, 31], False),
    (8, 256, 6144, [5, 0, 9, 2, 0, 11, 1, 64], True),
    (1, 4096, 1024, [1], False),
])
def test_grouped_gemm_i8(E, N, K, counts, gather, algo, rng):
    p = _problem(rng, E, N, K, counts, gather)
    say(f"grouped_gemm_i8 E={E} N={N} K={K} counts={counts} algo={algo}")
    got = _gemm(*p, algo)
    want = oracle.grouped_gemm_i8(p[0], p[1], p[3], p[4], p[5], p[6])
    zero = want == 0
    assert np.all(got[zero] == 0)
    rel = np.abs(got[~zero].astype(np.float64) - want[~zero]) / np.abs(want[~zero].astype(np.float64))
    assert rel.max(initial=0.0) <= 1e-6, rel.max()


# ------------------------------------------------------- steps 4 + 5, fused
@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("E,I,K,counts,gather", [
    (4, 128, 128, [3, 0, 17, 1], True),
    (3, 384, 384, [40, 1, 300], True),               # N = 768: a wide tile half past N
    (2, 256, 2048, [257, 31], False),
])
def test_grouped_gemm_swiglu_i8(E, I, K, counts, gather, algo, rng):
    codes, scale, rowsum, rows, offsets, words, ws = _problem(rng, E, 2 * I, K, counts, gather)
    R = int(offsets[-1])
    want = oracle.swiglu_f32(oracle.grouped_gemm_i8(codes, scale, rows, offsets, words, ws))
    say(f"grouped_gemm_swiglu_i8 E={E} I={I} K={K} counts={counts} algo={algo}")
    act, pmax = ops.w4a8_moe_grouped_gemm_swiglu_i8_prepacked(
        to_dev(codes), to_dev(scale), to_dev(rowsum), to_dev(rows) if rows is not None else None, to_dev(offsets),
        prepack_int4(words)[0], to_dev(ws), R, algo=algo)
    act, pmax = host(act), host(pmax)
    # the GEMM values differ from the oracle's by the rounding of the scale product only
    assert_float_parity(act, want, "grouped_gemm_swiglu_i8", fro_tight=1e-5)
    assert pmax.shape == (R, I // 64)
    assert np.array_equal(pmax.max(axis=1), np.abs(act).max(axis=1))
    assert np.all(pmax <= np.abs(act).max(axis=1, keepdims=True))


@pytest.mark.parametrize("M,I", [(1, 128), (300, 2048), (3, 8192), (2, 8320)])
def test_requant_i8(M, I, rng):
    act = (rng.standard_normal((M, I)) * 3.0).astype(np.float32)
    if M > 2:
        act[1] = 0.0
    pmax = np.abs(act).reshape(M, I // 64, 64).max(axis=2).astype(np.float32)
    say(f"requant_i8 M={M} I={I}")
    q, sq, rs = ops.w4a8_moe_requant_i8(to_dev(act), to_dev(pmax))
    q_ref, s_ref = oracle.quant_rows_i8(act)
    r_ref = oracle.code_row_sums(q_ref)
    assert np.array_equal(host(sq).view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(host(q), q_ref)
    assert np.array_equal(host(rs), r_ref)


# ------------------------------------------------------------------ step 5
@pytest.mark.parametrize("M,I", [(5, 128), (300, 2048)])
def test_swiglu_i8(M, I, rng):
    h = (rng.standard_normal((M, 2 * I)) * 2.0).astype(np.float32)
    say(f"swiglu_i8 M={M} I={I}")
    qa, sa, ra = ops.w4a8_moe_swiglu_i8(to_dev(h))
    qa, sa, ra = host(qa), host(sa), host(ra)
    act = oracle.swiglu_f32(h)
    c_ref, s_ref = oracle.quant_rows_i8(act)
    assert np.allclose(sa, s_ref, rtol=2e-6, atol=0)
    # codes: each side rounds its own fp32 quotient; a different code is only
    # allowed where the exact quotient lies within 1e-4 of a half-integer
    q = act.astype(np.float64) / s_ref.astype(np.float64)[:, None]
    near = np.abs(np.abs(q - np.floor(q)) - 0.5) < 1e-4
    diff = qa.astype(np.int32) != c_ref.astype(np.int32)
    assert np.all(np.abs(qa.astype(np.int32) - c_ref.astype(np.int32)) <= 1)
    assert np.all(near[diff]), f"{int((diff & ~near).sum())} codes differ away from a rounding boundary"
    assert np.array_equal(ra, qa.astype(np.int64).sum(axis=1))


# ------------------------------------------------------------------ offline quantizer
@pytest.mark.parametrize("N,K", [(64, 128), (300, 2048)])
def test_quantize_weights_channel(N, K, rng):
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    W[0] = 0.0
    W[1, :] = np.resize(np.float32([7.0, -3.5, 2.5, 0.5, -0.5]), K)    # exact ties at scale 1
    say(f"quantize_weights_channel N={N} K={K}")
    words, scales = ops.w4a8_moe_quantize_weights_channel(to_dev(W))
    q_ref, s_ref = oracle.quantize_int4_channel(W)
    assert np.array_equal(host(scales).view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(host(words), oracle.int4_pack(q_ref))


# ------------------------------------------------------------------ the layer
@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("cfg", [0, "mid"])
@pytest.mark.parametrize("algo", ALGOS)
def test_layer_channel_int8(cfg, algo, fused):
    wl = workloads.make_config(0) if cfg == 0 else workloads.make_custom(64, 1024, 256, 16, 4, seed=77)
    sh = wl.shape
    s13, s2 = workloads.channel_scales(wl)
    say(f"layer_i8 {sh.name} algo={algo} fused={fused}")
    moe = W4A8MoEChannel(to_dev(wl.w13), to_dev(s13), to_dev(wl.w2), to_dev(s2), k=sh.k, fused=fused)
    y = host(moe(bf16_to_dev(wl.x_bf16), to_dev(wl.logits), algo=algo))
    ref = oracle.moe_layer_i8(wl.x_bf16, wl.logits, wl.w13, s13, wl.w2, s2, k=sh.k)
    b = moe.buffers(sh.T)
    act_gpu = host(b["act"]) if fused else oracle.swiglu_f32(host(b["h"]))
    qa_gpu, sa_gpu = host(b["qa"]), host(b["sa"])
    flipped = check_requant(act_gpu, qa_gpu, sa_gpu, ref["qa"], int8=True, act_exact=fused)
    assert np.array_equal(host(b["ra"]), oracle.code_row_sums(qa_gpu))
    token_flipped = flipped.any(axis=1)[ref["inv_pos"]].reshape(sh.T, sh.k).any(axis=1)
    o_same = oracle.grouped_gemm_i8(qa_gpu, sa_gpu, None, ref["offsets"], wl.w2, s2)
    y_same = oracle.unpermute(o_same, ref["inv_pos"], ref["w"])
    r = check_layer_output(y, ref["y"], y_same, token_flipped, f"layer_i8 {sh.name}")
    say(f"layer_i8 output vs oracle: {r}; {int(flipped.sum())} codes differ from the independent run")
