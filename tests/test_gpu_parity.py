"""GPU parity: every library call against the CPU oracle, through the C ABI.

Bars: bit-exact FP8 codes, scales, routing ids, permutation and offsets;
routing weights within 1e-6 relative; float outputs within relative
Frobenius 2e-3 and max relative 1e-2 on elements above 1e-3 of the row norm
(and much tighter where both sides see bit-identical inputs).  The oracle is
always fed from the seeded generators or from its own earlier steps, never
from the GPU.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import (GEMM_FRO_TIGHT, assert_float_parity, bf16_to_dev, check_layer_output, check_requant,
                      edge_shape_maxrel, host, near_midpoint, prepack_int4, say, to_dev)
from quantized_grouped_gemm_token_amd import ops, workloads
from quantized_grouped_gemm_token_amd.layer import W4A8MoE

pytestmark = pytest.mark.gpu

ALGOS = (ops.W4A8_GG_STREAM, ops.W4A8_GG_TILED, ops.W4A8_GG_AUTO)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert ops.w4a8_moe_device_supported(), "the current device is not a gfx950"
    yield
    torch.cuda.synchronize()


def _bits(x32):
    return torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(torch.bfloat16).view(torch.int16).numpy() \
        .view(np.uint16)


# ------------------------------------------------------------------ step 1
def test_quant_act_special_values():
    pos = oracle.E4M3_VALUES[:0x7F]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)       # exact in bf16 (<= 5 significant bits)
    H = 384
    rows = np.zeros((6, H), np.float32)
    rows[0, 0] = 448.0                                           # scale exactly 1: midpoints hit ties
    rows[0, 1:1 + mids.size] = mids
    rows[0, 1 + mids.size:1 + 2 * mids.size] = -mids[: H - 1 - mids.size]
    rows[1, :] = -0.0                                            # all-zero row (signed zeros)
    rows[1, ::2] = 0.0
    rows[2, 0] = 3.0e38                                          # huge amax: the rest underflow to +-0
    rows[2, 1:] = np.linspace(-1e-3, 1e-3, H - 1)
    rows[3, :] = -7.5                                            # constant row
    rows[4, :] = np.float32(2.0 ** -130) * np.arange(H)          # bf16 subnormals
    rows[5, :] = np.exp2(np.linspace(-20, 20, H)) * np.where(np.arange(H) % 3 == 0, -1, 1)
    bits = _bits(rows)
    want_q, want_s = oracle.quant_act(bits)
    say("quant_act special values")
    qx, sx = ops.w4a8_moe_quant_act(bf16_to_dev(bits))
    assert np.array_equal(host(qx), want_q)
    assert np.array_equal(host(sx), want_s)


@pytest.mark.parametrize("T,H", [(1, 128), (37, 384), (300, 6144), (5, 2176), (3, 16384), (2, 17408),
                                 (1100, 6144), (1024, 2176), (1030, 1024), (1500, 8192), (1025, 9216)])
def test_quant_act_random(T, H, rng):
    mag = np.exp2(rng.integers(-12, 12, size=(T, 1))).astype(np.float32)
    x = (rng.standard_normal((T, H)).astype(np.float32) * mag)
    x[:, rng.choice(H, size=max(1, H // 100), replace=False)] *= 20
    bits = _bits(x)
    want_q, want_s = oracle.quant_act(bits)
    say(f"quant_act T={T} H={H}")
    qx, sx = ops.w4a8_moe_quant_act(bf16_to_dev(bits))
    assert np.array_equal(host(qx), want_q)
    assert np.array_equal(host(sx), want_s)


# ------------------------------------------------------------------ step 2
@pytest.mark.parametrize("T,E,k,renorm", [(1, 8, 8, True), (50, 256, 8, True), (50, 256, 8, False),
                                          (33, 1024, 16, True), (20, 100, 100, True), (7, 65, 3, False),
                                          (16, 4, 1, True), (9, 500, 8, True), (9, 500, 8, False)])
def test_route(T, E, k, renorm, rng):
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[:, 5 % E] = logits[:, 2 % E]                        # forced ties
    logits[:, 36 % E] = logits[:, 20 % E]                      # ... between lanes of different 16-lane rows
    logits[:, 67 % E] = logits[:, 3 % E]                       # ... between slots of one lane
    logits[0, :] = np.round(logits[0, :])                     # many ties in one row
    want_ids, want_w = oracle.route(logits, k, renorm)
    say(f"route T={T} E={E} k={k} renorm={renorm}")
    ids, w = ops.w4a8_moe_route(to_dev(logits), k, renorm)
    assert np.array_equal(host(ids), want_ids)
    gw = host(w).astype(np.float64)
    assert np.all(np.abs(gw - want_w) <= 1e-6 * np.abs(want_w))


# ------------------------------------------------------------------ step 3
@pytest.mark.parametrize("T,E,k", [(16, 8, 2), (128, 256, 8), (3000, 256, 8), (1500, 1024, 8), (700, 3, 2),
                                   (2048, 256, 8), (127, 256, 8), (100, 1024, 8), (1, 1024, 1), (129, 256, 8),
                                   (500, 256, 8), (512, 1024, 8), (513, 256, 8)])   # one block up to 4096 indices
def test_permute(T, E, k, rng):
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    if T == 700:
        ids[:] = rng.integers(0, E, size=ids.shape)            # repeated experts per token
    want = oracle.permute(ids, E)
    say(f"permute T={T} E={E} k={k}")
    got = ops.w4a8_moe_permute(to_dev(ids), E)
    for g, w_, name in zip(got, want, ("offsets", "row_token", "inv_pos")):
        assert np.array_equal(host(g), w_), name


@pytest.mark.parametrize("T,E,k", [(100, 64, 4), (700, 256, 8), (1000, 256, 8)])   # one block; three launches
def test_permute_skips_ids_out_of_range(T, E, k, rng):
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    bad = rng.random(ids.shape) < 0.05
    ids[bad] = np.where(rng.random(int(bad.sum())) < 0.5, -1, E + 3).astype(np.int32)
    # the oracle on the same ids with every out-of-range one sent to an extra expert E, which sorts last
    want_off, want_rt, want_inv = oracle.permute(np.where(bad, E, ids), E + 1)
    say(f"permute with {int(bad.sum())} ids out of range, T={T} E={E} k={k}")
    offsets, row_token, inv_pos = (host(t) for t in ops.w4a8_moe_permute(to_dev(ids), E))
    routed = int(want_off[E])
    assert routed == T * k - int(bad.sum())
    assert np.array_equal(offsets, want_off[:E + 1])
    assert np.array_equal(row_token[:routed], want_rt[:routed])
    assert np.array_equal(inv_pos[~bad.reshape(-1)], want_inv[~bad.reshape(-1)])
    assert np.all(inv_pos[bad.reshape(-1)] == -1)


def test_permute_empty():
    say("permute T=0")
    offsets, _, _ = ops.w4a8_moe_permute(torch.zeros((0, 4), dtype=torch.int32, device="cuda:0"), 16)
    assert np.array_equal(host(offsets), np.zeros(17, np.int32))


# --------------------------------------------------------------- steps 4/6
@pytest.mark.parametrize("E,N,K,scales", [(1, 16, 128, True), (3, 64, 384, True), (2, 48, 256, False),
                                          (2, 4096, 6144, True)])
def test_prepack_int4(E, N, K, scales, rng):
    w = rng.integers(0, 2**32, size=(E, N, K // 8), dtype=np.uint32).view(np.int32)
    s = rng.standard_normal((E, N, K // 128)).astype(np.float32) if scales else None
    say(f"prepack_int4 E={E} N={N} K={K} scales={scales}")
    wb, sb = prepack_int4(w, s)
    G = K // 128
    # GEMM storage: [E][N/16][G][16][16] words, [E][G][N] scales; inside a word the
    # nibble of k = 8c + i (i < 4) moves to nibble 2i, that of k = 8c + 4 + i to 2i + 1
    blk = w.reshape(E, N // 16, 16, G, 16).transpose(0, 1, 3, 2, 4).view(np.uint32)
    want = np.zeros_like(blk)
    for i in range(8):
        pos = 2 * i if i < 4 else 2 * (i - 4) + 1
        want |= ((blk >> np.uint32(4 * i)) & np.uint32(15)) << np.uint32(4 * pos)
    assert np.array_equal(host(wb).view(np.uint32), want)
    if scales:
        assert np.array_equal(host(sb).view(np.uint32), s.transpose(0, 2, 1).view(np.uint32))
    else:
        assert sb is None


def _gemm_problem(rng, E, N, K, counts, src_rows=None):
    w = rng.integers(0, 2**32, size=(E, N, K // 8), dtype=np.uint32).view(np.int32)
    s = rng.lognormal(-4, 0.5, size=(E, N, K // 128)).astype(np.float32)
    M = int(np.sum(counts))
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    src = M if src_rows is None else src_rows
    x = rng.standard_normal((src, K)).astype(np.float32) * np.exp2(rng.integers(-3, 3, size=(src, 1)))
    a, sa = oracle.quant_rows(x.astype(np.float32))
    rows = None if src_rows is None else rng.integers(0, src, size=M).astype(np.int32)
    return w, s, offsets, a, sa, rows


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("E,N,K,counts,gather", [
    (4, 256, 256, [3, 0, 17, 1], True),
    (3, 128, 384, [70, 1, 129], False),
    (5, 192, 128, [0, 0, 0, 5, 0], True),
    (2, 64, 1024, [300, 33], True),
    (8, 512, 640, [16, 16, 16, 16, 0, 15, 17, 1], False),
    (3, 320, 256, [200, 241, 0], True),            # partial tiles of 7/8 row blocks; N not a multiple of 256
    (4, 256, 256, [128, 129, 257, 513], False),    # one wide M block, one square, 3 and 5 wide of equal height
    (3, 512, 256, [70, 280, 525], True),           # wide bodies of 5, 6 and 7 A blocks; 1, 3 and 5 wide M blocks
    (2, 512, 384, [512, 769], True),
    (6, 128, 256, [17, 3, 0, 1, 2, 0], True),       # M_total <= 4 E: the one-block stream kernel, 2 row passes
    (3, 768, 256, [1500, 5, 300], True),            # 6 square M blocks: a group of 4 and a partial group of 2 (tiled order)
    (3, 768, 256, [1400, 5, 300], True),            # 11 wide M blocks: groups of 4, 4 and 3
    (8, 256, 384, [9, 40, 0, 3, 1, 0, 2, 5], False),  # AUTO: both kernels launched, the tiled one runs
    (8, 256, 384, [9, 20, 0, 3, 1, 0, 2, 5], True),   # AUTO: both kernels launched, the stream one runs
])
def test_grouped_gemm(E, N, K, counts, gather, algo, rng):
    w, s, offsets, a, sa, rows = _gemm_problem(rng, E, N, K, counts, src_rows=40 if gather else None)
    want = oracle.grouped_gemm(a, sa, rows, offsets, w, s)
    M = int(offsets[-1])
    say(f"grouped_gemm E={E} N={N} K={K} counts={counts} gather={gather} algo={algo}")
    out = ops.w4a8_moe_grouped_gemm_prepacked(to_dev(a), to_dev(sa), None if rows is None else to_dev(rows), to_dev(offsets),
                                    *prepack_int4(w, s), M, algo=algo)
    assert_float_parity(host(out), want, "grouped_gemm", fro_tight=GEMM_FRO_TIGHT, maxrel=edge_shape_maxrel(N))


@pytest.mark.parametrize("algo", ALGOS)
def test_grouped_gemm_exact_integers(algo, rng):
    # unit scales and small integer activations: every output is an exact
    # integer that fp32 holds, so the GPU must match it exactly
    E, N, K, M = 2, 128, 512, 24
    vals = rng.integers(-16, 17, size=(M, K)).astype(np.float32)
    codes = oracle.e4m3_encode(vals)
    w = rng.integers(0, 2**32, size=(E, N, K // 8), dtype=np.uint32).view(np.int32)
    s = np.ones((E, N, K // 128), np.float32)
    offsets = np.array([0, 10, M], np.int32)
    want = oracle.grouped_gemm(codes, np.ones(M, np.float32), None, offsets, w, s)
    say(f"grouped_gemm exact integers algo={algo}")
    out = ops.w4a8_moe_grouped_gemm_prepacked(to_dev(codes), to_dev(np.ones(M, np.float32)), None, to_dev(offsets),
                                    *prepack_int4(w, s), M, algo=algo)
    assert np.array_equal(host(out), want)


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("counts", [
    [17, 3, 0, 1, 2, 0],             # one-block stream kernel
    [9, 40, 0, 3, 1, 0],             # a 40-row expert: the tiled kernel under AUTO
    [18, 19, 20, 0, 2, 1],           # the most rows AUTO gives the stream kernel
    [64, 65, 33, 16, 0, 2],          # the multi-block stream kernel: 4, 2 and 1 blocks per load
    [1500, 3, 0, 1, 2, 0],           # 6 square M blocks of equal height in the tiled kernel, 24 row passes in the other
    [70, 280, 525, 0, 3, 1],         # wide M blocks: 1, 3 and 5 per expert, bodies of 5, 6 and 7 A blocks
])
def test_algos_agree_bitwise(counts, fused, rng):
    """The kernel choice is a matter of speed only: the three algos give the same bits (same
    products, same group order, same fp32 operations), whichever kernel runs each expert."""
    E, K = len(counts), 384
    N = 256
    w, s, offsets, a, sa, rows = _gemm_problem(rng, E, N, K, counts, src_rows=50)
    M = int(offsets[-1])
    wb, sb = prepack_int4(w, s)
    say(f"algos agree counts={counts} fused={fused}")
    outs = []
    for algo in ALGOS:
        if fused:
            act, pmax = ops.w4a8_moe_grouped_gemm_swiglu_prepacked(to_dev(a), to_dev(sa), to_dev(rows),
                                                                   to_dev(offsets), wb, sb, M, algo=algo)
            outs.append(np.concatenate([host(act).ravel(), host(pmax).max(axis=1)]))
        else:
            outs.append(host(ops.w4a8_moe_grouped_gemm_prepacked(to_dev(a), to_dev(sa), to_dev(rows),
                                                                 to_dev(offsets), wb, sb, M, algo=algo)).ravel())
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32))


@pytest.mark.parametrize("hot", [None, 517])
def test_auto_choice_many_experts(hot, rng):
    """The device-side kernel choice with more experts than one pass of its offsets scan covers (256):
    with every expert at 3 rows or fewer the streaming kernel runs, with a 100-row expert at index 517 the
    tiled one; either way the result holds the GEMM bar and equals both forced choices bit for bit."""
    E, N, K = 600, 128, 256
    counts = rng.integers(0, 4, size=E)
    if hot is not None:
        counts[hot] = 100
    w, s, offsets, a, sa, rows = _gemm_problem(rng, E, N, K, list(counts), src_rows=64)
    M = int(offsets[-1])
    assert 20 < M <= 10 * E                       # the band where both kernels are launched
    want = oracle.grouped_gemm(a, sa, rows, offsets, w, s)
    wb, sb = prepack_int4(w, s)
    say(f"auto choice E={E} hot={hot} M={M}")
    outs = [host(ops.w4a8_moe_grouped_gemm_prepacked(to_dev(a), to_dev(sa), to_dev(rows), to_dev(offsets), wb, sb, M,
                                                     algo=algo)) for algo in ALGOS]
    assert_float_parity(outs[-1], want, "grouped_gemm auto", fro_tight=GEMM_FRO_TIGHT, maxrel=edge_shape_maxrel(N))
    for o in outs[:-1]:
        assert np.array_equal(o.view(np.uint32), outs[-1].view(np.uint32))


# ------------------------------------------------------- steps 4 + 5, fused
def _pmax_of(act):
    """Partial row maxima of |act|, one per 64 columns (what the fused GEMM may write)."""
    M, I = act.shape
    return np.abs(act).reshape(M, I // 64, 64).max(axis=2).astype(np.float32)


def _check_pmax(pmax, act):
    # every entry is the max over some of the row's columns; their max is the row's
    M, I = act.shape
    assert pmax.shape == (M, I // 64)
    row = np.abs(act).max(axis=1)
    assert np.array_equal(pmax.max(axis=1), row)
    assert np.all(pmax <= row[:, None])

@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("E,I,K,counts,gather", [
    (4, 128, 256, [3, 0, 17, 1], True),
    (3, 256, 384, [70, 1, 129], False),
    (2, 384, 1024, [300, 33], True),                  # N = 768: a wide tile half past N
    (3, 128, 640, [200, 241, 0], True),
    (2, 256, 256, [1300, 9], False),                  # 6 M blocks in the tiled order's groups
])
def test_grouped_gemm_swiglu(E, I, K, counts, gather, algo, rng):
    w, s, offsets, a, sa, rows = _gemm_problem(rng, E, 2 * I, K, counts, src_rows=40 if gather else None)
    h = oracle.grouped_gemm(a, sa, rows, offsets, w, s)
    want = oracle.swiglu_f32(h)
    M = int(offsets[-1])
    say(f"grouped_gemm_swiglu E={E} I={I} K={K} counts={counts} gather={gather} algo={algo}")
    wb, sb = prepack_int4(w, s)
    act, pmax = ops.w4a8_moe_grouped_gemm_swiglu_prepacked(to_dev(a), to_dev(sa), None if rows is None else to_dev(rows),
                                                 to_dev(offsets), wb, sb, M, algo=algo)
    act, pmax = host(act), host(pmax)
    assert_float_parity(act, want, "grouped_gemm_swiglu", fro_tight=GEMM_FRO_TIGHT, maxrel=edge_shape_maxrel(I))
    _check_pmax(pmax, act)
    # the codes of the fused path against the unfused one on the same inputs
    out = ops.w4a8_moe_grouped_gemm_prepacked(to_dev(a), to_dev(sa), None if rows is None else to_dev(rows), to_dev(offsets),
                                    wb, sb, M, algo=algo)
    q_ref, s_ref = ops.w4a8_moe_swiglu(out)
    q, sq = ops.w4a8_moe_requant(to_dev(act), to_dev(pmax))
    q, sq, q_ref, s_ref = host(q), host(sq), host(q_ref), host(s_ref)
    assert np.allclose(sq, s_ref, rtol=1e-5, atol=0)
    diff = q != q_ref
    assert np.all(near_midpoint(want, s_ref, rel=1e-4)[diff]), f"{int(diff.sum())} codes differ off a midpoint"


@pytest.mark.parametrize("M,I", [(1, 128), (37, 256), (500, 2048), (7, 1152), (3, 8192), (2, 8320)])
def test_requant(M, I, rng):
    act = (rng.standard_normal((M, I)) * np.exp2(rng.integers(-6, 6, size=(M, 1)))).astype(np.float32)
    if M > 2:
        act[1] = 0.0                                   # zero row: scale 1, codes 0
    pmax = _pmax_of(act)
    say(f"requant M={M} I={I}")
    q, sq = ops.w4a8_moe_requant(to_dev(act), to_dev(pmax))
    q_ref, s_ref = oracle.quant_rows(act)
    assert np.array_equal(host(sq).view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(host(q), q_ref)


# ------------------------------------------------------------------ step 5
@pytest.mark.parametrize("M,I", [(1, 128), (37, 256), (500, 2048)])
def test_swiglu(M, I, rng):
    h = (rng.standard_normal((M, 2 * I)) * np.exp2(rng.integers(-4, 6, size=(M, 1)))).astype(np.float32)
    h[0, :4] = [0.0, -0.0, 80.0, -80.0]
    a32 = oracle.swiglu_f32(h)
    want_q, want_s = oracle.quant_rows(a32)
    say(f"swiglu M={M} I={I}")
    qa, sa = ops.w4a8_moe_swiglu(to_dev(h))
    gq, gs = host(qa), host(sa)
    assert np.all(np.abs(gs.astype(np.float64) - want_s) <= 1e-6 * want_s)
    diff = gq != want_q
    if diff.any():
        near = near_midpoint(a32, want_s)
        assert np.all(near[diff]), f"{int(diff.sum())} codes differ away from a rounding midpoint"
        assert diff.mean() < 1e-3


# ------------------------------------------------------------------ step 7
@pytest.mark.parametrize("T,k,H,dt", [(1, 1, 128, torch.float32), (37, 3, 384, torch.float32),
                                      (128, 8, 6144, torch.bfloat16), (64, 8, 256, torch.float32)])
def test_unpermute(T, k, H, dt, rng):
    o = rng.standard_normal((T * k, H)).astype(np.float32)
    inv = rng.permutation(T * k).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    want = oracle.unpermute(o, inv, w)
    say(f"unpermute T={T} k={k} H={H} {dt}")
    y32 = ops.w4a8_moe_unpermute(to_dev(o), to_dev(inv), to_dev(w))
    assert_float_parity(host(y32), want, "unpermute", fro_tight=1e-6)
    if dt == torch.bfloat16:
        # the bf16 output is the fp32 result rounded to nearest even (torch's CPU cast as the reference)
        yb = ops.w4a8_moe_unpermute(to_dev(o), to_dev(inv), to_dev(w), y_dtype=dt)
        assert np.array_equal(host(yb), _bits(host(y32)))
        assert_float_parity(oracle.bf16_bits_to_f32(host(yb)), want, "unpermute bf16")


@pytest.mark.parametrize("T,k,H", [(37, 3, 384), (200, 8, 1024)])
def test_unpermute_skips_unrouted(T, k, H, rng):
    """Routed indices the permutation left out (inv_pos = -1: ids out of range) contribute nothing: the
    oracle's step 7 with those weights set to zero (and any row index in their place)."""
    R = T * k
    unrouted = rng.random(R) < 0.1
    M = int((~unrouted).sum())
    inv = np.full(R, -1, np.int32)
    inv[~unrouted] = rng.permutation(M).astype(np.int32)
    o = rng.standard_normal((R, H)).astype(np.float32)      # rows M.. are never named
    w = rng.random((T, k)).astype(np.float32)
    w_zeroed = np.where(unrouted.reshape(T, k), np.float32(0), w)
    want = oracle.unpermute(o, np.maximum(inv, 0), w_zeroed)
    say(f"unpermute with {int(unrouted.sum())} unrouted indices T={T} k={k} H={H}")
    y = host(ops.w4a8_moe_unpermute(to_dev(o), to_dev(inv), to_dev(w)))
    assert_float_parity(y, want, "unpermute with unrouted indices", fro_tight=1e-6)


# -------------------------------------------------------------- whole layer
def _layer_vs_oracle(wl, algo=ops.W4A8_GG_AUTO, y_dtype=torch.float32, fused=True):
    sh = wl.shape
    maxrel_bar = edge_shape_maxrel(sh.H) if sh.name.startswith("custom") else 1e-2
    res = oracle.moe_layer(wl.x_bf16, wl.logits, wl.w13, wl.s13, wl.w2, wl.s2, k=sh.k)
    say(f"layer {sh.name} algo={algo} fused={fused}")
    moe = W4A8MoE(to_dev(wl.w13), to_dev(wl.s13), to_dev(wl.w2), to_dev(wl.s2), k=sh.k, fused=fused)
    y = moe(bf16_to_dev(wl.x_bf16), to_dev(wl.logits), algo=algo, y_dtype=y_dtype)
    b = moe.buffers(sh.T)
    assert np.array_equal(host(b["qx"]), res["qx"])
    assert np.array_equal(host(b["sx"]), res["sx"])
    assert np.array_equal(host(b["ids"]), res["ids"])
    assert np.all(np.abs(host(b["w"]).astype(np.float64) - res["w"]) <= 1e-6 * np.abs(res["w"]))
    for name in ("offsets", "row_token", "inv_pos"):
        assert np.array_equal(host(b[name]), res[name]), name
    if fused:
        act = host(b["act"])
        assert_float_parity(act, res["a_f32"], "gate/up + SwiGLU", fro_tight=GEMM_FRO_TIGHT)
        assert np.array_equal(host(b["pmax"]).max(axis=1), np.abs(act).max(axis=1)), "row maxima of act"
    else:
        assert_float_parity(host(b["h"]), res["h"], "gate/up", fro_tight=GEMM_FRO_TIGHT)
    yy = host(y)
    if y_dtype == torch.bfloat16:
        yy = oracle.bf16_bits_to_f32(yy)
    # the re-quantized codes: exact on the GPU's own act (recomputed from its h on the unfused
    # path), and where they differ from the independent run, explained by the act difference
    act_gpu = host(b["act"]) if fused else oracle.swiglu_f32(host(b["h"]))
    qa_gpu, sa_gpu = host(b["qa"]), host(b["sa"])
    flipped = check_requant(act_gpu, qa_gpu, sa_gpu, res["qa"], act_exact=fused)
    token_flipped = flipped.any(axis=1)[res["inv_pos"]].reshape(sh.T, sh.k).any(axis=1)
    o_same = oracle.grouped_gemm(qa_gpu, sa_gpu, None, res["offsets"], wl.w2, wl.s2)
    y_same = oracle.unpermute(o_same, res["inv_pos"], res["w"])
    if y_dtype == torch.bfloat16:
        # the bf16 output carries its own rounding (2^-9 relative): the per-element bars are its own
        fro = np.linalg.norm(yy - res["y"]) / np.linalg.norm(res["y"])
        assert fro <= 2e-3, fro
        r = assert_float_parity(yy, y_same, "layer output (bf16)", maxrel=maxrel_bar)
    else:
        r = check_layer_output(yy, res["y"], y_same, token_flipped, "layer output", maxrel=maxrel_bar)
    say(f"layer output vs oracle: {r}; {int(flipped.sum())} codes differ from the independent run")
    return moe, y, r


@pytest.mark.parametrize("algo", ALGOS)
def test_layer_unfused(algo):
    _layer_vs_oracle(workloads.make_custom(37, 384, 256, 5, 3, seed=21), algo=algo, fused=False)


@pytest.mark.parametrize("algo", ALGOS)
def test_layer_tiny(algo):
    _layer_vs_oracle(workloads.make_config(0), algo)


@pytest.mark.parametrize("T,H,I,E,k", [(37, 384, 256, 5, 3), (1, 256, 128, 8, 8), (64, 256, 128, 1, 1),
                                       (200, 256, 128, 4, 2), (130, 512, 384, 16, 4)])
def test_layer_shapes(T, H, I, E, k):
    wl = workloads.make_custom(T, H, I, E, k, seed=T * 1000 + E)
    for algo in ALGOS:
        _layer_vs_oracle(wl, algo)


def test_layer_all_tokens_one_expert():
    wl = workloads.make_custom(96, 256, 128, 6, 1, seed=5)
    wl.logits[:, 4] += 100.0
    _, _, _ = _layer_vs_oracle(wl, ops.W4A8_GG_TILED)
    _layer_vs_oracle(wl, ops.W4A8_GG_STREAM)


def test_layer_bf16_output_and_determinism():
    wl = workloads.make_config(0)
    moe, y32, _ = _layer_vs_oracle(wl)
    y_first = host(y32).copy()
    yb = moe(bf16_to_dev(wl.x_bf16), to_dev(wl.logits), y_dtype=torch.bfloat16)
    assert np.array_equal(host(yb), _bits(y_first))
    for _ in range(3):
        y2 = moe(bf16_to_dev(wl.x_bf16), to_dev(wl.logits))
        assert np.array_equal(host(y2), y_first)


def test_layer_zero_tokens():
    wl = workloads.make_config(0)
    moe = W4A8MoE(to_dev(wl.w13), to_dev(wl.s13), to_dev(wl.w2), to_dev(wl.s2), k=2)
    say("layer T=0")
    y = moe(torch.zeros((0, 256), dtype=torch.bfloat16, device="cuda:0"),
            torch.zeros((0, 8), dtype=torch.float32, device="cuda:0"))
    assert tuple(y.shape) == (0, 256)
    assert np.array_equal(host(moe.buffers(0)["offsets"]), np.zeros(9, np.int32))
