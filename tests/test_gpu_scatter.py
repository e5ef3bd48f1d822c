"""GPU parity of step 7 done as a scatter from the down GEMM, called through the C-ABI.

The routing-weighted combine of the layer's last step, y[t] = sum_j w[t, j]
o[inv_pos[t k + j]] ("从 755GB 到 395GB", section 我们量化了什么: each token's
expert outputs are weighted by its gate weights and summed), taken in three
calls: row_sources inverts the permutation and folds w[t, j] into the down
GEMM's token scales, the scatter GEMM stores each row p at its routed index
f = t k + j, and combine sums each token's k contiguous rows.

  * row_sources: exact (an inverse permutation and one fp32 product per row);
  * the scatter GEMMs: row f of their output is, bit for bit, row p of the
    plain GEMM on the same codes with the same token scales (both kernels,
    all three weight forms), rows no routed index names stay untouched, and
    the rows match the oracle's GEMM;
  * combine: the oracle's step 7 with unit weights (zero for unrouted j);
  * the layer on this path: the oracle's end-to-end bars, all three forms.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_util import (GEMM_FRO_TIGHT, assert_float_parity, bf16_to_dev, check_layer_output, check_requant,
                      edge_shape_maxrel, host, prepack_int4, say, to_dev)
from oracle import mxfp4_oracle as mx
from quantized_grouped_gemm_token_amd import ops, workloads
from quantized_grouped_gemm_token_amd.layer import W4A8MoE, W4A8MoEChannel, W4A8MoEMxfp4

pytestmark = pytest.mark.gpu

ALGOS = (ops.W4A8_GG_STREAM, ops.W4A8_GG_TILED, ops.W4A8_GG_AUTO)
SENTINEL = np.float32(-1.2345e30)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert ops.w4a8_moe_device_supported(), "the current device is not a gfx950"
    yield
    torch.cuda.synchronize()


def _routing(rng, T, k, unrouted=0.0):
    """inv_pos [T k] mapping each routed index to a distinct row of [0, M_total) (-1 where the
    index is not routed), and gate weights w [T, k]."""
    R = T * k
    routed = rng.random(R) >= unrouted
    M = int(routed.sum())
    inv = np.full(R, -1, np.int32)
    inv[routed] = rng.permutation(M).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32) + np.float32(0.05)
    return inv, w, M


# ------------------------------------------------------------------ row sources
@pytest.mark.parametrize("T,k,unrouted", [(1, 1, 0.0), (37, 3, 0.0), (128, 8, 0.0), (300, 8, 0.2),
                                          (1000, 8, 0.05), (5, 2, 1.0)])
def test_row_sources(T, k, unrouted, rng):
    inv, w, M = _routing(rng, T, k, unrouted)
    sa = rng.lognormal(-3, 1, size=max(M, 1)).astype(np.float32)
    say(f"row_sources T={T} k={k} M={M}")
    src, scale = ops.w4a8_moe_row_sources(to_dev(inv), to_dev(w), to_dev(sa), M)
    src, scale = host(src)[:M], host(scale)[:M]
    f = np.flatnonzero(inv >= 0)
    want_src = np.empty(M, np.int32)
    want_src[inv[f]] = f
    assert np.array_equal(src, want_src)
    # one fp32 product per row: numpy's float32 multiply rounds the same way
    want_scale = sa[:M] * w.reshape(-1)[want_src]
    assert np.array_equal(scale.view(np.uint32), want_scale.astype(np.float32).view(np.uint32))


# ------------------------------------------------------------------ scatter GEMMs
def _g128_problem(rng, E, N, K, counts):
    w = rng.integers(0, 2**32, size=(E, N, K // 8), dtype=np.uint32).view(np.int32)
    s = rng.lognormal(-4, 0.5, size=(E, N, K // 128)).astype(np.float32)
    return w, s


def _scatter_case(rng, counts, K, i8):
    M = int(np.sum(counts))
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    x = rng.standard_normal((M, K)).astype(np.float32) * np.exp2(rng.integers(-3, 3, size=(M, 1)))
    if i8:
        a, sa = oracle.quant_rows_i8(x)
    else:
        a, sa = oracle.quant_rows(x)
    # destinations: a permutation of M rows into a larger output (rows left over stay untouched)
    R = M + 11
    dst = rng.permutation(R)[:M].astype(np.int32)
    return a, sa, offsets, dst, R


@pytest.mark.parametrize("form", ["g128", "channel", "mxfp4"])
@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("E,N,K,counts", [
    (4, 256, 256, [3, 0, 17, 1]),                   # one-block stream kernel
    (3, 320, 384, [70, 1, 129]),                    # ragged tiles, N not a multiple of 256
    (8, 256, 384, [9, 40, 0, 3, 1, 0, 2, 5]),       # AUTO: the tiled kernel runs
    (6, 256, 256, [64, 65, 33, 16, 0, 2]),          # multi-block stream kernel
    (3, 768, 256, [1400, 5, 300]),                  # several M blocks per expert (11 wide)
    (3, 768, 256, [1500, 5, 300]),                  # 6 square M blocks
])
def test_grouped_gemm_scatter(form, E, N, K, counts, algo, rng):
    a, sa, offsets, dst, R = _scatter_case(rng, counts, K, form == "channel")
    M = int(offsets[-1])
    say(f"grouped_gemm_scatter {form} E={E} N={N} K={K} counts={counts} algo={algo}")
    out = torch.full((R, N), float(SENTINEL), dtype=torch.float32, device="cuda:0")
    if form == "g128":
        w, s = _g128_problem(rng, E, N, K, counts)
        wb, sb = prepack_int4(w, s)
        plain = ops.w4a8_moe_grouped_gemm_prepacked(to_dev(a), to_dev(sa), None, to_dev(offsets), wb, sb, M,
                                                    algo=algo)
        ops.w4a8_moe_grouped_gemm_scatter_prepacked(to_dev(a), to_dev(sa), None, to_dev(offsets), wb, sb, M,
                                                    to_dev(dst), out, algo=algo)
        want = oracle.grouped_gemm(a, sa, None, offsets, w, s)
    elif form == "channel":
        w = rng.integers(0, 2**32, size=(E, N, K // 8), dtype=np.uint32).view(np.int32)
        ws = rng.lognormal(-4, 0.5, size=(E, N)).astype(np.float32)
        rowsum = oracle.code_row_sums(a)
        wb = prepack_int4(w)[0]
        plain = ops.w4a8_moe_grouped_gemm_i8_prepacked(to_dev(a), to_dev(sa), to_dev(rowsum), None, to_dev(offsets),
                                                       wb, to_dev(ws), M_total=M, algo=algo)
        ops.w4a8_moe_grouped_gemm_scatter_i8_prepacked(to_dev(a), to_dev(sa), to_dev(rowsum), None, to_dev(offsets),
                                                       wb, to_dev(ws), M, to_dev(dst), out, algo=algo)
        want = oracle.grouped_gemm_i8(a, sa, None, offsets, w, ws)
    else:
        w = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
        s = rng.integers(118, 136, size=(E, N, K // 32)).astype(np.uint8)
        wb, sb = ops.w4a8_moe_prepack_mxfp4(to_dev(w), to_dev(s))
        plain = ops.w4a8_moe_grouped_gemm_mxfp4_prepacked(to_dev(a), to_dev(sa), None, to_dev(offsets), wb, sb, M,
                                                          algo=algo)
        ops.w4a8_moe_grouped_gemm_scatter_mxfp4_prepacked(to_dev(a), to_dev(sa), None, to_dev(offsets), wb, sb, M,
                                                          to_dev(dst), out, algo=algo)
        want = mx.grouped_gemm_mxfp4(a, sa, None, offsets, w, s)
    got = host(out)
    assert np.array_equal(got[dst].view(np.uint32), host(plain).view(np.uint32)), "scatter rows != plain rows"
    untouched = np.setdiff1d(np.arange(R), dst)
    assert np.all(got[untouched].view(np.uint32) == SENTINEL.view(np.uint32)), "a row no index names was written"
    if form == "channel":
        zero = want == 0
        assert np.all(got[dst][zero] == 0)
        rel = np.abs(got[dst][~zero].astype(np.float64) - want[~zero]) / np.abs(want[~zero].astype(np.float64))
        assert rel.max(initial=0.0) <= 1e-6, rel.max()
    else:
        assert_float_parity(got[dst], want, f"scatter {form}", fro_tight=GEMM_FRO_TIGHT, maxrel=edge_shape_maxrel(N))


def test_grouped_gemm_scatter_empty():
    out = torch.zeros((4, 256), dtype=torch.float32, device="cuda:0")
    dst = torch.zeros((1,), dtype=torch.int32, device="cuda:0")
    a = torch.zeros((1, 256), dtype=torch.uint8, device="cuda:0")
    sa = torch.ones((1,), dtype=torch.float32, device="cuda:0")
    offsets = torch.zeros((3,), dtype=torch.int32, device="cuda:0")
    wb, sb = prepack_int4(np.zeros((2, 256, 32), np.int32), np.ones((2, 256, 2), np.float32))
    say("grouped_gemm_scatter M_total=0")
    ops.w4a8_moe_grouped_gemm_scatter_prepacked(a, sa, None, offsets, wb, sb, 0, dst, out)
    torch.cuda.synchronize()
    assert not out.any()


# ------------------------------------------------------------------ combine
@pytest.mark.parametrize("T,k,H,unrouted", [(1, 1, 128, 0.0), (37, 3, 384, 0.0), (128, 8, 6144, 0.0),
                                            (64, 8, 256, 0.3), (300, 10, 1152, 0.1), (9, 2, 128, 1.0)])
def test_combine(T, k, H, unrouted, rng):
    inv, _, _ = _routing(rng, T, k, unrouted)
    o_tok = rng.standard_normal((T * k, H)).astype(np.float32)
    # the oracle's step 7 on rows in routed order, unit weights, zero weight where unrouted
    o_perm = np.zeros_like(o_tok)
    routed = inv >= 0
    o_perm[inv[routed]] = o_tok[routed]
    want = oracle.unpermute(o_perm, np.maximum(inv, 0), routed.reshape(T, k).astype(np.float32))
    say(f"combine T={T} k={k} H={H} unrouted={unrouted}")
    y = host(ops.w4a8_moe_combine(to_dev(o_tok), to_dev(inv), T, k))
    assert_float_parity(y, want, "combine", fro_tight=1e-6)
    if unrouted == 1.0:
        assert not y.any()
    yb = host(ops.w4a8_moe_combine(to_dev(o_tok), to_dev(inv), T, k, y_dtype=torch.bfloat16))
    assert np.array_equal(yb, oracle.f32_to_bf16_bits(y))


# ------------------------------------------------------------------ the layer
def _layer(wl, scheme, scatter):
    sh = wl.shape
    if scheme == "g128":
        return W4A8MoE(to_dev(wl.w13), to_dev(wl.s13), to_dev(wl.w2), to_dev(wl.s2), k=sh.k, scatter=scatter)
    if scheme == "channel":
        s13, s2 = workloads.channel_scales(wl)
        return W4A8MoEChannel(to_dev(wl.w13), to_dev(s13), to_dev(wl.w2), to_dev(s2), k=sh.k, scatter=scatter)
    w13, s13, w2, s2 = workloads.mxfp4_weights(wl)
    return W4A8MoEMxfp4(to_dev(w13), to_dev(s13), to_dev(w2), to_dev(s2), k=sh.k, scatter=scatter)


def _oracle_layer(wl, scheme):
    """The independent oracle run, and its down GEMM as a function of the GPU's re-quantized rows."""
    sh = wl.shape
    if scheme == "g128":
        res = oracle.moe_layer(wl.x_bf16, wl.logits, wl.w13, wl.s13, wl.w2, wl.s2, k=sh.k)
        return res, lambda qa, sa: oracle.grouped_gemm(qa, sa, None, res["offsets"], wl.w2, wl.s2)
    if scheme == "channel":
        s13, s2 = workloads.channel_scales(wl)
        res = oracle.moe_layer_i8(wl.x_bf16, wl.logits, wl.w13, s13, wl.w2, s2, k=sh.k)
        return res, lambda qa, sa: oracle.grouped_gemm_i8(qa, sa, None, res["offsets"], wl.w2, s2)
    w13, s13, w2, s2 = workloads.mxfp4_weights(wl)
    res = mx.moe_layer_mxfp4(wl.x_bf16, wl.logits, w13, s13, w2, s2, k=sh.k)
    return res, lambda qa, sa: mx.grouped_gemm_mxfp4(qa, sa, None, res["offsets"], w2, s2)


@pytest.mark.parametrize("scheme", ["g128", "channel", "mxfp4"])
@pytest.mark.parametrize("case", ["tiny", "mid", "wide"])
def test_layer_scatter(scheme, case):
    wl = {"tiny": lambda: workloads.make_config(0),
          "mid": lambda: workloads.make_custom(300, 1024, 256, 16, 4, seed=43),
          "wide": lambda: workloads.make_custom(600, 512, 384, 8, 8, seed=44)}[case]()
    sh = wl.shape
    res, down = _oracle_layer(wl, scheme)
    x, logits = bf16_to_dev(wl.x_bf16), to_dev(wl.logits)
    for algo in ALGOS:
        say(f"layer scatter {scheme} {sh.name} algo={algo}")
        moe = _layer(wl, scheme, scatter=True)
        assert moe.uses_scatter(sh.T)
        y = host(moe(x, logits, algo=algo))
        b = moe.buffers(sh.T)
        for name in ("offsets", "row_token", "inv_pos"):
            assert np.array_equal(host(b[name]), res[name]), name
        act_gpu, qa_gpu, sa_gpu = host(b["act"]), host(b["qa"]), host(b["sa"])
        flipped = check_requant(act_gpu, qa_gpu, sa_gpu, res["qa"], int8=scheme == "channel", act_exact=True)
        token_flipped = flipped.any(axis=1)[res["inv_pos"]].reshape(sh.T, sh.k).any(axis=1)
        y_same = oracle.unpermute(down(qa_gpu, sa_gpu), res["inv_pos"], res["w"])
        maxrel_bar = edge_shape_maxrel(sh.H) if sh.name.startswith("custom") else 1e-2
        r = check_layer_output(y, res["y"], y_same, token_flipped, f"layer scatter {scheme}", maxrel=maxrel_bar)
        say(f"layer scatter output vs oracle: {r}")
        # the gather path on the same layer: the same sums, rounded in another order
        gather = _layer(wl, scheme, scatter=False)
        y_g = host(gather(x, logits, algo=algo))
        assert_float_parity(y, y_g, "scatter vs gather combine", fro_tight=1e-6)
        # deterministic: the same bits on every run, and bf16 output = the fp32 result rounded
        assert np.array_equal(host(moe(x, logits, algo=algo)), y)
        yb = host(moe(x, logits, algo=algo, y_dtype=torch.bfloat16))
        assert np.array_equal(yb, oracle.f32_to_bf16_bits(y))


@pytest.mark.parametrize("scheme", ["g128", "mxfp4"])
def test_layer_scatter_graph_replay(scheme):
    wl = workloads.make_custom(300, 1024, 256, 16, 4, seed=45)
    sh = wl.shape
    say(f"graph replay scatter {scheme} {sh.name}")
    moe = _layer(wl, scheme, scatter=True)
    x, logits = bf16_to_dev(wl.x_bf16), to_dev(wl.logits)
    rng = np.random.Generator(np.random.PCG64(8))
    x2 = (torch.from_numpy(rng.standard_normal(tuple(x.shape)).astype(np.float32)).to(x.device) * 3).to(torch.bfloat16)
    logits2 = torch.from_numpy(rng.standard_normal(tuple(logits.shape)).astype(np.float32)).to(x.device)
    y_eager = moe(x, logits).clone()
    torch.cuda.synchronize()
    y = torch.empty_like(y_eager)
    g = moe.capture(x, logits, y)
    for i in range(3):
        moe(x2, logits2)
        torch.cuda.synchronize()
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), f"replay {i} differs from the eager step"


@pytest.mark.parametrize("form", ["g128", "channel", "mxfp4"])
@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("E,N,K,counts,src_rows", [
    (4, 256, 256, [3, 0, 17, 1], 9),                # gathered rows (a_rows), one-block stream kernel
    (3, 320, 384, [70, 1, 129], 40),                # gathered rows, ragged tiles
    (1, 64, 128, [1], 1),                           # one row
    (1024, 128, 128, [1 if e % 97 == 0 else 0 for e in range(1023)] + [40], 30),   # 1024 experts, 11 used
])
def test_grouped_gemm_scatter_gather_and_edges(form, E, N, K, counts, src_rows, algo, rng):
    """The scatter forms with gathered activation rows (row p of A is a[a_rows[p]]), a single row and the
    most experts: rows bit-identical to the plain GEMM's at their destinations."""
    M = int(np.sum(counts))
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    x = rng.standard_normal((src_rows, K)).astype(np.float32)
    a, sa = oracle.quant_rows_i8(x) if form == "channel" else oracle.quant_rows(x)
    rows = rng.integers(0, src_rows, size=M).astype(np.int32)
    R = M + 5
    dst = rng.permutation(R)[:M].astype(np.int32)
    out = torch.full((R, N), float(SENTINEL), dtype=torch.float32, device="cuda:0")
    say(f"scatter gather/edges {form} E={E} N={N} K={K} M={M} algo={algo}")
    if form == "g128":
        w = rng.integers(0, 2**32, size=(E, N, K // 8), dtype=np.uint32).view(np.int32)
        s = rng.lognormal(-4, 0.5, size=(E, N, K // 128)).astype(np.float32)
        wb, sb = prepack_int4(w, s)
        plain = ops.w4a8_moe_grouped_gemm_prepacked(to_dev(a), to_dev(sa), to_dev(rows), to_dev(offsets), wb, sb, M,
                                                    algo=algo)
        ops.w4a8_moe_grouped_gemm_scatter_prepacked(to_dev(a), to_dev(sa), to_dev(rows), to_dev(offsets), wb, sb, M,
                                                    to_dev(dst), out, algo=algo)
    elif form == "channel":
        w = rng.integers(0, 2**32, size=(E, N, K // 8), dtype=np.uint32).view(np.int32)
        ws = rng.lognormal(-4, 0.5, size=(E, N)).astype(np.float32)
        rowsum = oracle.code_row_sums(a)
        wb = prepack_int4(w)[0]
        plain = ops.w4a8_moe_grouped_gemm_i8_prepacked(to_dev(a), to_dev(sa), to_dev(rowsum), to_dev(rows),
                                                       to_dev(offsets), wb, to_dev(ws), M_total=M, algo=algo)
        ops.w4a8_moe_grouped_gemm_scatter_i8_prepacked(to_dev(a), to_dev(sa), to_dev(rowsum), to_dev(rows),
                                                       to_dev(offsets), wb, to_dev(ws), M, to_dev(dst), out,
                                                       algo=algo)
    else:
        w = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
        s = rng.integers(118, 136, size=(E, N, K // 32)).astype(np.uint8)
        wb, sb = ops.w4a8_moe_prepack_mxfp4(to_dev(w), to_dev(s))
        plain = ops.w4a8_moe_grouped_gemm_mxfp4_prepacked(to_dev(a), to_dev(sa), to_dev(rows), to_dev(offsets), wb,
                                                          sb, M, algo=algo)
        ops.w4a8_moe_grouped_gemm_scatter_mxfp4_prepacked(to_dev(a), to_dev(sa), to_dev(rows), to_dev(offsets), wb,
                                                          sb, M, to_dev(dst), out, algo=algo)
    got = host(out)
    assert np.array_equal(got[dst].view(np.uint32), host(plain).view(np.uint32))
    untouched = np.setdiff1d(np.arange(R), dst)
    assert np.all(got[untouched].view(np.uint32) == SENTINEL.view(np.uint32))
