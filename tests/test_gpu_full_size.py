"""GPU parity at the full workload sizes (decode 128/256, prefill 8K, skewed 16K).

The layer runs on the GPU exactly as the benchmark runs it (automatic kernel
choice).  The oracle is too slow for every output at these sizes, so it is
run on what it can compute one by one:
  * routing and the permutation: every token, bit-exact;
  * FP8 activation codes and end-to-end outputs: a sample of tokens (the
    layer is token-local, so the oracle runs on those tokens alone);
  * each grouped GEMM, SwiGLU and the combine: a sample of routed rows
    chosen across the experts (first, middle and last rows of the first,
    last, hottest and some random experts), with both sides fed identical
    inputs.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import (GEMM_FRO_TIGHT, assert_float_parity, bf16_to_dev, host, near_midpoint, say, to_dev,
                      valid_code_choice)
from quantized_grouped_gemm_token_amd import ops, workloads
from quantized_grouped_gemm_token_amd.layer import W4A8MoE

pytestmark = pytest.mark.gpu

_cache = {}


def _run(index):
    """Workload + one GPU forward pass, kept for the tests of one config."""
    if index not in _cache:
        _cache.clear()
        torch.cuda.empty_cache()
        say(f"generate config {index}")
        wl = workloads.make_config(index)
        moe = W4A8MoE(to_dev(wl.w13), to_dev(wl.s13), to_dev(wl.w2), to_dev(wl.s2), k=wl.shape.k)
        x, lg = bf16_to_dev(wl.x_bf16), to_dev(wl.logits)
        say(f"forward {wl.shape.name}")
        y = moe(x, lg)
        b = moe.buffers(wl.shape.T)
        got = {k: host(v) for k, v in b.items() if k != "workspace"}
        got["y"] = host(y)
        _cache[index] = (wl, moe, got)
    return _cache[index]


def _sample_rows(offsets, rng, per_expert=3, n_random=4):
    counts = np.diff(offsets)
    nonempty = np.nonzero(counts)[0]
    experts = {int(nonempty[0]), int(nonempty[-1]), int(np.argmax(counts))}
    experts.update(int(e) for e in rng.choice(nonempty, size=min(n_random, nonempty.size), replace=False))
    rows = set()
    for e in sorted(experts):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        rows.update({r0, r1 - 1, (r0 + r1) // 2})
        if r1 - r0 > 300:            # deep inside a large expert (M tiling)
            rows.update(int(r) for r in rng.integers(r0, r1, size=per_expert))
    return np.array(sorted(rows), dtype=np.int64)


WORKLOADS = [1, 2, 3, 4]


@pytest.mark.parametrize("index", WORKLOADS)
def test_routing_and_permutation(index):
    wl, _, got = _run(index)
    ids, w = oracle.route(wl.logits, wl.shape.k)
    assert np.array_equal(got["ids"], ids)
    assert np.all(np.abs(got["w"].astype(np.float64) - w) <= 1e-6 * np.abs(w))
    offsets, row_token, inv_pos = oracle.permute(ids, wl.shape.E)
    assert np.array_equal(got["offsets"], offsets)
    assert np.array_equal(got["row_token"], row_token)
    assert np.array_equal(got["inv_pos"], inv_pos)
    counts = np.diff(offsets)
    say(f"config {index}: touched {int((counts > 0).sum())} experts, max rows {int(counts.max())}, "
        f"empty {int((counts == 0).sum())}")
    if index == 4:
        assert (counts == 0).sum() >= 1                    # skew leaves some experts empty


@pytest.mark.parametrize("index", WORKLOADS)
def test_sampled_tokens_end_to_end(index):
    wl, _, got = _run(index)
    T = wl.shape.T
    rng = np.random.Generator(np.random.PCG64(index))
    sel = np.unique(np.concatenate([[0, T - 1], rng.integers(0, T, size=2)]))
    res = oracle.moe_layer(wl.x_bf16[sel], wl.logits[sel], wl.w13, wl.s13, wl.w2, wl.s2, k=wl.shape.k)
    assert np.array_equal(got["qx"][sel], res["qx"])
    assert np.array_equal(got["sx"][sel], res["sx"])
    k = wl.shape.k
    # GPU routed rows of these tokens, in the oracle sub-run's row order
    gpu_rows = np.empty(sel.size * k, np.int64)
    for i, t in enumerate(sel):
        for j in range(k):
            gpu_rows[res["inv_pos"][i * k + j]] = got["inv_pos"][t * k + j]
    codes, flips = valid_code_choice(res["a_f32"], res["sa"], res["qa"], got["qa"][gpu_rows])
    assert flips <= max(2, 1e-2 * codes.size), flips
    o_ref = oracle.grouped_gemm(codes, res["sa"], None, res["offsets"], wl.w2, wl.s2)
    y_ref = oracle.unpermute(o_ref, res["inv_pos"], res["w"])
    fro_own = np.linalg.norm(got["y"][sel] - res["y"]) / np.linalg.norm(res["y"])
    assert fro_own <= 2e-3, fro_own
    r = assert_float_parity(got["y"][sel], y_ref, f"config {index} output")
    say(f"config {index} output vs oracle: fro {fro_own:.2e}; {flips} midpoint code choices; vs matching "
        f"reference {r}")
    # the combine alone, on the oracle's own expert outputs of these tokens
    say(f"config {index}: unpermute on oracle rows")
    y = ops.w4a8_moe_unpermute(to_dev(res["o"]), to_dev(res["inv_pos"]), to_dev(res["w"]))
    assert_float_parity(host(y), res["y"], "unpermute", fro_tight=1e-6)


@pytest.mark.parametrize("index", WORKLOADS)
def test_sampled_rows_per_call(index):
    wl, moe, got = _run(index)
    sh = wl.shape
    rng = np.random.Generator(np.random.PCG64(100 + index))
    offsets = got["offsets"]                     # equal to the oracle's (checked above)
    P = _sample_rows(offsets, rng)
    experts = np.searchsorted(offsets, P, side="right") - 1
    sub_off = np.zeros(sh.E + 1, np.int32)
    np.add.at(sub_off, experts + 1, 1)
    sub_off = np.cumsum(sub_off).astype(np.int32)
    tokens = got["row_token"][P]
    qx, sx = oracle.quant_act(wl.x_bf16[tokens])
    # gate/up GEMM: GPU rows P of the full run vs the oracle on those rows
    h = oracle.grouped_gemm(qx, sx, None, sub_off, wl.w13, wl.s13)
    a32 = oracle.swiglu_f32(h)
    # the layer runs the gate/up GEMM with SwiGLU fused into its epilogue
    assert_float_parity(got["act"][P], a32, f"config {index} gate/up + SwiGLU", fro_tight=GEMM_FRO_TIGHT)
    assert np.array_equal(got["pmax"][P].max(axis=1), np.abs(got["act"][P]).max(axis=1))
    qa, sa = oracle.quant_rows(a32)
    # the fused path's requant on the oracle's activations: bit-exact
    pm = np.abs(a32).reshape(a32.shape[0], -1, 64).max(axis=2).astype(np.float32)
    rq, rs = ops.w4a8_moe_requant(to_dev(a32), to_dev(pm))
    assert np.array_equal(host(rq), qa) and np.array_equal(host(rs).view(np.uint32), sa.view(np.uint32))
    # the unfused gate/up GEMM on the sampled rows, both kernels
    for algo in (ops.W4A8_GG_STREAM, ops.W4A8_GG_TILED):
        say(f"config {index}: gate/up GEMM on {P.size} rows algo={algo}")
        gh = ops.w4a8_moe_grouped_gemm_prepacked(to_dev(qx), to_dev(sx), None, to_dev(sub_off), moe.w13, moe.s13, P.size,
                                       algo=algo)
        assert_float_parity(host(gh), h, f"config {index} gate/up algo={algo}", fro_tight=GEMM_FRO_TIGHT)
    # SwiGLU on the oracle's h
    say(f"config {index}: swiglu on {P.size} oracle rows")
    gq, gs = ops.w4a8_moe_swiglu(to_dev(h))
    gq, gs = host(gq), host(gs)
    assert np.all(np.abs(gs.astype(np.float64) - sa) <= 1e-6 * sa)
    diff = gq != qa
    assert np.all(near_midpoint(a32, sa)[diff])
    # down GEMM on the oracle's codes, with both kernels
    o = oracle.grouped_gemm(qa, sa, None, sub_off, wl.w2, wl.s2)
    for algo in (ops.W4A8_GG_STREAM, ops.W4A8_GG_TILED):
        say(f"config {index}: down GEMM on {P.size} oracle rows algo={algo}")
        go = ops.w4a8_moe_grouped_gemm_prepacked(to_dev(qa), to_dev(sa), None, to_dev(sub_off), moe.w2, moe.s2, P.size,
                                       algo=algo)
        assert_float_parity(host(go), o, f"config {index} down algo={algo}", fro_tight=GEMM_FRO_TIGHT)
