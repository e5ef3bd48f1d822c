"""GPU parity of the per-channel INT4 x per-token INT8 form at the full decode and prefill sizes.

The layer runs on the GPU as the benchmark runs it (automatic kernel choice,
prepacked experts, fused gate/up epilogue).  The oracle checks what it can
compute one by one: routing and the permutation for every token
(bit-exact); a sample of tokens end to end; and sampled routed rows of the
fused gate/up GEMM, the requant and the down GEMM (both kernels), with both
sides fed identical inputs.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import GEMM_FRO_TIGHT, assert_float_parity, bf16_to_dev, host, say, to_dev
from quantized_grouped_gemm_token_amd import ops, workloads
from quantized_grouped_gemm_token_amd.layer import W4A8MoEChannel

pytestmark = pytest.mark.gpu

_cache = {}


def _run(index):
    if index not in _cache:
        _cache.clear()
        torch.cuda.empty_cache()
        say(f"generate config {index} (per-channel INT8)")
        wl = workloads.make_config(index)
        s13, s2 = workloads.channel_scales(wl)
        moe = W4A8MoEChannel(to_dev(wl.w13), to_dev(s13), to_dev(wl.w2), to_dev(s2), k=wl.shape.k)
        say(f"forward {wl.shape.name} (per-channel INT8)")
        y = moe(bf16_to_dev(wl.x_bf16), to_dev(wl.logits))
        b = moe.buffers(wl.shape.T)
        got = {k: host(v) for k, v in b.items() if k != "workspace"}
        got["y"] = host(y)
        _cache[index] = (wl, (s13, s2), moe, got)
    return _cache[index]


def _sample_rows(offsets, rng, n_random=4):
    counts = np.diff(offsets)
    nonempty = np.nonzero(counts)[0]
    experts = {int(nonempty[0]), int(nonempty[-1]), int(np.argmax(counts))}
    experts.update(int(e) for e in rng.choice(nonempty, size=min(n_random, nonempty.size), replace=False))
    rows = set()
    for e in sorted(experts):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        rows.update({r0, r1 - 1, (r0 + r1) // 2})
    return np.array(sorted(rows), dtype=np.int64)


WORKLOADS = [1, 3]


@pytest.mark.parametrize("index", WORKLOADS)
def test_channel_routing_and_tokens(index):
    wl, (s13, s2), _, got = _run(index)
    ids, _ = oracle.route(wl.logits, wl.shape.k)
    offsets, row_token, inv_pos = oracle.permute(ids, wl.shape.E)
    assert np.array_equal(got["ids"], ids)
    assert np.array_equal(got["offsets"], offsets)
    assert np.array_equal(got["row_token"], row_token) and np.array_equal(got["inv_pos"], inv_pos)
    qx, sx, rx = oracle.quant_act_i8(wl.x_bf16)
    assert np.array_equal(got["qx"], qx) and np.array_equal(got["rx"], rx)
    assert np.array_equal(got["sx"].view(np.uint32), sx.view(np.uint32))
    T = wl.shape.T
    rng = np.random.Generator(np.random.PCG64(400 + index))
    sel = np.unique(np.concatenate([[0, T - 1], rng.integers(0, T, size=1)]))
    say(f"config {index}: per-channel oracle on tokens {sel.tolist()}")
    res = oracle.moe_layer_i8(wl.x_bf16[sel], wl.logits[sel], wl.w13, s13, wl.w2, s2, k=wl.shape.k)
    r = assert_float_parity(got["y"][sel], res["y"], f"config {index} per-channel output")
    say(f"config {index} per-channel output vs oracle: {r}")


@pytest.mark.parametrize("index", WORKLOADS)
def test_channel_sampled_rows_per_call(index):
    wl, (s13, s2), moe, got = _run(index)
    sh = wl.shape
    rng = np.random.Generator(np.random.PCG64(500 + index))
    offsets = got["offsets"]
    P = _sample_rows(offsets, rng)
    experts = np.searchsorted(offsets, P, side="right") - 1
    sub_off = np.zeros(sh.E + 1, np.int32)
    np.add.at(sub_off, experts + 1, 1)
    sub_off = np.cumsum(sub_off).astype(np.int32)
    qx, sx, _ = oracle.quant_act_i8(wl.x_bf16[got["row_token"][P]])
    say(f"config {index}: per-channel oracle gate/up on {P.size} rows")
    a32 = oracle.swiglu_f32(oracle.grouped_gemm_i8(qx, sx, None, sub_off, wl.w13, s13))
    assert_float_parity(got["act"][P], a32, f"config {index} per-channel gate/up + SwiGLU", fro_tight=GEMM_FRO_TIGHT)
    assert np.array_equal(got["pmax"][P].max(axis=1), np.abs(got["act"][P]).max(axis=1))
    qa, sa, ra = oracle.quant_rows_i8(a32)
    pm = np.abs(a32).reshape(a32.shape[0], -1, 64).max(axis=2).astype(np.float32)
    rq, rs, rr = ops.w4a8_moe_requant_i8(to_dev(a32), to_dev(pm))
    assert np.array_equal(host(rq), qa) and np.array_equal(host(rr), ra)
    assert np.array_equal(host(rs).view(np.uint32), sa.view(np.uint32))
    o = oracle.grouped_gemm_i8(qa, sa, None, sub_off, wl.w2, s2)
    for algo in (ops.W4A8_GG_STREAM, ops.W4A8_GG_TILED):
        say(f"config {index}: per-channel down GEMM on {P.size} oracle rows algo={algo}")
        go = ops.w4a8_moe_grouped_gemm_i8(to_dev(qa), to_dev(sa), to_dev(ra), None, to_dev(sub_off), moe.w2, moe.s2,
                                          M_total=P.size, algo=algo)
        assert_float_parity(host(go), o, f"config {index} per-channel down algo={algo}", fro_tight=GEMM_FRO_TIGHT)
