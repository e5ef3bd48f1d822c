"""The threaded layer of tests/oracle_par.py equals the oracle's own layers bit for bit."""
import numpy as np
import pytest

import oracle
import oracle_par
from oracle import mxfp4_oracle as mx
from quantized_grouped_gemm_token_amd import workloads


def _weights(wl, form):
    if form == "g128":
        return wl.w13, wl.s13, wl.w2, wl.s2
    if form == "channel":
        s13, s2 = workloads.channel_scales(wl)
        return wl.w13, s13, wl.w2, s2
    return workloads.mxfp4_weights(wl)


@pytest.mark.parametrize("form", ["g128", "channel", "mxfp4"])
@pytest.mark.parametrize("shape", [(0, None), (-1, (48, 512, 256, 12, 4))])
def test_threaded_layer_equals_oracle(form, shape):
    index, custom = shape
    wl = workloads.make_config(0) if custom is None else workloads.make_custom(*custom, seed=77)
    w13, s13, w2, s2 = _weights(wl, form)
    ref_fn = {"g128": oracle.moe_layer, "channel": oracle.moe_layer_i8, "mxfp4": mx.moe_layer_mxfp4}[form]
    ref = ref_fn(wl.x_bf16, wl.logits, w13, s13, w2, s2, k=wl.shape.k)
    got = oracle_par.layer(form, wl.x_bf16, wl.logits, w13, s13, w2, s2, k=wl.shape.k)
    for name in ("qx", "sx", "ids", "w", "offsets", "row_token", "inv_pos", "h", "a_f32", "qa", "sa", "o", "y"):
        assert np.array_equal(np.asarray(got[name]).view(np.uint8), np.asarray(ref[name]).view(np.uint8)), name


def test_expert_subset_leaves_other_rows_zero():
    wl = workloads.make_custom(40, 256, 128, 6, 2, seed=3)
    qx, sx = oracle.quant_act(wl.x_bf16)
    ids, _ = oracle.route(wl.logits, 2)
    offsets, row_token, _ = oracle.permute(ids, 6)
    full = oracle.grouped_gemm(qx, sx, row_token, offsets, wl.w13, wl.s13)
    part = oracle_par.gemm_experts("g128", qx, sx, row_token, offsets, wl.w13, wl.s13, experts=[1, 4])
    for e in range(6):
        r0, r1 = offsets[e], offsets[e + 1]
        if e in (1, 4):
            assert np.array_equal(part[r0:r1], full[r0:r1])
        else:
            assert not part[r0:r1].any()
