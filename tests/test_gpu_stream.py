"""The library enqueues on the caller's stream (torch's current stream).

A bounded spin kernel keeps the default stream busy while a layer step runs
on a side stream: the step must finish before the spin does (it never waits
on the default stream), and its result must equal the default-stream step's,
bit for bit.
"""
from __future__ import annotations

import pytest
import torch

from gpu_util import bf16_to_dev, say, to_dev
from quantized_grouped_gemm_token_amd import workloads
from quantized_grouped_gemm_token_amd.layer import W4A8MoE, W4A8MoEChannel, W4A8MoEMxfp4

pytestmark = pytest.mark.gpu

SPIN_CYCLES = 400_000_000      # a few hundred ms of one spinning wave on the default stream


def _layer(wl, scheme):
    sh = wl.shape
    if scheme == "g128":
        return W4A8MoE(to_dev(wl.w13), to_dev(wl.s13), to_dev(wl.w2), to_dev(wl.s2), k=sh.k)
    if scheme == "channel":
        s13, s2 = workloads.channel_scales(wl)
        return W4A8MoEChannel(to_dev(wl.w13), to_dev(s13), to_dev(wl.w2), to_dev(s2), k=sh.k)
    w13, s13, w2, s2 = workloads.mxfp4_weights(wl)
    return W4A8MoEMxfp4(to_dev(w13), to_dev(s13), to_dev(w2), to_dev(s2), k=sh.k)


@pytest.mark.parametrize("scheme", ["g128", "channel", "mxfp4"])
def test_layer_on_side_stream(scheme):
    if not hasattr(torch.cuda, "_sleep"):
        pytest.skip("torch.cuda._sleep is not available")
    wl = workloads.make_custom(64, 512, 256, 8, 4, seed=43)
    say(f"side stream {scheme} {wl.shape.name}")
    moe = _layer(wl, scheme)
    x, logits = bf16_to_dev(wl.x_bf16), to_dev(wl.logits)
    y_ref = moe(x, logits).clone()
    torch.cuda.synchronize()

    side = torch.cuda.Stream()                     # default priority
    y = torch.empty_like(y_ref)
    with torch.cuda.stream(side):
        moe(x, logits, y)                          # warm-up on the side stream (buffers, first launches)
    side.synchronize()
    y.zero_()
    torch.cuda.synchronize()

    torch.cuda._sleep(SPIN_CYCLES)                 # the default stream is busy from here
    with torch.cuda.stream(side):
        moe(x, logits, y)
        y_host = y.to("cpu", non_blocking=False)   # a copy ordered on the side stream
    side.synchronize()
    still_spinning = not torch.cuda.default_stream().query()
    torch.cuda.synchronize()
    assert still_spinning, "the side-stream step waited for the default stream"
    assert torch.equal(y_host, y_ref.cpu())
