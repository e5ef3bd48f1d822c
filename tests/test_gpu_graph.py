"""A layer step captured into a HIP graph, replayed, against the eager step.

Each replay is preceded by eager work on other inputs (which overwrites the
buffers the graph shares) and a synchronization, and every replay must give
the eager result bit for bit: every kernel of the step is deterministic.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from gpu_util import bf16_to_dev, say, to_dev
from quantized_grouped_gemm_token_amd import workloads
from quantized_grouped_gemm_token_amd.layer import W4A8MoE, W4A8MoEChannel, W4A8MoEMxfp4

pytestmark = pytest.mark.gpu


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
@pytest.mark.parametrize("shape", ["tiny", "mid"])
def test_graph_replay_matches_eager(scheme, shape):
    wl = workloads.make_config(0) if shape == "tiny" else workloads.make_custom(300, 1024, 256, 16, 4, seed=41)
    sh = wl.shape
    say(f"graph replay {scheme} {sh.name}")
    moe = _layer(wl, scheme)
    x, logits = bf16_to_dev(wl.x_bf16), to_dev(wl.logits)
    rng = np.random.Generator(np.random.PCG64(7))
    x2 = (torch.from_numpy(rng.standard_normal(tuple(x.shape)).astype(np.float32)).to(x.device) * 3).to(torch.bfloat16)
    logits2 = torch.from_numpy(rng.standard_normal(tuple(logits.shape)).astype(np.float32)).to(x.device)
    y_eager = moe(x, logits).clone()
    y2_eager = moe(x2, logits2).clone()
    torch.cuda.synchronize()
    y = torch.empty_like(y_eager)
    g = moe.capture(x, logits, y)
    for i in range(3):
        moe(x2, logits2)                      # eager work on the shared buffers between replays
        torch.cuda.synchronize()
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), f"replay {i} differs from the eager step"
    # a replay reads the tensors' current contents
    x.copy_(x2)
    logits.copy_(logits2)
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(y, y2_eager)


@pytest.mark.parametrize("scheme", ["g128", "channel", "mxfp4"])
def test_graph_follows_the_routing(scheme):
    """The automatic kernel choice is taken on the device, so one captured graph serves batches that
    call for either kernel: captured on uniform routing (a few rows per expert: the streaming kernel
    runs), replayed on routing that sends 100 tokens to one expert (the tiled kernel runs), and back.
    Before each replay an eager step on the other batch leaves its values in every shared buffer, so a
    replay in which neither kernel ran would not give the expected output."""
    wl = workloads.make_custom(128, 512, 256, 64, 2, seed=61)
    say(f"graph follows the routing {scheme}")
    moe = _layer(wl, scheme)
    x, logits = bf16_to_dev(wl.x_bf16), to_dev(wl.logits)
    skew = logits.clone()
    skew[:100, 5] += 100.0                      # expert 5: 100 rows, past the streaming kernel's 32
    uniform = logits.clone()
    y_uni = moe(x, uniform).clone()
    y_skew = moe(x, skew).clone()
    torch.cuda.synchronize()
    assert not torch.equal(y_uni, y_skew)
    counts = torch.diff(moe.buffers(128)["offsets"]).cpu()
    assert int(counts.max()) >= 100
    y = torch.empty_like(y_uni)
    g = moe.capture(x, logits, y)                # captured on the uniform batch
    for i, (src, other, want) in enumerate([(skew, uniform, y_skew), (uniform, skew, y_uni), (skew, uniform, y_skew)]):
        moe(x, other)                            # the other batch's values in every buffer
        torch.cuda.synchronize()
        logits.copy_(src)
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, want), f"replay {i} differs from the eager step on the same routing"
