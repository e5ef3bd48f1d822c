"""Whole-layer pins: a token-by-token brute force and routing invariance."""
import numpy as np
import torch
from scipy.special import expit

import oracle
from quantized_grouped_gemm_token_amd import workloads


def _torch_quant(x64):
    x = torch.from_numpy(np.ascontiguousarray(x64, dtype=np.float32))
    amax = x.abs().amax()
    sc = amax / 448.0 if amax > 0 else torch.tensor(1.0)
    return (x / sc).to(torch.float8_e4m3fn).to(torch.float64) * sc.double()


def _brute_layer(wl, k):
    sh = wl.shape
    x = torch.from_numpy(wl.x_bf16.view(np.int16)).view(torch.bfloat16).float().numpy()
    y = np.zeros((sh.T, sh.H), np.float64)
    W13 = oracle.int4_unpack(wl.w13).astype(np.float64) * np.repeat(wl.s13, 128, axis=2)
    W2 = oracle.int4_unpack(wl.w2).astype(np.float64) * np.repeat(wl.s2, 128, axis=2)
    for t in range(sh.T):
        order = sorted(range(sh.E), key=lambda e: (-float(wl.logits[t, e]), e))[:k]
        lg = wl.logits[t, order].astype(np.float64)
        p = np.exp(lg - lg.max())
        wts = (p / p.sum()).astype(np.float32)
        a = _torch_quant(x[t]).numpy()
        for j, e in enumerate(order):
            h = (W13[e] @ a).astype(np.float32).astype(np.float64)
            gte, up = h[:sh.I], h[sh.I:]
            act = (gte * expit(gte) * up).astype(np.float32)
            aq = _torch_quant(act).numpy()
            o = (W2[e] @ aq).astype(np.float32)
            y[t] += float(wts[j]) * o.astype(np.float64)
    return y.astype(np.float32)


def test_tiny_layer_brute_force():
    wl = workloads.make_config(0)
    res = oracle.moe_layer(wl.x_bf16, wl.logits, wl.w13, wl.s13, wl.w2, wl.s2, k=2)
    yb = _brute_layer(wl, 2)
    rel = np.linalg.norm(res["y"] - yb) / np.linalg.norm(yb)
    assert rel < 1e-5
    close = np.abs(res["y"] - yb) <= 1e-5 * np.abs(yb) + 1e-6
    assert close.mean() > 0.99


def test_identical_experts_make_routing_irrelevant():
    wl = workloads.make_custom(T=12, H=256, I=128, E=6, k=3, seed=7)
    w13 = np.repeat(wl.w13[:1], 6, axis=0)
    s13 = np.repeat(wl.s13[:1], 6, axis=0)
    w2 = np.repeat(wl.w2[:1], 6, axis=0)
    s2 = np.repeat(wl.s2[:1], 6, axis=0)
    r1 = oracle.moe_layer(wl.x_bf16, wl.logits, w13, s13, w2, s2, k=3)
    logits2 = np.random.Generator(np.random.PCG64(3)).standard_normal(wl.logits.shape).astype(np.float32)
    r2 = oracle.moe_layer(wl.x_bf16, logits2, w13, s13, w2, s2, k=3)
    assert not np.array_equal(r1["ids"], r2["ids"])
    assert np.allclose(r1["y"], r2["y"], rtol=1e-5, atol=1e-6)
    # and equal to one expert applied with weight 1
    r3 = oracle.moe_layer(wl.x_bf16, wl.logits, w13, s13, w2, s2, k=1)
    assert np.allclose(r1["y"], r3["y"], rtol=1e-5, atol=1e-6)


def test_layer_is_token_local():
    wl = workloads.make_config(0)
    full = oracle.moe_layer(wl.x_bf16, wl.logits, wl.w13, wl.s13, wl.w2, wl.s2, k=2)
    sel = np.array([3, 11, 0])
    sub = oracle.moe_layer(wl.x_bf16[sel], wl.logits[sel], wl.w13, wl.s13, wl.w2, wl.s2, k=2)
    for key in ("qx", "sx", "ids", "w", "y"):
        assert np.array_equal(full[key][sel], sub[key]), key
