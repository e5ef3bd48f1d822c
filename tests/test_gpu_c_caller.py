"""The C ABI called from native code: a C++ program (tests/c_caller/moe_layer.cpp, built with the library)
allocates its buffers with hipMalloc, creates its own HIP stream and runs one layer step through the
library's entry points, with no Python or torch in the process.  Its output must equal, bit for bit, the
Python layer's on the same inputs (the same kernels in the same order, all deterministic), and meet the
layer's bar against the oracle."""
from __future__ import annotations

import subprocess

import numpy as np
import pytest
import torch

import oracle
from gpu_util import bf16_to_dev, host, say, to_dev
from quantized_grouped_gemm_token_amd import build as B
from quantized_grouped_gemm_token_amd import ops, workloads
from quantized_grouped_gemm_token_amd.layer import W4A8MoE

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert ops.w4a8_moe_device_supported(), "the current device is not a gfx950"
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("T,H,I,E,k", [
    (16, 256, 128, 64, 2),      # 32 routed rows: the streaming kernel
    (64, 512, 256, 16, 4),      # 256 routed rows over 16 experts: the tiled kernel
    (100, 384, 256, 64, 4),     # 400 routed rows over 64 experts: both launched, the device picks
])
def test_native_caller_matches_layer(T, H, I, E, k, tmp_path):
    wl = workloads.make_custom(T, H, I, E, k, seed=T + E)
    for name, arr in (("x", wl.x_bf16), ("logits", wl.logits), ("w13", wl.w13), ("s13", wl.s13),
                      ("w2", wl.w2), ("s2", wl.s2)):
        np.ascontiguousarray(arr).tofile(tmp_path / f"{name}.bin")
    say(f"native caller T={T} H={H} I={I} E={E} k={k}")
    r = subprocess.run([B.C_CALLER, str(tmp_path), str(T), str(H), str(I), str(E), str(k)], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    y_c = np.fromfile(tmp_path / "y.bin", dtype=np.float32).reshape(T, H)
    moe = W4A8MoE(to_dev(wl.w13), to_dev(wl.s13), to_dev(wl.w2), to_dev(wl.s2), k=k)
    y_py = host(moe(bf16_to_dev(wl.x_bf16), to_dev(wl.logits)))
    assert np.array_equal(y_c.view(np.uint32), y_py.view(np.uint32)), "native caller and Python layer differ"
    res = oracle.moe_layer(wl.x_bf16, wl.logits, wl.w13, wl.s13, wl.w2, wl.s2, k=k)
    fro = np.linalg.norm(y_c.astype(np.float64) - res["y"]) / np.linalg.norm(res["y"])
    assert fro <= 2e-3, fro
    say(f"native caller output: bit-identical to the layer; Frobenius {fro:.2e} against the oracle")
