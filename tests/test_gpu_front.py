"""Steps 1-3 in one call (w4a8_moe_front / w4a8_moe_front_i8) against the oracle.

The decode shapes (T*k <= 4096, H <= 8192) run the fused kernel, whose last
routing workgroup sorts the routed rows; the others run the three kernels.
Three calls in a row on one counter, the last on new inputs, must each give
the oracle's codes, routing and permutation, and leave the counter at zero.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import bf16_to_dev, host, say, to_dev
from quantized_grouped_gemm_token_amd import ops

pytestmark = pytest.mark.gpu


def _bits(x):
    return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("T,H,E,k,int8,renorm", [(128, 6144, 256, 8, False, False), (100, 1024, 100, 6, True, False)] + [
    c + (True,) for c in [
    (128, 6144, 256, 8, False), (128, 6144, 256, 8, True),       # the decode workload, both quantizers
    (16, 256, 8, 2, False), (100, 1024, 100, 6, False), (64, 2048, 500, 8, True), (30, 512, 1024, 16, False),
    (1, 128, 4, 1, False), (127, 8192, 256, 8, True),             # one token; the largest fused row
    (200, 1024, 256, 8, False), (512, 1024, 64, 8, True),         # 1600 and 4096 routed rows: still one kernel
    (600, 512, 256, 8, False), (64, 12288, 64, 4, True),          # three kernels: T*k > 4096; H > 8192
]])
def test_front_matches_oracle(T, H, E, k, int8, renorm, rng):
    counter = torch.zeros((1,), dtype=torch.int32, device="cuda:0")
    for call in range(3):
        if call != 1:   # calls 0 and 1 on the same inputs, call 2 on new ones
            x = (rng.standard_normal((T, H)) * np.exp2(rng.integers(-4, 4, size=(T, 1)))).astype(np.float32)
            logits = rng.standard_normal((T, E)).astype(np.float32)
            logits[:, 5 % E] = logits[:, 2 % E]                      # forced ties
            bits = _bits(x)
        say(f"front T={T} H={H} E={E} k={k} int8={int8} renorm={renorm} call {call}")
        qx, sx, rs, ids, w, offsets, row_token, inv_pos = ops.w4a8_moe_front(bf16_to_dev(bits), to_dev(logits), k,
                                                                             counter, renormalize=renorm,
                                                                             int8=int8)
        if int8:
            q_ref, s_ref = oracle.quant_act_i8(bits)
            r_ref = oracle.code_row_sums(q_ref)
            assert np.array_equal(host(rs), r_ref)
        else:
            q_ref, s_ref = oracle.quant_act(bits)
        assert np.array_equal(host(qx), q_ref)
        assert np.array_equal(host(sx).view(np.uint32), s_ref.view(np.uint32))
        ids_ref, w_ref = oracle.route(logits, k, renorm)
        assert np.array_equal(host(ids), ids_ref)
        assert np.all(np.abs(host(w).astype(np.float64) - w_ref) <= 1e-6 * np.abs(w_ref))
        off_ref, rt_ref, inv_ref = oracle.permute(ids_ref, E)
        assert np.array_equal(host(offsets), off_ref)
        assert np.array_equal(host(row_token), rt_ref) and np.array_equal(host(inv_pos), inv_ref)
        assert int(host(counter)[0]) == 0


def test_front_empty():
    say("front T=0")
    counter = torch.zeros((1,), dtype=torch.int32, device="cuda:0")
    x = torch.zeros((0, 256), dtype=torch.bfloat16, device="cuda:0")
    logits = torch.zeros((0, 16), dtype=torch.float32, device="cuda:0")
    out = ops.w4a8_moe_front(x, logits, 4, counter)
    assert np.array_equal(host(out[5]), np.zeros(17, np.int32))
    assert int(host(counter)[0]) == 0
