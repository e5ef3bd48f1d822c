"""w4a8_moe_permute_noalloc: the permutation with its workspace in the
library's own device buffer, for callers that cannot allocate.

Checked through the C ABI against w4a8_moe_permute (with a caller-allocated
workspace) and the oracle, bit for bit, on calls in a row whose sizes shrink
(the buffer keeps the last call's contents), on the one-block path that uses
no buffer, on ids outside [0, E), under HIP graph capture with eager work
between replays, and on the size limit (an error, no launch).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import host, say
from quantized_grouped_gemm_token_amd import ops

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert ops.w4a8_moe_device_supported(), "the current device is not a gfx950"
    yield
    torch.cuda.synchronize()


def _ids(seed, T, k, E, out_of_range=0):
    g = np.random.Generator(np.random.PCG64(seed))
    ids = np.stack([g.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    if out_of_range:
        flat = ids.reshape(-1)
        flat[g.choice(flat.size, size=out_of_range, replace=False)] = E + 3
    return ids


def _both(ids, E):
    t = torch.from_numpy(ids).to(DEV)
    a = [host(v) for v in ops.w4a8_moe_permute_noalloc(t, E)]
    b = [host(v) for v in ops.w4a8_moe_permute(t, E)]
    return a, b


@pytest.mark.parametrize("sizes", [[(4096, 8, 256), (700, 8, 256)], [(20000, 8, 256), (513, 6, 64), (2, 2, 8)]])
def test_calls_in_a_row_shrinking(sizes):
    for i, (T, k, E) in enumerate(sizes):
        ids = _ids(100 + i, T, k, E)
        say(f"permute_noalloc T={T} k={k} E={E} (call {i})")
        got, ref = _both(ids, E)
        for g, r, name in zip(got, ref, ("offsets", "row_token", "inv_pos")):
            assert np.array_equal(g, r), name
        offsets, row_token, inv_pos = oracle.permute(ids, E)
        assert np.array_equal(got[0], offsets)
        assert np.array_equal(got[1], row_token)
        assert np.array_equal(got[2], inv_pos)


def test_ids_out_of_range():
    T, k, E = 1500, 8, 128
    ids = _ids(7, T, k, E, out_of_range=37)
    say("permute_noalloc with ids outside [0, E)")
    got, ref = _both(ids, E)
    for g, r in zip(got, ref):
        assert np.array_equal(g, r)
    assert got[0][-1] == T * k - 37
    assert (got[2] == -1).sum() == 37


def test_graph_replays():
    T, k, E = 3000, 8, 256
    ids_t = torch.from_numpy(_ids(11, T, k, E)).to(DEV)
    offsets = torch.empty((E + 1,), dtype=torch.int32, device=DEV)
    row_token = torch.empty((T * k,), dtype=torch.int32, device=DEV)
    inv_pos = torch.empty((T * k,), dtype=torch.int32, device=DEV)
    ops.w4a8_moe_permute_noalloc(ids_t, E, offsets, row_token, inv_pos)   # eager call first
    torch.cuda.synchronize()
    say("permute_noalloc under graph capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ops.w4a8_moe_permute_noalloc(ids_t, E, offsets, row_token, inv_pos)
    for r in range(4):
        ids = _ids(200 + r, T, k, E)
        ids_t.copy_(torch.from_numpy(ids).to(DEV))
        # eager use of the same buffer between replays, with another size
        small = torch.from_numpy(_ids(300 + r, 900, 8, 256)).to(DEV)
        o2 = [host(v) for v in ops.w4a8_moe_permute_noalloc(small, 256)]
        assert np.array_equal(o2[1], oracle.permute(small.cpu().numpy(), 256)[1])
        g.replay()
        torch.cuda.synchronize()
        want = oracle.permute(ids, E)
        assert np.array_equal(host(offsets), want[0])
        assert np.array_equal(host(row_token), want[1])
        assert np.array_equal(host(inv_pos), want[2])


def test_size_limit_is_an_error():
    # 2^21 routed rows at E = 256 would need 2 MiB of counts: refused on the host
    T, k, E = 1 << 18, 8, 256
    assert ops.w4a8_moe_permute_workspace_bytes(T, k, E) > (1 << 20)
    ids = torch.zeros((T, k), dtype=torch.int32, device=DEV)
    with pytest.raises(ops.W4A8Error) as err:
        ops.w4a8_moe_permute_noalloc(ids, E)
    assert err.value.status == 6                      # W4A8_ERR_WORKSPACE
    # the largest size that fits still runs
    T2 = (1 << 20) // 8
    assert ops.w4a8_moe_permute_workspace_bytes(T2, k, E) <= (1 << 20)
    ids2 = torch.from_numpy(_ids(5, 4096, 8, 256)).to(DEV).repeat(T2 // 4096, 1)
    say("permute_noalloc at the largest size the buffer holds")
    got = [host(v) for v in ops.w4a8_moe_permute_noalloc(ids2, E)]
    ref = [host(v) for v in ops.w4a8_moe_permute(ids2, E)]
    for a, b in zip(got, ref):
        assert np.array_equal(a, b)
