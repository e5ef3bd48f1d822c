"""GPU parity of the grouped GEMMs on the weights as the pages store them.

The calls without "_prepacked" take the row-major stored format of the
"GLM-5.3-W4A8" card, section 量化方式 (compressed-tensors pack-quantized:
uint4b8 nibbles, eight per int32 word along K, fp32 scales [E][N][K/128]),
and the row-major MXFP4 bytes.  Each is checked against the oracle (to the
bars of the prepacked calls) and against the prepacked call on the same
weights, with the streaming kernel on both sides: the two read the same
bytes in a different order and perform the same arithmetic in the same
order, so their outputs are bit-identical.  Shapes include N % 64 != 0
(N % 16 is the stored format's rule), empty experts, experts with more than
16 rows (several M blocks) and gathered activation rows.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import GEMM_FRO_TIGHT, assert_float_parity, edge_shape_maxrel, host, say, to_dev
from oracle import mxfp4_oracle as mx
from quantized_grouped_gemm_token_amd import ops

pytestmark = pytest.mark.gpu

STREAM = ops.W4A8_GG_STREAM

SHAPES = [
    (4, 48, 256, [3, 0, 17, 1], True),           # N = 48: three 16-column subtiles, one wave half-used
    (3, 80, 384, [20, 1, 40], False),            # odd group count, N = 80
    (2, 256, 1024, [33, 0], True),
    (5, 208, 128, [0, 0, 0, 5, 0], True),        # one group, N % 64 == 16
    (1, 16, 640, [7], False),                    # one subtile
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert ops.w4a8_moe_device_supported(), "the current device is not a gfx950"
    yield
    torch.cuda.synchronize()


def _activations(rng, K, counts, gather):
    M = int(np.sum(counts))
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    src = 29 if gather else M
    x = rng.standard_normal((src, K)).astype(np.float32) * np.exp2(rng.integers(-3, 3, size=(src, 1)))
    rows = rng.integers(0, src, size=M).astype(np.int32) if gather else None
    return offsets, x, rows


def _dev(t):
    return None if t is None else to_dev(t)


@pytest.mark.parametrize("E,N,K,counts,gather", SHAPES)
def test_grouped_gemm_stored(E, N, K, counts, gather, rng):
    offsets, x, rows = _activations(rng, K, counts, gather)
    a, sa = oracle.quant_rows(x)
    w = rng.integers(0, 2**32, size=(E, N, K // 8), dtype=np.uint32).view(np.int32)
    s = rng.lognormal(-4, 0.5, size=(E, N, K // 128)).astype(np.float32)
    M = int(offsets[-1])
    want = oracle.grouped_gemm(a, sa, rows, offsets, w, s)
    say(f"grouped_gemm (stored) E={E} N={N} K={K} counts={counts}")
    got = host(ops.w4a8_moe_grouped_gemm(to_dev(a), to_dev(sa), _dev(rows), to_dev(offsets), to_dev(w), to_dev(s), M))
    assert_float_parity(got, want, "grouped_gemm stored", fro_tight=GEMM_FRO_TIGHT, maxrel=edge_shape_maxrel(N))
    if N % 64 == 0:
        wb, sb = ops.w4a8_moe_prepack_int4(to_dev(w), to_dev(s))
        ref = host(ops.w4a8_moe_grouped_gemm_prepacked(to_dev(a), to_dev(sa), _dev(rows), to_dev(offsets), wb, sb, M,
                                                       algo=STREAM))
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("E,N,K,counts,gather", SHAPES)
def test_grouped_gemm_i8_stored(E, N, K, counts, gather, rng):
    offsets, x, rows = _activations(rng, K, counts, gather)
    codes, scale = oracle.quant_rows_i8(x)
    rowsum = oracle.code_row_sums(codes)
    w = rng.integers(0, 2**32, size=(E, N, K // 8), dtype=np.uint32).view(np.int32)
    ws = rng.lognormal(-4, 0.5, size=(E, N)).astype(np.float32)
    M = int(offsets[-1])
    want = oracle.grouped_gemm_i8(codes, scale, rows, offsets, w, ws)
    say(f"grouped_gemm_i8 (stored) E={E} N={N} K={K} counts={counts}")
    got = host(ops.w4a8_moe_grouped_gemm_i8(to_dev(codes), to_dev(scale), to_dev(rowsum), _dev(rows), to_dev(offsets),
                                            to_dev(w), to_dev(ws), M_total=M))
    zero = want == 0
    assert np.all(got[zero] == 0)
    rel = np.abs(got[~zero].astype(np.float64) - want[~zero]) / np.abs(want[~zero].astype(np.float64))
    assert rel.max(initial=0.0) <= 1e-6, rel.max()
    if N % 64 == 0:
        ref = host(ops.w4a8_moe_grouped_gemm_i8_prepacked(
            to_dev(codes), to_dev(scale), to_dev(rowsum), _dev(rows), to_dev(offsets),
            ops.w4a8_moe_prepack_int4(to_dev(w))[0], to_dev(ws), M_total=M, algo=STREAM))
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("E,N,K,counts,gather", SHAPES)
def test_grouped_gemm_mxfp4_stored(E, N, K, counts, gather, rng):
    offsets, x, rows = _activations(rng, K, counts, gather)
    a, sa = oracle.quant_rows(x)
    w = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    s = rng.integers(118, 136, size=(E, N, K // 32)).astype(np.uint8)
    M = int(offsets[-1])
    want = mx.grouped_gemm_mxfp4(a, sa, rows, offsets, w, s)
    say(f"grouped_gemm_mxfp4 (stored) E={E} N={N} K={K} counts={counts}")
    got = host(ops.w4a8_moe_grouped_gemm_mxfp4(to_dev(a), to_dev(sa), _dev(rows), to_dev(offsets), to_dev(w),
                                               to_dev(s), M))
    assert_float_parity(got, want, "grouped_gemm_mxfp4 stored", fro_tight=GEMM_FRO_TIGHT,
                        maxrel=edge_shape_maxrel(N))
    if N % 64 == 0:
        wb, sb = ops.w4a8_moe_prepack_mxfp4(to_dev(w), to_dev(s))
        ref = host(ops.w4a8_moe_grouped_gemm_mxfp4_prepacked(to_dev(a), to_dev(sa), _dev(rows), to_dev(offsets), wb,
                                                             sb, M, algo=STREAM))
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


FUSED = [
    (4, 128, 256, [3, 0, 17, 1], True),
    (3, 256, 384, [20, 1, 40], False),
    (2, 384, 1024, [33, 0], True),
]


@pytest.mark.parametrize("form", ["g128", "i8", "mxfp4"])
@pytest.mark.parametrize("E,I,K,counts,gather", FUSED)
def test_grouped_gemm_swiglu_stored(form, E, I, K, counts, gather, rng):
    offsets, x, rows = _activations(rng, K, counts, gather)
    M = int(offsets[-1])
    N = 2 * I
    if form == "i8":
        a, sa = oracle.quant_rows_i8(x)
        rs = oracle.code_row_sums(a)
        w = rng.integers(0, 2**32, size=(E, N, K // 8), dtype=np.uint32).view(np.int32)
        s = rng.lognormal(-4, 0.5, size=(E, N)).astype(np.float32)
        h = oracle.grouped_gemm_i8(a, sa, rows, offsets, w, s)
        fro = 1e-5
    else:
        a, sa = oracle.quant_rows(x)
        rs = None
        if form == "g128":
            w = rng.integers(0, 2**32, size=(E, N, K // 8), dtype=np.uint32).view(np.int32)
            s = rng.lognormal(-4, 0.5, size=(E, N, K // 128)).astype(np.float32)
            h = oracle.grouped_gemm(a, sa, rows, offsets, w, s)
        else:
            w = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
            s = rng.integers(118, 136, size=(E, N, K // 32)).astype(np.uint8)
            h = mx.grouped_gemm_mxfp4(a, sa, rows, offsets, w, s)
        fro = GEMM_FRO_TIGHT
    want = oracle.swiglu_f32(h)
    say(f"grouped_gemm_swiglu_{form} (stored) E={E} I={I} K={K} counts={counts}")
    args = (to_dev(a), to_dev(sa)) + ((to_dev(rs),) if form == "i8" else ()) + (_dev(rows), to_dev(offsets))
    if form == "g128":
        act, pmax = ops.w4a8_moe_grouped_gemm_swiglu(*args, to_dev(w), to_dev(s), M)
        wb, sb = ops.w4a8_moe_prepack_int4(to_dev(w), to_dev(s))
        ref, _ = ops.w4a8_moe_grouped_gemm_swiglu_prepacked(*args, wb, sb, M, algo=STREAM)
    elif form == "i8":
        act, pmax = ops.w4a8_moe_grouped_gemm_swiglu_i8(*args, to_dev(w), to_dev(s), M)
        ref, _ = ops.w4a8_moe_grouped_gemm_swiglu_i8_prepacked(*args, ops.w4a8_moe_prepack_int4(to_dev(w))[0],
                                                               to_dev(s), M, algo=STREAM)
    else:
        act, pmax = ops.w4a8_moe_grouped_gemm_swiglu_mxfp4(*args, to_dev(w), to_dev(s), M)
        wb, sb = ops.w4a8_moe_prepack_mxfp4(to_dev(w), to_dev(s))
        ref, _ = ops.w4a8_moe_grouped_gemm_swiglu_mxfp4_prepacked(*args, wb, sb, M, algo=STREAM)
    act, pmax, ref = host(act), host(pmax), host(ref)
    assert_float_parity(act, want, f"grouped_gemm_swiglu_{form} stored", fro_tight=fro, maxrel=edge_shape_maxrel(I))
    assert np.array_equal(pmax.max(axis=1), np.abs(act).max(axis=1))
    assert np.array_equal(act.view(np.uint32), ref.view(np.uint32))
