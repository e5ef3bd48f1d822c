"""The oracle's layer, step by step, with its grouped GEMMs spread over threads.

Test infrastructure.  Every number comes from an oracle function: each
grouped GEMM is the oracle's own, called on one expert's row range at a time
(the oracle computes every expert independently, so the pieces are the rows
it would produce in one call), with the experts shared out to a thread pool
(numpy releases the interpreter lock inside its array loops and BLAS).  The
other steps are the oracle's calls in the order of oracle.moe_layer.
tests/test_oracle_par.py checks these layers against oracle.moe_layer,
moe_layer_i8 and moe_layer_mxfp4 bit for bit.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
from threadpoolctl import threadpool_limits

import oracle
from oracle import mxfp4_oracle as mx

# per weight form: (activation quantizer, row re-quantizer, grouped GEMM)
FORMS = {
    "g128": (oracle.quant_act, oracle.quant_rows, oracle.grouped_gemm),
    "channel": (oracle.quant_act_i8, oracle.quant_rows_i8, oracle.grouped_gemm_i8),
    "mxfp4": (oracle.quant_act, oracle.quant_rows, mx.grouped_gemm_mxfp4),
}


def workers() -> int:
    """Threads to use: the host's cores, at most 16 (the CPU share of a one-GPU host)."""
    return max(1, min(16, os.cpu_count() or 1))


def gemm_experts(form: str, a, a_scale, a_rows, offsets, w, s, experts=None) -> np.ndarray:
    """The oracle grouped GEMM of `form` on the rows of `experts` (all experts if None).

    Returns out fp32 [offsets[-1], N]; rows of other experts are left zero.
    Experts with many rows run one at a time on every BLAS thread; the rest
    run side by side, one BLAS thread each.
    """
    gemm = FORMS[form][2]
    offsets = np.asarray(offsets, np.int64)
    E = offsets.size - 1
    out = np.zeros((int(offsets[-1]), w.shape[1]), np.float32)
    ex = np.arange(E) if experts is None else np.asarray(sorted(set(int(e) for e in experts)), np.int64)
    ex = ex[offsets[ex + 1] > offsets[ex]]

    def one(e):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        sub = np.array([0, r1 - r0], np.int64)
        if a_rows is None:
            out[r0:r1] = gemm(a[r0:r1], a_scale[r0:r1], None, sub, w[e:e + 1], s[e:e + 1])
        else:
            out[r0:r1] = gemm(a, a_scale, np.asarray(a_rows[r0:r1]), sub, w[e:e + 1], s[e:e + 1])

    big = [int(e) for e in ex if offsets[e + 1] - offsets[e] >= 512]
    small = [int(e) for e in ex if offsets[e + 1] - offsets[e] < 512]
    with threadpool_limits(workers()):
        for e in big:
            one(e)
    if small:
        with threadpool_limits(1), ThreadPoolExecutor(workers()) as pool:
            list(pool.map(one, small))
    return out


def layer(form: str, x_bf16_bits, logits, w13, s13, w2, s2, k: int, renormalize: bool = True) -> dict:
    """oracle.moe_layer (or its INT8 / MXFP4 form) with the GEMMs spread over threads."""
    quant, requant, _ = FORMS[form]
    E = w13.shape[0]
    qx, sx = quant(x_bf16_bits)
    ids, w = oracle.route(logits, k, renormalize)
    offsets, row_token, inv_pos = oracle.permute(ids, E)
    h = gemm_experts(form, qx, sx, row_token, offsets, w13, s13)
    a_f32 = oracle.swiglu_f32(h)
    qa, sa = requant(a_f32)
    o = gemm_experts(form, qa, sa, None, offsets, w2, s2)
    y = oracle.unpermute(o, inv_pos, w)
    return dict(qx=qx, sx=sx, ids=ids, w=w, offsets=offsets, row_token=row_token, inv_pos=inv_pos,
                h=h, a_f32=a_f32, qa=qa, sa=sa, o=o, y=y)
