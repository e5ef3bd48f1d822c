"""CPU oracle of the per-channel INT4 x per-token INT8 variant of the layer.

TEST INFRASTRUCTURE, like the rest of this package: only the tests, the smoke
check and the benchmark's CPU-baseline leg may import it; the product path
never does, and it shares no code with the HIP kernels.

What it computes, and where that is stated:

* "GLM-5.3-Channel-INT4-w4a8" card (hygon), section 1 (基本信息, the table):
  the routed experts are INT4 W4A8 with weights quantized RTN, static,
  per channel, in the compressed-tensors format; activations are INT8,
  dynamic, per token, without calibration data.
* The rest of the layer (routing, permutation, SwiGLU, the routing-weighted
  combine) is the same as in the group-128 FP8 variant of w4a8_oracle.

Readings where the page is silent:
  * a weight row n has one fp32 scale s[n] = fl32(amax_n / 7) (1/7 for an
    all-zero row); q = clamp(round-half-even(w / s), -8, 7) from the exact
    quotient; the codes are packed as uint4b8 (q + 8) in int32 words, the
    same layout as the group-128 variant;
  * an activation row has scale = fl32(amax / 127) (1.0 for an all-zero
    row) and codes clamp(round-half-even(fl32(x / scale)), -127, 127) -- the
    fp32 quotient, then integer rounding;
  * the product sums the integer codes exactly and applies the two scales
    once: out = a_scale[row] * w_scale[n] * sum_k a[k] q[n, k].

Every integer sum here is exact (integers below 2^30, held exactly by fp64);
scales are applied in fp64 and the result rounded once to fp32.
"""
from __future__ import annotations

import numpy as np

from .w4a8_oracle import (bf16_bits_to_f32, int4_unpack, permute, route, swiglu_f32,
                          unpermute)

INT8_MAX = 127.0
INT4_MAX = 7.0


def quant_rows_i8(x) -> tuple[np.ndarray, np.ndarray]:
    """Per-row INT8 codes of an fp32 matrix [M, K] -> (codes int8 [M, K], scale fp32 [M])."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=1) if x.shape[1] else np.zeros(x.shape[0], np.float32)
    scale = np.where(amax > 0, (amax / np.float32(INT8_MAX)).astype(np.float32), np.float32(1.0))
    q = np.rint((x / scale[:, None]).astype(np.float32))
    codes = np.clip(q, -INT8_MAX, INT8_MAX).astype(np.int8)
    return codes, scale.astype(np.float32)


def quant_act_i8(x_bf16_bits) -> tuple[np.ndarray, np.ndarray]:
    """Step 1 of the variant: bf16 activations [T, H] -> INT8 codes and per-token scales."""
    return quant_rows_i8(bf16_bits_to_f32(x_bf16_bits))


def code_row_sums(codes) -> np.ndarray:
    """Sum of each row's INT8 codes (int32 [M]).

    Not a step of the method: the library's INT8 calls return these sums next
    to the codes (its GEMM subtracts 8 times them to undo the uint4b8 offset),
    and the tests compare them with this plain sum.
    """
    return np.asarray(codes, dtype=np.int64).sum(axis=1).astype(np.int32)


def quantize_int4_channel(W) -> tuple[np.ndarray, np.ndarray]:
    """Per-channel symmetric INT4 RTN of a weight matrix [N, K] -> (q int8 [N, K], s fp32 [N])."""
    W64 = np.asarray(W, dtype=np.float32).astype(np.float64)
    amax = np.abs(W64).max(axis=1)
    amax = np.where(amax > 0, amax, 1.0)
    s = (amax / INT4_MAX).astype(np.float32)
    q = np.clip(np.rint(W64 / s.astype(np.float64)[:, None]), -8, 7).astype(np.int8)
    return q, s


def grouped_gemm_i8(a_codes, a_scale, a_rows, offsets, w_packed, w_scale) -> np.ndarray:
    """out[p, n] = a_scale[r] * w_scale[e, n] * sum_k a[r, k] * q[e, n, k].

    r = a_rows[p] when a gather list is given, else p; e is the expert whose
    row range holds p.  a_codes [*, K] int8, a_scale [*] fp32, offsets [E+1],
    w_packed [E, N, K/8] int32 (uint4b8), w_scale [E, N] fp32.  The integer
    sums are exact (each partial sum an integer below 2^30); the scales are
    applied in fp64.
    """
    offsets = np.asarray(offsets, dtype=np.int64)
    E = offsets.size - 1
    N = w_packed.shape[1]
    M = int(offsets[-1])
    out = np.zeros((M, N), dtype=np.float32)
    a_scale = np.asarray(a_scale, dtype=np.float32)
    w_scale = np.asarray(w_scale, dtype=np.float32)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        rows = np.asarray(a_rows[r0:r1]) if a_rows is not None else np.arange(r0, r1)
        # the integer sums, formed exactly: |a q| <= 127 * 8, so with K <= 2^20 every
        # partial sum is an integer below 2^30, which fp64 holds exactly in any order
        A = np.asarray(a_codes[rows], dtype=np.int8).astype(np.float64)
        Q = int4_unpack(w_packed[e]).astype(np.float64)
        if A.shape[1] > 1 << 20:
            raise ValueError("K above 2^20: the integer sums would not be exact in fp64")
        acc = A @ Q.T
        out[r0:r1] = (acc * a_scale[rows].astype(np.float64)[:, None]
                      * w_scale[e].astype(np.float64)[None, :]).astype(np.float32)
    return out


def swiglu_i8(h) -> tuple[np.ndarray, np.ndarray]:
    """Step 5 of the variant: silu(gate) * up in fp64 -> fp32, then per-row INT8 codes."""
    return quant_rows_i8(swiglu_f32(h))


def moe_layer_i8(x_bf16_bits, logits, w13, s13, w2, s2, k: int, renormalize: bool = True) -> dict:
    """The whole layer in the per-channel INT4 x per-token INT8 variant.

    w13 [E, 2I, H/8] and w2 [E, H, I/8] are packed uint4b8; s13 [E, 2I] and
    s2 [E, H] are the per-channel scales.
    """
    E = w13.shape[0]
    qx, sx = quant_act_i8(x_bf16_bits)
    ids, w = route(logits, k, renormalize)
    offsets, row_token, inv_pos = permute(ids, E)
    h = grouped_gemm_i8(qx, sx, row_token, offsets, w13, s13)
    a_f32 = swiglu_f32(h)
    qa, sa = quant_rows_i8(a_f32)
    o = grouped_gemm_i8(qa, sa, None, offsets, w2, s2)
    y = unpermute(o, inv_pos, w)
    return dict(qx=qx, sx=sx, ids=ids, w=w, offsets=offsets, row_token=row_token, inv_pos=inv_pos,
                h=h, a_f32=a_f32, qa=qa, sa=sa, o=o, y=y)
