"""CPU oracle of the MXFP4 group-32 weight variant of the layer.

TEST INFRASTRUCTURE, like the rest of this package: only the tests, the smoke
check and the benchmark's CPU-baseline leg may import it; the product path
never does, and it shares no code with the HIP kernels.

What it computes, and where that is stated:

* "GLM-5.3-W4A8" model card (gpustack), section 量化方式: the alternative
  4-bit format the card compares against is MXFP4 with groups of 32 (its
  weight-reconstruction error, 0.113, is quoted next to INT4 group 128); the
  same card, section on the kernels, says Hopper has no FP4 matrix cores, so
  MXFP4 would have run as W4A16 there.  gfx950 multiplies FP4 by FP8 in its
  matrix cores, so here MXFP4 weights meet the same per-token FP8
  activations as the INT4 form (W4A8).
* The format itself is the Open Compute Project microscaling (MX) format:
  blocks of 32 elements along K share one E8M0 scale (a power of two, byte
  b meaning 2^(b - 127)); elements are FP4 E2M1 (1 sign, 2 exponent bits with
  bias 1, 1 mantissa bit): magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.

Readings where the pages are silent:
  * the block scale follows the MX rule: X = floor(log2(amax)) - 2 (2 is the
    largest E2M1 exponent), so amax / 2^X lies in [4, 8) and values above 6
    saturate; an all-zero block is treated as amax = 1.  This rule gives
    0.114 on Gaussian weights, next to the card's 0.113;
  * elements are w / 2^X (exact) rounded to the nearest E2M1 value, ties to
    the even code (mantissa bit 0), saturating at 6, sign kept on zero;
  * storage: codes packed two per byte along K, element k in the low nibble
    of byte k/2 when k is even, the high nibble when odd; scales as bytes
    [N][K/32];
  * activations, routing, permutation, SwiGLU and the combine are those of
    the INT4 group-128 form (w4a8_oracle).

The products are exact in fp64 (an E4M3 value times an E2M1 value times a
power of two); sums are taken in fp64 and rounded once to fp32.
"""
from __future__ import annotations

import numpy as np

from .w4a8_oracle import e4m3_decode, permute, quant_act, quant_rows, route, swiglu_f32, unpermute

MX_BLOCK = 32                      # elements per shared scale
E2M1_MAX = 6.0
E2M1_EMAX = 2                      # exponent of the largest E2M1 binade (4 and 6)
E8M0_BIAS = 127
# magnitude of the 8 non-negative E2M1 codes (code = exponent bits e, mantissa bit m: e == 0 -> m / 2,
# else (1 + m / 2) * 2^(e - 1))
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_decode(codes) -> np.ndarray:
    """fp64 value of 4-bit E2M1 codes (0..15; bit 3 is the sign)."""
    codes = np.asarray(codes, dtype=np.int64)
    mag = E2M1_MAGNITUDES[codes & 7]
    return np.where(codes & 8, -mag, mag)


def e2m1_encode(v) -> np.ndarray:
    """E2M1 code of real values: nearest magnitude, ties to the even code, saturating at 6.

    The inputs are exact (fp64 holding w / 2^X exactly); the nearest of the 8
    magnitudes is found by comparing distances, and a tie goes to the code
    whose mantissa bit is 0 (an even code).  A negative value keeps its sign
    bit even when it rounds to 0.
    """
    v = np.asarray(v, dtype=np.float64)
    if np.isnan(v).any():
        raise ValueError("e2m1_encode: NaN input")
    a = np.minimum(np.abs(v), E2M1_MAX)
    d = np.abs(a[..., None] - E2M1_MAGNITUDES)                 # distance to each of the 8 codes
    best = d.min(axis=-1, keepdims=True)
    cand = d == best                                            # one code, or two on a tie
    even = cand & (np.arange(8) % 2 == 0)
    code = np.where(even.any(axis=-1), np.argmax(even, axis=-1), np.argmax(cand, axis=-1))
    return (code | np.where(np.signbit(v), 8, 0)).astype(np.uint8)


def mx_block_exponent(amax) -> np.ndarray:
    """Shared exponent X of blocks with the given max |w|: floor(log2 amax) - 2 (amax 0 counts as 1),
    clamped to the E8M0 range [-127, 127]."""
    amax = np.asarray(amax, dtype=np.float64)
    amax = np.where(amax > 0, amax, 1.0)
    _, e = np.frexp(amax)                                       # amax = f * 2^e, f in [0.5, 1): floor(log2) = e - 1
    return np.clip(e - 1 - E2M1_EMAX, -E8M0_BIAS, E8M0_BIAS).astype(np.int64)


def quantize_mxfp4(W) -> tuple[np.ndarray, np.ndarray]:
    """MXFP4 of a weight matrix [N, K] -> (codes uint8 [N, K] (0..15), scales uint8 [N, K/32] (E8M0))."""
    W = np.asarray(W, dtype=np.float32).astype(np.float64)
    N, K = W.shape
    if K % MX_BLOCK:
        raise ValueError("K must be a multiple of 32")
    B = W.reshape(N, K // MX_BLOCK, MX_BLOCK)
    X = mx_block_exponent(np.abs(B).max(axis=2))
    codes = e2m1_encode(B / np.exp2(X)[..., None]).reshape(N, K)   # w / 2^X is exact in fp64
    return codes, (X + E8M0_BIAS).astype(np.uint8)


def fp4_pack(codes) -> np.ndarray:
    """E2M1 codes [..., K] -> bytes [..., K/2]: even k in the low nibble, odd k in the high one."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def fp4_unpack(packed) -> np.ndarray:
    """Inverse of fp4_pack."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def dequant_mxfp4(packed, scales) -> np.ndarray:
    """fp64 weights [..., K] of packed codes [..., K/2] and E8M0 scales [..., K/32] (exact)."""
    vals = e2m1_decode(fp4_unpack(packed))
    s = np.exp2(np.asarray(scales, dtype=np.float64) - E8M0_BIAS)
    return vals * np.repeat(s, MX_BLOCK, axis=-1)


def grouped_gemm_mxfp4(a_codes, a_scale, a_rows, offsets, w_packed, w_scale) -> np.ndarray:
    """out[p, n] = a_scale[r] * sum_k dec(a[r, k]) * w[e, n, k] (fp64, rounded once to fp32).

    r = a_rows[p] when a gather list is given, else p; e is the expert whose
    row range holds p.  a_codes [*, K] E4M3, w_packed [E, N, K/2] uint8,
    w_scale [E, N, K/32] uint8 (E8M0).
    """
    offsets = np.asarray(offsets, dtype=np.int64)
    E = offsets.size - 1
    N = w_packed.shape[1]
    M = int(offsets[-1])
    out = np.zeros((M, N), dtype=np.float32)
    a_scale = np.asarray(a_scale, dtype=np.float32).astype(np.float64)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        rows = np.asarray(a_rows[r0:r1]) if a_rows is not None else np.arange(r0, r1)
        A = e4m3_decode(np.asarray(a_codes)[rows])
        Wd = dequant_mxfp4(w_packed[e], w_scale[e])
        out[r0:r1] = ((A @ Wd.T) * a_scale[rows][:, None]).astype(np.float32)
    return out


def moe_layer_mxfp4(x_bf16_bits, logits, w13, s13, w2, s2, k: int, renormalize: bool = True) -> dict:
    """The whole layer with MXFP4 experts: w13 [E, 2I, H/2], s13 [E, 2I, H/32], w2 [E, H, I/2], s2 [E, H, I/32]."""
    E = w13.shape[0]
    qx, sx = quant_act(x_bf16_bits)
    ids, w = route(logits, k, renormalize)
    offsets, row_token, inv_pos = permute(ids, E)
    h = grouped_gemm_mxfp4(qx, sx, row_token, offsets, w13, s13)
    a_f32 = swiglu_f32(h)
    qa, sa = quant_rows(a_f32)
    o = grouped_gemm_mxfp4(qa, sa, None, offsets, w2, s2)
    y = unpermute(o, inv_pos, w)
    return dict(qx=qx, sx=sx, ids=ids, w=w, offsets=offsets, row_token=row_token, inv_pos=inv_pos,
                h=h, a_f32=a_f32, qa=qa, sa=sa, o=o, y=y)
