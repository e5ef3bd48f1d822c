"""CPU oracle for the W4A8 mixture-of-experts routed-expert layer.

TEST INFRASTRUCTURE. This module is the slow, plain reference that the GPU
path is checked against. Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import it; the product path never does.
It shares no code with the HIP kernels or their Python binding.

What it computes, and where that is stated (page title, then section):

* "GLM-5.3-W4A8" model card (gpustack), section 量化方式 (quantization
  method): routed-expert weights are symmetric INT4 with one scale per group
  of 128 along the contraction axis, stored compressed-tensors
  ``pack-quantized`` as uint4b8 (nibble = q + 8) inside int32 words;
  activations are quantized to FP8 per token, dynamically, at run time; the
  grouped GEMM turns the INT4 weights into FP8 inside the kernel and never
  goes through BF16.  The intro note of the same card says eight 4-bit
  weights share one int32 slot.
* Same card, section 与其他 4-bit 版本的差异 (table): "FP8 per-token dynamic"
  activations, INT4 group-128 experts.
* "从 755GB 到 395GB" (Bitdeer AI blog), section 难点在于显存限制: each routed
  expert has three projection matrices (gate, up, down).
* The layer structure (top-k routing, gate/up projection, SwiGLU, down
  projection, routing-weighted combine) and the FP8 format (E4M3, amax/448)
  are the problem statement's; the pages give no formula for them.

Readings where the pages are silent:
  * FP8 is OCP E4M3FN (bias 7, max 448, no infinities); conversion is round
    to nearest, ties to even, saturating at 448, sign kept on zero.
  * per-token scale = fl32(amax / 448) (1.0 for an all-zero row); the code of
    x is enc(fl32(x / scale)) -- both divisions IEEE fp32, so the double
    rounding is part of the definition.
  * nibble for k sits at bits 4*(k mod 8) of word k // 8 (packing along K).
  * scales are fp32, laid out [E][N][K/128].
  * routing: softmax over the logits, the k largest logits in descending
    order with ties to the lower expert index, weights renormalised over the
    chosen k (optional).
  * W13 is [E][2I][H] with the I gate rows first, then the I up rows;
    SwiGLU is silu(gate) * up with no clamp; its output is re-quantized per
    routed row with the same FP8 rule.
  * the routing weights are applied after the down projection.

Floating point: every sum is taken in fp64 and rounded once to fp32 at the
end of each step, which is where the GPU path also materialises a result.
"""
from __future__ import annotations

import sys

import numpy as np

FP8_MAX = 448.0          # largest finite E4M3FN magnitude
GROUP = 128              # INT4 group size along K
NIBBLES_PER_WORD = 8     # eight 4-bit weights per int32 word
UINT4B8_BIAS = 8         # stored nibble u = q + 8


# --------------------------------------------------------------------------
# O1. E4M3FN codec (OCP 8-bit floating point, E4M3 variant)
# --------------------------------------------------------------------------
def _build_e4m3_values() -> np.ndarray:
    """Value of every one of the 256 E4M3FN codes, as fp64 (NaN for 0x7F/0xFF).

    Field layout: sign (1 bit), exponent (4 bits, bias 7), mantissa (3 bits).
    Exponent field 0 is subnormal: m * 2^-9.  Otherwise (1 + m/8) * 2^(e-7).
    The all-ones exponent with all-ones mantissa is NaN; there is no infinity.
    """
    vals = np.empty(256, dtype=np.float64)
    for c in range(256):
        s = (c >> 7) & 1
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            vals[c] = np.nan
            continue
        if e == 0:
            mag = m * 2.0 ** -9
        else:
            mag = (1.0 + m / 8.0) * 2.0 ** (e - 7)
        vals[c] = -mag if s else mag
    return vals


E4M3_VALUES = _build_e4m3_values()
# codes 0x00 .. 0x7E are the non-negative finite values in increasing order
_E4M3_POS = E4M3_VALUES[:0x7F].copy()


def e4m3_decode(codes) -> np.ndarray:
    """fp64 value of E4M3FN codes (uint8 array)."""
    codes = np.asarray(codes, dtype=np.uint8)
    return E4M3_VALUES[codes]


def e4m3_encode(v) -> np.ndarray:
    """E4M3FN code of fp32 values: nearest, ties to the even code, saturating.

    |v| >= 448 maps to +-448 (0x7E / 0xFE); a negative value that rounds to
    zero keeps its sign (0x80).  The nearest code is found by comparing the
    distances to the two neighbouring codes in fp64, which is exact for any
    fp32 input.  NaN inputs are outside the method's domain and rejected.
    """
    v = np.asarray(v, dtype=np.float32)
    if np.isnan(v).any():
        raise ValueError("e4m3_encode: NaN input")
    a = np.abs(v.astype(np.float64))
    neg = np.signbit(v)
    sat = a >= FP8_MAX
    a_c = np.where(sat, 0.0, a)
    lo = np.searchsorted(_E4M3_POS, a_c, side="right") - 1   # _E4M3_POS[lo] <= a
    lo = np.clip(lo, 0, 0x7D)
    hi = lo + 1
    d_lo = a_c - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - a_c
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(sat, 0x7E, code)
    code = np.where(neg, code | 0x80, code)
    return code.astype(np.uint8)


# --------------------------------------------------------------------------
# O2. INT4 uint4b8 packing, 8 nibbles per int32 word, along K
# --------------------------------------------------------------------------
def int4_pack(q) -> np.ndarray:
    """Pack signed INT4 values q in [-8, 7] (last axis K, K % 8 == 0) to int32.

    Word c of a row holds k = 8c .. 8c+7; nibble j (bits 4j..4j+3) stores
    u = q[8c + j] + 8 (uint4b8).
    """
    q = np.asarray(q)
    if q.shape[-1] % NIBBLES_PER_WORD:
        raise ValueError("K must be a multiple of 8")
    if q.min(initial=0) < -8 or q.max(initial=0) > 7:
        raise ValueError("INT4 values must lie in [-8, 7]")
    u = (q.astype(np.int64) + UINT4B8_BIAS).astype(np.uint64)
    u = u.reshape(*q.shape[:-1], q.shape[-1] // NIBBLES_PER_WORD, NIBBLES_PER_WORD)
    shifts = (4 * np.arange(NIBBLES_PER_WORD, dtype=np.uint64))
    words = np.bitwise_or.reduce(u << shifts, axis=-1)
    return words.astype(np.uint32).view(np.int32)


def int4_unpack(words) -> np.ndarray:
    """Inverse of int4_pack: int32 words [..., K/8] -> int8 q [..., K].

    Read byte by byte: byte j of word c (little-endian) holds k = 8c + 2j in
    its low nibble and k = 8c + 2j + 1 in its high nibble.
    """
    if sys.byteorder != "little":
        raise RuntimeError("the oracle reads packed words as little-endian bytes")
    w = np.ascontiguousarray(np.asarray(words, dtype=np.int32))
    b = w.view(np.uint8).reshape(*w.shape[:-1], w.shape[-1] * 4)
    q = np.empty((*w.shape[:-1], w.shape[-1] * NIBBLES_PER_WORD), dtype=np.int8)
    q[..., 0::2] = b & 0xF
    q[..., 1::2] = b >> 4
    q -= UINT4B8_BIAS
    return q


def dequant_weights(words, scales) -> np.ndarray:
    """fp64 weights q[n, k] * s[n, k // 128] of one expert (exact in fp64)."""
    q = int4_unpack(words)
    K = q.shape[-1]
    W = q.astype(np.float64).reshape(*q.shape[:-1], K // GROUP, GROUP)
    W *= np.asarray(scales, dtype=np.float32).astype(np.float64)[..., None]
    return W.reshape(*q.shape[:-1], K)


# --------------------------------------------------------------------------
# O3. per-token dynamic FP8 quantization
# --------------------------------------------------------------------------
def bf16_bits_to_f32(bits) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to fp32 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def quant_rows(x) -> tuple[np.ndarray, np.ndarray]:
    """Per-row FP8 quantization of an fp32 matrix [M, K].

    amax = max |x| over the row, scale = fl32(amax / 448) (1.0 when the row
    is all zero), code = enc(fl32(x / scale)).  Returns (codes u8, scales f32).
    """
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=1) if x.shape[1] else np.zeros(x.shape[0], np.float32)
    scale = np.where(amax > 0, amax / np.float32(FP8_MAX), np.float32(1.0)).astype(np.float32)
    q = (x / scale[:, None]).astype(np.float32)
    return e4m3_encode(q), scale


def quant_act(x_bf16_bits) -> tuple[np.ndarray, np.ndarray]:
    """S1: bf16 activations [T, H] -> (FP8 codes [T, H], per-token scale [T])."""
    return quant_rows(bf16_bits_to_f32(x_bf16_bits))


# --------------------------------------------------------------------------
# O4. top-k softmax routing
# --------------------------------------------------------------------------
def route(logits, k: int, renormalize: bool = True) -> tuple[np.ndarray, np.ndarray]:
    """S2: router logits [T, E] fp32 -> (ids int32 [T, k], weights fp32 [T, k]).

    ids are the k largest logits of each row in descending order, equal
    logits ordered by the lower expert index first.  p = softmax(logits) in
    fp64; weight j = p[id_j] / sum_j' p[id_j'] (renormalised) or p[id_j].
    """
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    idx = np.arange(E)
    for t in range(T):
        l64 = logits[t].astype(np.float64)
        order = np.lexsort((idx, -l64))[:k]       # primary: logit desc; then index asc
        e = np.exp(l64 - l64.max())
        p = e / e.sum()
        sel = p[order]
        ids[t] = order
        w[t] = (sel / sel.sum()) if renormalize else sel
    return ids, w


# --------------------------------------------------------------------------
# O5. permutation into expert-contiguous rows
# --------------------------------------------------------------------------
def permute(ids, E: int) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """S3: ids [T, k] -> (offsets [E+1], row_token [T*k], inv_pos [T*k]).

    Flat routed index f = t*k + j.  Rows are grouped by expert in ascending
    expert order and, inside an expert, by ascending f (a stable counting
    sort).  offsets is the exclusive prefix sum of the per-expert counts;
    row_token[p] is the token of routed row p; inv_pos[f] is the row that
    routed index f landed on.
    """
    ids = np.asarray(ids, dtype=np.int64)
    T, k = ids.shape
    flat = ids.reshape(-1)
    if flat.size and (flat.min() < 0 or flat.max() >= E):
        raise ValueError("expert id out of range")
    counts = np.bincount(flat, minlength=E)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    order = np.argsort(flat, kind="stable")
    row_token = order // k
    inv_pos = np.empty_like(order)
    inv_pos[order] = np.arange(flat.size)
    return offsets.astype(np.int32), row_token.astype(np.int32), inv_pos.astype(np.int32)


# --------------------------------------------------------------------------
# O6 / O8. grouped W4A8 GEMM
# --------------------------------------------------------------------------
def grouped_gemm(a_codes, a_scale, a_rows, offsets, w_packed, w_scale) -> np.ndarray:
    """S4 / S6: out[p, n] = a_scale[r] * sum_k dec(a[r, k]) * q[e, n, k] * s[e, n, k//128].

    r = a_rows[p] when a gather list is given, else p; e is the expert whose
    row range [offsets[e], offsets[e+1]) holds p.  Operands are dequantized
    exactly to fp64, multiplied with one BLAS fp64 matmul per expert, and the
    result is rounded once to fp32.  Shapes: a_codes [*, K] u8, a_scale [*]
    f32, offsets [E+1], w_packed [E, N, K/8] i32, w_scale [E, N, K/128] f32.
    """
    offsets = np.asarray(offsets, dtype=np.int64)
    E = offsets.size - 1
    N = w_packed.shape[1]
    M = int(offsets[-1])
    out = np.zeros((M, N), dtype=np.float32)
    a_scale = np.asarray(a_scale, dtype=np.float32)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        rows = np.asarray(a_rows[r0:r1]) if a_rows is not None else np.arange(r0, r1)
        A = e4m3_decode(a_codes[rows]) * a_scale[rows].astype(np.float64)[:, None]
        W = dequant_weights(w_packed[e], w_scale[e])
        out[r0:r1] = (A @ W.T).astype(np.float32)
    return out


def grouped_gemm_exact_groups(a_codes, a_scale, a_rows, offsets, w_packed, w_scale) -> np.ndarray:
    """Slow variant of grouped_gemm for tiny inputs, with exact group sums.

    Every product dec(a) * q is an integer multiple of 2^-9 bounded by
    448 * 8, so the 128-term sum of one group is an integer times 2^-9 that
    fits in 28 bits: it is formed exactly (Python integers), then scaled by
    the group scale and summed over groups in fp64.
    """
    offsets = np.asarray(offsets, dtype=np.int64)
    E = offsets.size - 1
    N = w_packed.shape[1]
    K = a_codes.shape[1]
    G = K // GROUP
    M = int(offsets[-1])
    out = np.zeros((M, N), dtype=np.float32)
    for e in range(E):
        q = int4_unpack(w_packed[e]).astype(np.int64)
        for p in range(int(offsets[e]), int(offsets[e + 1])):
            r = int(a_rows[p]) if a_rows is not None else p
            a_int = np.rint(e4m3_decode(a_codes[r]) * 512.0).astype(np.int64)  # exact: multiples of 2^-9
            for n in range(N):
                tot = 0.0
                for g in range(G):
                    sl = slice(g * GROUP, (g + 1) * GROUP)
                    isum = int(np.dot(a_int[sl], q[n, sl]))
                    tot += float(np.float32(w_scale[e, n, g])) * (isum * 2.0 ** -9)
                out[p, n] = np.float32(tot * float(np.float32(a_scale[r])))
    return out


# --------------------------------------------------------------------------
# O7. SwiGLU and re-quantization of the intermediate activation
# --------------------------------------------------------------------------
def swiglu_f32(h) -> np.ndarray:
    """silu(gate) * up with gate = h[:, :I], up = h[:, I:], in fp64, rounded to fp32."""
    h = np.asarray(h, dtype=np.float32).astype(np.float64)
    I = h.shape[1] // 2
    g, u = h[:, :I], h[:, I:]
    with np.errstate(over="ignore"):
        silu = g / (1.0 + np.exp(-g))
    return (silu * u).astype(np.float32)


def swiglu(h) -> tuple[np.ndarray, np.ndarray]:
    """S5: h [M, 2I] fp32 -> (FP8 codes [M, I], per-row scale [M])."""
    return quant_rows(swiglu_f32(h))


# --------------------------------------------------------------------------
# O9. routing-weighted combine back to token order
# --------------------------------------------------------------------------
def unpermute(o, inv_pos, w) -> np.ndarray:
    """S7: y[t] = sum_j w[t, j] * o[inv_pos[t*k + j]], j ascending, fp64 -> fp32."""
    w = np.asarray(w, dtype=np.float32)
    T, k = w.shape
    o64 = np.asarray(o, dtype=np.float32).astype(np.float64)
    inv = np.asarray(inv_pos, dtype=np.int64).reshape(T, k)
    y = np.zeros((T, o64.shape[1]), dtype=np.float64)
    for j in range(k):
        y += w[:, j].astype(np.float64)[:, None] * o64[inv[:, j]]
    return y.astype(np.float32)


def f32_to_bf16_bits(y) -> np.ndarray:
    """Round fp32 to bfloat16 (nearest, ties to even); returns uint16 bits."""
    b = np.asarray(y, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return r.astype(np.uint16)


# --------------------------------------------------------------------------
# the whole layer
# --------------------------------------------------------------------------
def moe_layer(x_bf16_bits, logits, w13, s13, w2, s2, k: int, renormalize: bool = True) -> dict:
    """All seven steps in order; returns every intermediate by name."""
    E = w13.shape[0]
    qx, sx = quant_act(x_bf16_bits)
    ids, w = route(logits, k, renormalize)
    offsets, row_token, inv_pos = permute(ids, E)
    h = grouped_gemm(qx, sx, row_token, offsets, w13, s13)
    a_f32 = swiglu_f32(h)
    qa, sa = quant_rows(a_f32)
    o = grouped_gemm(qa, sa, None, offsets, w2, s2)
    y = unpermute(o, inv_pos, w)
    return dict(qx=qx, sx=sx, ids=ids, w=w, offsets=offsets, row_token=row_token,
                inv_pos=inv_pos, h=h, a_f32=a_f32, qa=qa, sa=sa, o=o, y=y)


# --------------------------------------------------------------------------
# Offline weight quantizer (self-check of the format against the pages'
# reconstruction-error figures; not on the layer's path)
# --------------------------------------------------------------------------
SHRINK_RATIOS = tuple(round(1.0 - 0.03 * i, 2) for i in range(11))   # 1.00, 0.97, ..., 0.70


def quantize_int4_g128(W, mse_clip: bool = True) -> tuple[np.ndarray, np.ndarray]:
    """Symmetric INT4 group-128 quantizer of a weight matrix [N, K].

    Section 量化方式 of the "GLM-5.3-W4A8" card: symmetric INT4, group 128,
    each group's scale chosen by the smallest squared error over 11 shrink
    ratios from 1.00 down to 0.70.  Reading: scale = r * amax / 7,
    q = clamp(round-half-even(w / scale), -8, 7), ratios in steps of 0.03,
    ties kept at the larger ratio.  mse_clip=False is plain round-to-nearest
    with r = 1.  Returns (q int8 [N, K], scales fp32 [N, K/128]).
    """
    W = np.asarray(W, dtype=np.float64)
    N, K = W.shape
    G = K // GROUP
    Wg = W.reshape(N, G, GROUP)
    amax = np.abs(Wg).max(axis=2)
    amax = np.where(amax > 0, amax, 1.0)
    ratios = SHRINK_RATIOS if mse_clip else (1.0,)
    best_err = np.full((N, G), np.inf)
    best_s = np.zeros((N, G), dtype=np.float32)
    for r in ratios:
        s = (r * amax / 7.0).astype(np.float32)
        s64 = s.astype(np.float64)[..., None]
        q = np.clip(np.rint(Wg / s64), -8, 7)
        err = ((Wg - q * s64) ** 2).sum(axis=2)
        better = err < best_err
        best_err = np.where(better, err, best_err)
        best_s = np.where(better, s, best_s)
    q = np.clip(np.rint(Wg / best_s.astype(np.float64)[..., None]), -8, 7).astype(np.int8)
    return q.reshape(N, K), best_s


def relative_l2(W, W_hat) -> float:
    """||W - W_hat||_F / ||W||_F."""
    W = np.asarray(W, dtype=np.float64)
    return float(np.linalg.norm(W - W_hat) / np.linalg.norm(W))


def fp8_block_quant_dequant(W, block: int = 128) -> np.ndarray:
    """FP8 E4M3 block quantization (one amax/448 scale per block x block tile), dequantized.

    The non-expert layers of the checkpoints keep FP8 128x128 blocks
    ("GLM-5.3-W4A8" card, section 量化方式); used only as a check of the
    E4M3 codec against the pages' reconstruction-error figure.
    """
    W = np.asarray(W, dtype=np.float32)
    N, K = W.shape
    out = np.empty((N, K), dtype=np.float64)
    for i in range(0, N, block):
        for j in range(0, K, block):
            t = W[i:i + block, j:j + block]
            amax = np.float32(np.abs(t).max())
            sc = amax / np.float32(FP8_MAX) if amax > 0 else np.float32(1.0)
            codes = e4m3_encode((t / sc).astype(np.float32))
            out[i:i + block, j:j + block] = e4m3_decode(codes) * float(sc)
    return out
