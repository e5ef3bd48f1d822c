"""Seeded synthetic inputs for the W4A8 MoE layer.

This module only draws random inputs; it holds none of the layer's
arithmetic, and both the GPU path and the CPU oracle are fed from it.

The five workloads mirror the serving shapes reported on the "GLM-5.3-W4A8"
model card (gpustack), section 性能 (performance table): decode at 128 and 256
concurrent tokens, prefill of one 8K-token prompt, with 256 routed experts per
MoE layer ("从 755GB 到 395GB" blog, section 我们量化了什么) and the expert
intermediate size 2048 implied by the card's section 局限性 (TP8 slices of
2048).  No dataset or trained weight is involved:

* packed INT4 words are uniform random 32-bit words, i.e. every nibble is an
  independent uniform value in 0..15 (q in -8..7);
* group scales are lognormal(mean=-4, sigma=0.5), fp32;
* activations are N(0, 1) fp32 rounded to bf16; the decode shapes scale 1% of
  the hidden channels (a seeded choice shared by all tokens) by 20 first;
* router logits are N(0, 1) fp32; the skewed prefill adds log p(rank) of a
  Zipf(1.1) law over a seeded ranking of the experts (and so does a sixth
  shape, skewed decode at 256 tokens, seed 1005, which is no benchmark
  config).

Streams: numpy PCG64 seeded by SeedSequence(1000 + index), spawned in the
fixed order W13, S13, W2, S2, x, outlier channels, logits, expert ranking;
a ninth child draws the per-channel scales of the per-channel INT4 x INT8
variant (lognormal(-4, 0.5), fp32 [E, 2I] and [E, H]), which reuses the
same packed words; a tenth draws the MXFP4 experts: uniform random bytes
(every E2M1 code equally likely, as the INT4 nibbles are) and E8M0 scale bytes
127 + rint(log2 s), s ~ lognormal(-4, 0.5) (the group-128 scale law, rounded
to a power of two).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

GROUP = 128


@dataclass(frozen=True)
class Shape:
    name: str
    T: int          # tokens
    H: int          # hidden size (K of the gate/up projection)
    I: int          # expert intermediate size (K of the down projection)
    E: int          # routed experts
    k: int          # experts per token
    outlier_frac: float = 0.0
    outlier_gain: float = 20.0
    zipf_s: float | None = None

    @property
    def R(self) -> int:
        return self.T * self.k


WORKLOADS = (
    Shape("tiny T=16 H=256 I=128 E=8 top-2", 16, 256, 128, 8, 2),
    Shape("decode T=128 H=6144 I=2048 E=256 top-8", 128, 6144, 2048, 256, 8, outlier_frac=0.01),
    Shape("decode T=256 H=6144 I=2048 E=256 top-8", 256, 6144, 2048, 256, 8, outlier_frac=0.01),
    Shape("prefill T=8192 H=6144 I=2048 E=256 top-8", 8192, 6144, 2048, 256, 8),
    Shape("skewed prefill T=16384 H=6144 I=2048 E=256 top-8 zipf1.1", 16384, 6144, 2048, 256, 8,
          zipf_s=1.1),
)


# decode at 256 tokens with the routing of the skewed prefill (Zipf(1.1) over a
# seeded ranking): a test case and a benchmark option, not one of the five above
SKEWED_DECODE = Shape("skewed decode T=256 H=6144 I=2048 E=256 top-8 zipf1.1", 256, 6144, 2048, 256, 8,
                      outlier_frac=0.01, zipf_s=1.1)
SKEWED_DECODE_SEED = 1005


@dataclass
class Workload:
    shape: Shape
    seed: int
    x_bf16: np.ndarray      # uint16 bf16 bit patterns [T, H]
    logits: np.ndarray      # fp32 [T, E]
    w13: np.ndarray         # int32 [E, 2I, H/8]
    s13: np.ndarray         # fp32 [E, 2I, H/128]
    w2: np.ndarray          # int32 [E, H, I/8]
    s2: np.ndarray          # fp32 [E, H, I/128]
    outlier_channels: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int64))


def _streams(seed: int, n: int = 8):
    return [np.random.Generator(np.random.PCG64(c)) for c in np.random.SeedSequence(seed).spawn(n)]


def _to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def make_workload(shape: Shape, seed: int, with_weights: bool = True) -> Workload:
    """Draw one workload.  with_weights=False skips the (large) expert weights."""
    T, H, I, E = shape.T, shape.H, shape.I, shape.E
    if H % GROUP or I % GROUP:
        raise ValueError("H and I must be multiples of 128")
    g_w13, g_s13, g_w2, g_s2, g_x, g_out, g_lg, g_perm = _streams(seed)
    if with_weights:
        w13 = g_w13.integers(0, 2**32, size=(E, 2 * I, H // 8), dtype=np.uint32).view(np.int32)
        s13 = g_s13.lognormal(mean=-4.0, sigma=0.5, size=(E, 2 * I, H // GROUP)).astype(np.float32)
        w2 = g_w2.integers(0, 2**32, size=(E, H, I // 8), dtype=np.uint32).view(np.int32)
        s2 = g_s2.lognormal(mean=-4.0, sigma=0.5, size=(E, H, I // GROUP)).astype(np.float32)
    else:
        w13 = np.zeros((0, 2 * I, H // 8), np.int32)
        s13 = np.zeros((0, 2 * I, H // GROUP), np.float32)
        w2 = np.zeros((0, H, I // 8), np.int32)
        s2 = np.zeros((0, H, I // GROUP), np.float32)
    x = g_x.standard_normal((T, H), dtype=np.float32)
    ch = np.zeros(0, np.int64)
    if shape.outlier_frac > 0:
        n_out = int(round(shape.outlier_frac * H))
        ch = np.sort(g_out.choice(H, size=n_out, replace=False))
        x[:, ch] *= np.float32(shape.outlier_gain)
    logits = g_lg.standard_normal((T, E), dtype=np.float32)
    if shape.zipf_s is not None:
        perm = g_perm.permutation(E)
        rank = np.empty(E, dtype=np.float64)
        rank[perm] = np.arange(1, E + 1, dtype=np.float64)
        p = rank ** (-shape.zipf_s)
        p /= p.sum()
        logits = (logits + np.log(p).astype(np.float32)[None, :]).astype(np.float32)
    return Workload(shape, seed, _to_bf16_bits(x), logits, w13, s13, w2, s2, ch)


def make_config(index: int, with_weights: bool = True) -> Workload:
    """Workload index 0..4 (tiny, decode 128, decode 256, prefill 8K, skewed 16K)."""
    return make_workload(WORKLOADS[index], 1000 + index, with_weights)


def make_skewed_decode(with_weights: bool = True) -> Workload:
    """The skewed decode workload (SKEWED_DECODE)."""
    return make_workload(SKEWED_DECODE, SKEWED_DECODE_SEED, with_weights)


def make_custom(T: int, H: int, I: int, E: int, k: int, seed: int, **kw) -> Workload:
    """A workload of any shape (tests: ragged tails, edge cases)."""
    return make_workload(Shape(f"custom T={T} H={H} I={I} E={E} top-{k}", T, H, I, E, k, **kw), seed)


def channel_scales(wl: Workload) -> tuple[np.ndarray, np.ndarray]:
    """Per-channel weight scales of the per-channel variant: fp32 [E, 2I] and [E, H]."""
    sh = wl.shape
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(wl.seed).spawn(9)[8]))
    s13 = g.lognormal(mean=-4.0, sigma=0.5, size=(sh.E, 2 * sh.I)).astype(np.float32)
    s2 = g.lognormal(mean=-4.0, sigma=0.5, size=(sh.E, sh.H)).astype(np.float32)
    return s13, s2


def mxfp4_weights(wl: Workload) -> tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """MXFP4 experts of the workload's shape: w13 uint8 [E, 2I, H/2], s13 uint8 [E, 2I, H/32],
    w2 uint8 [E, H, I/2], s2 uint8 [E, H, I/32]."""
    sh = wl.shape
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(wl.seed).spawn(10)[9]))

    def scales(shape):
        return (127 + np.rint(np.log2(g.lognormal(mean=-4.0, sigma=0.5, size=shape)))).astype(np.uint8)

    w13 = g.integers(0, 256, size=(sh.E, 2 * sh.I, sh.H // 2), dtype=np.uint8)
    s13 = scales((sh.E, 2 * sh.I, sh.H // 32))
    w2 = g.integers(0, 256, size=(sh.E, sh.H, sh.I // 2), dtype=np.uint8)
    s2 = scales((sh.E, sh.H, sh.I // 32))
    return w13, s13, w2, s2
