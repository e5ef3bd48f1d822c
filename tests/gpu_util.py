"""Helpers of the GPU parity tests: device transfer and the comparison rules."""
from __future__ import annotations

import sys

import numpy as np
import torch

DEV = "cuda:0"

# Frobenius bound for a grouped GEMM whose inputs are bit-identical on both
# sides.  gfx950's FP8 MFMA sums the 128 products of one instruction with
# less than fp32 precision: measured error up to 7.5e-6 of the sum of the
# products' magnitudes, unbiased (as many positive as negative errors).  The
# INT4 offset form of the weights (u = q + 8) makes that sum ~15x the result,
# so one group carries up to ~1e-4 relative error and K/128 groups add in
# quadrature; 1e-4 Frobenius covers K = 6144 with margin.
GEMM_FRO_TIGHT = 1e-4


def edge_shape_maxrel(n_cols: int) -> float:
    """Per-element bar for the extra edge-case shapes (not the five workloads).

    The 1e-2 bar on elements above 1e-3 of the row norm amounts to an
    absolute error below 1e-5 of the row norm.  The GPU's error per element
    comes from the FP8 MFMA accumulation and does not shrink with the row
    length, while the row norm grows as sqrt(N); the bar is therefore kept
    at the absolute level it has for the workloads' rows (N = 6144), i.e.
    1e-2 * sqrt(6144 / N) for shorter rows.  The five workloads themselves
    are held to 1e-2.
    """
    return 1e-2 * max(1.0, (6144.0 / n_cols) ** 0.5)


def say(msg: str) -> None:
    """Name the case before each GPU step (flushed), so a failing run shows it."""
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def bf16_to_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def prepack_int4(w: np.ndarray, s: np.ndarray | None = None):
    """Device copies of row-major INT4 experts (and group scales) in the GEMM storage, through the library."""
    from quantized_grouped_gemm_token_amd import ops
    return ops.w4a8_moe_prepack_int4(to_dev(w), None if s is None else to_dev(s))


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def float_parity(got: np.ndarray, want: np.ndarray) -> dict:
    """Relative Frobenius error, and the largest relative error over the
    elements whose magnitude exceeds 1e-3 of their row's L2 norm."""
    g = np.asarray(got, np.float64)
    w = np.asarray(want, np.float64)
    assert g.shape == w.shape, (g.shape, w.shape)
    if w.size == 0:
        return dict(fro=0.0, maxrel=0.0)
    den = np.linalg.norm(w)
    fro = float(np.linalg.norm(g - w) / den) if den > 0 else float(np.linalg.norm(g - w))
    w2 = w.reshape(w.shape[0], -1)
    g2 = g.reshape(g.shape[0], -1)
    rn = np.linalg.norm(w2, axis=1, keepdims=True)
    mask = np.abs(w2) > 1e-3 * rn
    maxrel = float((np.abs(g2 - w2)[mask] / np.abs(w2)[mask]).max()) if mask.any() else 0.0
    return dict(fro=fro, maxrel=maxrel)


def assert_float_parity(got, want, what: str, fro_tight: float | None = None, maxrel: float = 1e-2) -> dict:
    """The float bar: relative Frobenius <= 2e-3 and max relative <= 1e-2 on
    elements above 1e-3 of the row norm; fro_tight adds a stricter Frobenius
    bound where both sides saw bit-identical inputs."""
    r = float_parity(got, want)
    assert r["fro"] <= 2e-3 and r["maxrel"] <= maxrel, f"{what}: {r}"
    if fro_tight is not None:
        assert r["fro"] <= fro_tight, f"{what}: {r} (tight bound {fro_tight})"
    return r


def near_midpoint(vals_f32: np.ndarray, scale: np.ndarray, rel: float = 1e-5) -> np.ndarray:
    """Mask of elements whose quotient vals/scale lies within `rel` (relative)
    of a rounding midpoint of E4M3 -- where a 1-ulp difference upstream may
    legitimately change the code."""
    import oracle
    q = np.abs(vals_f32.astype(np.float64) / scale.astype(np.float64)[:, None])
    pos = oracle.E4M3_VALUES[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2
    idx = np.clip(np.searchsorted(mids, q), 1, len(mids) - 1)
    d = np.minimum(np.abs(q - mids[idx - 1]), np.abs(q - mids[idx]))
    return d <= rel * np.maximum(q, 2.0 ** -9)



def _code_rank(codes: np.ndarray, int8: bool) -> np.ndarray:
    """Position of each code on the number line (adjacent representable values differ by 1)."""
    if int8:
        return codes.astype(np.int64)
    c = codes.astype(np.int64)
    return np.where(c & 0x80, -(c & 0x7F), c)


def _near_rounding_midpoint(vals: np.ndarray, scale: np.ndarray, int8: bool, rel: float) -> np.ndarray:
    """Elements whose quotient vals / scale lies within rel (relative) of a rounding midpoint."""
    if not int8:
        return near_midpoint(vals, scale, rel)
    q = np.abs(vals.astype(np.float64) / scale.astype(np.float64)[:, None])
    return np.abs(q - np.floor(q) - 0.5) <= rel * np.maximum(q, 1.0)


def check_requant(act_gpu: np.ndarray, qa_gpu: np.ndarray, sa_gpu: np.ndarray, qa_oracle: np.ndarray,
                  int8: bool = False, act_exact: bool = True) -> np.ndarray:
    """Check the GPU's re-quantized activations; return where they differ from an independent oracle run.

    The re-quantization itself is bit-exact: the GPU's codes and scales must
    be exactly the oracle's quantization of the GPU's own act.  With
    act_exact=False, act_gpu is only a recomputation of the GPU's act (the
    unfused path keeps it inside its SwiGLU kernel): scales then agree to
    1e-6 and codes except at rounding midpoints (1e-5 relative).
    Where the codes differ from the independent run's (qa_oracle), the two
    sides re-quantized act values that differ by their GEMMs' rounding (the
    caller holds act to the GEMM bar); the mask of those codes is returned.
    """
    import oracle
    q_own, s_own = (oracle.quant_rows_i8 if int8 else oracle.quant_rows)(act_gpu)
    if act_exact:
        assert np.array_equal(sa_gpu.view(np.uint32), s_own.view(np.uint32)), "GPU scales are not those of its act"
        assert np.array_equal(qa_gpu, q_own), "GPU codes are not the quantization of its own act"
    else:
        assert np.all(np.abs(sa_gpu.astype(np.float64) - s_own) <= 1e-6 * s_own), "GPU scales"
        d = qa_gpu != q_own
        assert np.all(_near_rounding_midpoint(act_gpu, s_own, int8, 1e-5)[d]), "GPU codes off a midpoint"
    return qa_gpu != qa_oracle


def check_swiglu_epilogue(act_gpu: np.ndarray, h_gpu: np.ndarray, what: str) -> float:
    """act of the fused gate/up GEMM against SwiGLU of the GPU's own gate/up output h.

    The fused epilogue computes silu(gate) * up from the fp32 gate and up
    values that the unfused GEMM stores, with the hardware exponential and
    reciprocal; the oracle's SwiGLU of the same h is exact and rounded once.
    Bound per element: 16 fp32 ulp of the value, plus 2^-24 of the row's
    largest |act|.  The absolute part covers the far negative tail of silu
    (gate below about -20), where the fast exponential's argument rounding
    costs tens of ulp and where exp(-gate) overflows fp32 below -88 and the
    GPU's act is 0 instead of a value under 1e-38: differences some 2^15
    times smaller than the FP8 code step of the row.  Returns the largest
    difference in ulp among the elements above the absolute part.
    """
    import oracle
    ref = oracle.swiglu_f32(h_gpu).astype(np.float64)
    ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    floor = 2.0 ** -24 * np.abs(ref).max(axis=1, keepdims=True)
    diff = np.abs(act_gpu.astype(np.float64) - ref)
    bad = diff > 16 * ulp + floor
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements differ from SwiGLU of the GPU's gate/up output by "
                           f"more than 16 ulp + 2^-24 of the row max")
    big = np.abs(ref) > floor
    return float((diff[big] / ulp[big]).max(initial=0.0))


def check_layer_output(y_gpu: np.ndarray, y_oracle: np.ndarray, y_same_codes: np.ndarray, token_flipped: np.ndarray,
                       what: str, maxrel: float = 1e-2) -> dict:
    """The end-to-end bars of the layer output.

    y_oracle is an independent oracle run; y_same_codes is the oracle's down
    GEMM and combine applied to the GPU's (checked) re-quantized activations;
    token_flipped marks the tokens with a re-quantized code that differs from
    the independent run's.
      * relative Frobenius <= 2e-3 against the independent run, all tokens;
      * max relative <= maxrel (elements above 1e-3 of the row norm) against
        the independent run, on every token without a differing code;
      * the same per-element bar, and the tight GEMM Frobenius bar, against
        y_same_codes on every token.
    """
    den = np.linalg.norm(y_oracle.astype(np.float64))
    fro = float(np.linalg.norm(y_gpu.astype(np.float64) - y_oracle) / den) if den > 0 else 0.0
    assert fro <= 2e-3, f"{what}: Frobenius {fro:.3e} against the independent oracle"
    clean = ~token_flipped
    r_clean = float_parity(y_gpu[clean], y_oracle[clean]) if clean.any() else dict(fro=0.0, maxrel=0.0)
    assert r_clean["maxrel"] <= maxrel, f"{what}: tokens without a code flip {r_clean}"
    r_same = assert_float_parity(y_gpu, y_same_codes, f"{what} (same codes)", fro_tight=GEMM_FRO_TIGHT, maxrel=maxrel)
    return dict(fro=fro, maxrel_clean=r_clean["maxrel"], clean_tokens=int(clean.sum()), tokens=int(clean.size),
                same_codes=r_same)
