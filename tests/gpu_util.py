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



# Band, in units of the FP8 quotient q = a / scale, inside which the GPU and
# the oracle may round an activation of the SwiGLU output to different
# (adjacent) E4M3 codes: both codes are correct results of the method when
# the oracle's q lies this close to the midpoint between them.  It bounds
# |q_gpu - q_oracle| given the gate/up GEMM bound above (about 1e-4 of the
# row's largest value, i.e. 448 * 1e-4 in q units) plus the scale's own
# relative difference.
def flip_band(q_abs: np.ndarray) -> np.ndarray:
    return 0.05 + 1e-3 * q_abs


def valid_code_choice(a_oracle: np.ndarray, sa_oracle: np.ndarray, codes_oracle: np.ndarray,
                      codes_gpu: np.ndarray) -> tuple[np.ndarray, int]:
    """Check the GPU's re-quantization codes against the oracle's.

    With q the oracle's quotient a / scale, a GPU code is valid when it is
    the E4M3 rounding of some value within flip_band(|q|) of q, i.e. when
    its value lies between enc(q - band) and enc(q + band).  Returns the code
    array to build the reference from (the oracle's, with the GPU's valid
    alternative choices) and the number of such choices; raises if a GPU
    code is not a valid result.
    """
    import oracle
    q = a_oracle.astype(np.float64) / sa_oracle.astype(np.float64)[:, None]
    diff = codes_gpu != codes_oracle
    if not diff.any():
        return codes_oracle, 0
    qd = q[diff]
    band = flip_band(np.abs(qd))
    lo = oracle.e4m3_decode(oracle.e4m3_encode((qd - band).astype(np.float32)))
    hi = oracle.e4m3_decode(oracle.e4m3_encode((qd + band).astype(np.float32)))
    vg = oracle.e4m3_decode(codes_gpu[diff])
    ok = (vg >= lo) & (vg <= hi)
    if not ok.all():
        bad = np.nonzero(~ok)[0][:5]
        raise AssertionError(f"{int((~ok).sum())} GPU codes are not valid roundings; e.g. q={qd[bad]}, "
                             f"oracle={oracle.e4m3_decode(codes_oracle[diff][bad])}, gpu={vg[bad]}")
    chosen = codes_oracle.copy()
    chosen[diff] = codes_gpu[diff]
    return chosen, int(diff.sum())
