"""Python binding of the W4A8 MoE C ABI (include/w4a8_moe.h).

Argument marshalling only: each function checks dtypes, devices, shapes and
contiguity of torch tensors, allocates outputs the caller did not pass, and
calls the library function of the same name on torch's current stream.
Every step of the layer runs in the library's HIP kernels.  The library must
have been built (``quantized_grouped_gemm_token_amd.build``); without it
every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

# the in-tree build; W4A8_MOE_LIB names another build of the same library (the tests load a host
# sanitizer build of the C ABI this way)
LIB_PATH = os.environ.get("W4A8_MOE_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libw4a8moe.so")

W4A8_Y_F32 = 0
W4A8_Y_BF16 = 1
W4A8_GG_AUTO = 0
W4A8_GG_STREAM = 1
W4A8_GG_TILED = 2

_lib = None

_c_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32

_SIGNATURES = {
    "w4a8_moe_quant_act": (ctypes.c_int, [_c_p, _i64, _i64, _i64, _c_p, _c_p, _c_p]),
    "w4a8_moe_route": (ctypes.c_int, [_c_p, _i64, _i32, _i32, _i32, _c_p, _c_p, _c_p]),
    "w4a8_moe_permute_workspace_bytes": (ctypes.c_int64, [_i64, _i32, _i32]),
    "w4a8_moe_permute": (ctypes.c_int, [_c_p, _i64, _i32, _i32, _c_p, _c_p, _c_p, _c_p, _i64, _c_p]),
    "w4a8_moe_swiglu": (ctypes.c_int, [_c_p, _i64, _i64, _c_p, _c_p, _c_p]),
    "w4a8_moe_unpermute": (ctypes.c_int, [_c_p, _c_p, _c_p, _i64, _i32, _i64, _c_p, _i32, _c_p]),
    "w4a8_moe_quantize_weights": (ctypes.c_int, [_c_p, _i64, _i64, _i32, _c_p, _c_p, _c_p]),
    "w4a8_moe_quant_act_i8": (ctypes.c_int, [_c_p, _i64, _i64, _i64, _c_p, _c_p, _c_p, _c_p]),
    "w4a8_moe_swiglu_i8": (ctypes.c_int, [_c_p, _i64, _i64, _c_p, _c_p, _c_p, _c_p]),
    "w4a8_moe_quantize_weights_channel": (ctypes.c_int, [_c_p, _i64, _i64, _c_p, _c_p, _c_p]),
    "w4a8_moe_requant": (ctypes.c_int, [_c_p, _c_p, _i64, _i64, _c_p, _c_p, _c_p]),
    "w4a8_moe_requant_i8": (ctypes.c_int, [_c_p, _c_p, _i64, _i64, _c_p, _c_p, _c_p, _c_p]),
    "w4a8_moe_quantize_weights_mxfp4": (ctypes.c_int, [_c_p, _i64, _i64, _c_p, _c_p, _c_p]),
    "w4a8_moe_prepack_int4": (ctypes.c_int, [_c_p, _c_p, _i32, _i64, _i64, _c_p, _c_p, _c_p]),
    "w4a8_moe_prepack_mxfp4": (ctypes.c_int, [_c_p, _c_p, _i32, _i64, _i64, _c_p, _c_p, _c_p]),
    "w4a8_moe_permute_noalloc": (ctypes.c_int, [_c_p, _i64, _i32, _i32, _c_p, _c_p, _c_p, _c_p]),
    "w4a8_moe_front": (ctypes.c_int, [_c_p, _i64, _i64, _i64, _c_p, _c_p, _c_p, _i32, _i32, _i32, _c_p, _c_p, _c_p,
                                      _c_p, _c_p, _c_p, _i64, _c_p, _c_p]),
    "w4a8_moe_front_i8": (ctypes.c_int, [_c_p, _i64, _i64, _i64, _c_p, _c_p, _c_p, _c_p, _i32, _i32, _i32, _c_p,
                                         _c_p, _c_p, _c_p, _c_p, _c_p, _i64, _c_p, _c_p]),
    "w4a8_moe_grouped_gemm": (ctypes.c_int, [_c_p, _c_p, _c_p, _i64, _c_p, _i32, _c_p, _c_p, _i64, _i64, _c_p, _c_p]),
    "w4a8_moe_grouped_gemm_prepacked": (ctypes.c_int,
        [_c_p, _c_p, _c_p, _i64, _c_p, _i32, _c_p, _c_p, _i64, _i64, _c_p, _i32, _c_p]),
    "w4a8_moe_grouped_gemm_swiglu": (ctypes.c_int,
        [_c_p, _c_p, _c_p, _i64, _c_p, _i32, _c_p, _c_p, _i64, _i64, _c_p, _c_p, _c_p]),
    "w4a8_moe_grouped_gemm_swiglu_prepacked": (ctypes.c_int,
        [_c_p, _c_p, _c_p, _i64, _c_p, _i32, _c_p, _c_p, _i64, _i64, _c_p, _c_p, _i32, _c_p]),
    "w4a8_moe_grouped_gemm_i8": (ctypes.c_int,
        [_c_p, _c_p, _c_p, _c_p, _i64, _c_p, _i32, _c_p, _c_p, _i64, _i64, _c_p, _c_p]),
    "w4a8_moe_grouped_gemm_i8_prepacked": (ctypes.c_int,
        [_c_p, _c_p, _c_p, _c_p, _i64, _c_p, _i32, _c_p, _c_p, _i64, _i64, _c_p, _i32, _c_p]),
    "w4a8_moe_grouped_gemm_swiglu_i8": (ctypes.c_int,
        [_c_p, _c_p, _c_p, _c_p, _i64, _c_p, _i32, _c_p, _c_p, _i64, _i64, _c_p, _c_p, _c_p]),
    "w4a8_moe_grouped_gemm_swiglu_i8_prepacked": (ctypes.c_int,
        [_c_p, _c_p, _c_p, _c_p, _i64, _c_p, _i32, _c_p, _c_p, _i64, _i64, _c_p, _c_p, _i32, _c_p]),
    "w4a8_moe_grouped_gemm_mxfp4": (ctypes.c_int,
        [_c_p, _c_p, _c_p, _i64, _c_p, _i32, _c_p, _c_p, _i64, _i64, _c_p, _c_p]),
    "w4a8_moe_grouped_gemm_mxfp4_prepacked": (ctypes.c_int,
        [_c_p, _c_p, _c_p, _i64, _c_p, _i32, _c_p, _c_p, _i64, _i64, _c_p, _i32, _c_p]),
    "w4a8_moe_grouped_gemm_swiglu_mxfp4": (ctypes.c_int,
        [_c_p, _c_p, _c_p, _i64, _c_p, _i32, _c_p, _c_p, _i64, _i64, _c_p, _c_p, _c_p]),
    "w4a8_moe_grouped_gemm_swiglu_mxfp4_prepacked": (ctypes.c_int,
        [_c_p, _c_p, _c_p, _i64, _c_p, _i32, _c_p, _c_p, _i64, _i64, _c_p, _c_p, _i32, _c_p]),
    "w4a8_moe_row_sources": (ctypes.c_int, [_c_p, _c_p, _c_p, _i64, _i32, _i64, _c_p, _c_p, _c_p]),
    "w4a8_moe_grouped_gemm_scatter_prepacked": (ctypes.c_int,
        [_c_p, _c_p, _c_p, _i64, _c_p, _i32, _c_p, _c_p, _i64, _i64, _c_p, _c_p, _i32, _c_p]),
    "w4a8_moe_grouped_gemm_scatter_i8_prepacked": (ctypes.c_int,
        [_c_p, _c_p, _c_p, _c_p, _i64, _c_p, _i32, _c_p, _c_p, _i64, _i64, _c_p, _c_p, _i32, _c_p]),
    "w4a8_moe_grouped_gemm_scatter_mxfp4_prepacked": (ctypes.c_int,
        [_c_p, _c_p, _c_p, _i64, _c_p, _i32, _c_p, _c_p, _i64, _i64, _c_p, _c_p, _i32, _c_p]),
    "w4a8_moe_combine": (ctypes.c_int, [_c_p, _c_p, _i64, _i32, _i64, _c_p, _i32, _c_p]),
    "w4a8_moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "w4a8_moe_last_error": (ctypes.c_char_p, []),
    "w4a8_moe_device_supported": (ctypes.c_int, []),
}


class W4A8Error(RuntimeError):
    """A nonzero status from the library."""

    def __init__(self, func: str, status: int, detail: str):
        super().__init__(f"{func}: {detail} [{status_string(status)}]")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m quantized_grouped_gemm_token_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().w4a8_moe_status_string(status).decode()


def last_error() -> str:
    return lib().w4a8_moe_last_error().decode()


def _check(func: str, status: int) -> None:
    if status != 0:
        raise W4A8Error(func, status, last_error())


def w4a8_moe_device_supported() -> bool:
    return bool(lib().w4a8_moe_device_supported())


# ---------------------------------------------------------------- helpers
def _p(t):
    return None if t is None else t.data_ptr()


def _stream(dev: torch.device):
    return torch.cuda.current_stream(dev).cuda_stream


def _need(t: torch.Tensor, name: str, dtype, ndim: int, dev: torch.device | None = None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if dev is not None and t.device != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _int4_storage(w: torch.Tensor, name: str, dev) -> tuple[int, int, int]:
    """(E, N, K) of INT4 weights in the GEMM storage, int32 [E, N/16, K/128, 16, 16]."""
    _need(w, name, torch.int32, 5, dev)
    E, NB, G, sixteen, words = w.shape
    if (sixteen, words) != (16, 16):
        raise ValueError(f"{name} must be the GEMM storage [E, N/16, K/128, 16, 16] (w4a8_moe_prepack_int4)")
    return E, 16 * NB, 128 * G


# ------------------------------------------------------------------ calls
def w4a8_moe_quant_act(x: torch.Tensor, qx: torch.Tensor | None = None, sx: torch.Tensor | None = None):
    """bf16 [T, H] -> (E4M3 codes uint8 [T, H], per-token scales fp32 [T])."""
    _need(x, "x", torch.bfloat16, 2)
    T, H = x.shape
    dev = x.device
    qx = torch.empty((T, H), dtype=torch.uint8, device=dev) if qx is None else qx
    sx = torch.empty((T,), dtype=torch.float32, device=dev) if sx is None else sx
    _need(qx, "qx", torch.uint8, 2, dev)
    _need(sx, "sx", torch.float32, 1, dev)
    if tuple(qx.shape) != (T, H) or tuple(sx.shape) != (T,):
        raise ValueError("qx / sx shapes do not match x")
    _check("w4a8_moe_quant_act", lib().w4a8_moe_quant_act(_p(x), T, H, H, _p(qx), _p(sx), _stream(dev)))
    return qx, sx


def w4a8_moe_route(logits: torch.Tensor, k: int, renormalize: bool = True,
                   ids: torch.Tensor | None = None, w: torch.Tensor | None = None):
    """fp32 logits [T, E] -> (expert ids int32 [T, k], weights fp32 [T, k])."""
    _need(logits, "logits", torch.float32, 2)
    T, E = logits.shape
    dev = logits.device
    ids = torch.empty((T, k), dtype=torch.int32, device=dev) if ids is None else ids
    w = torch.empty((T, k), dtype=torch.float32, device=dev) if w is None else w
    _need(ids, "ids", torch.int32, 2, dev)
    _need(w, "w", torch.float32, 2, dev)
    if tuple(ids.shape) != (T, k) or tuple(w.shape) != (T, k):
        raise ValueError("ids / w must be [T, k]")
    _check("w4a8_moe_route", lib().w4a8_moe_route(_p(logits), T, E, k, int(bool(renormalize)), _p(ids), _p(w),
                                                  _stream(dev)))
    return ids, w


def w4a8_moe_permute_workspace_bytes(T: int, k: int, E: int) -> int:
    n = lib().w4a8_moe_permute_workspace_bytes(T, k, E)
    if n < 0:
        raise ValueError(f"bad sizes T={T} k={k} E={E}")
    return n


def w4a8_moe_front(x: torch.Tensor, logits: torch.Tensor, k: int, counter: torch.Tensor, renormalize: bool = True,
                   int8: bool = False, qx=None, sx=None, rowsum=None, ids=None, w=None, offsets=None, row_token=None,
                   inv_pos=None, workspace=None):
    """Steps 1-3 in one call (w4a8_moe_front, or w4a8_moe_front_i8 with int8): x bf16 [T, H], router
    logits fp32 [T, E], counter int32 [1] on the device (zero before the first call; left zero)
    -> (qx, sx, rowsum or None, ids, w, offsets, row_token, inv_pos)."""
    _need(x, "x", torch.bfloat16, 2)
    _need(logits, "logits", torch.float32, 2, x.device)
    _need(counter, "counter", torch.int32, 1, x.device)
    T, H = x.shape
    E = logits.shape[1]
    if logits.shape[0] != T or counter.numel() < 1:
        raise ValueError("logits must be [T, E] for x [T, H]; counter must hold one int32")
    dev = x.device
    R = T * k
    cdt = torch.int8 if int8 else torch.uint8
    qx = torch.empty((T, H), dtype=cdt, device=dev) if qx is None else qx
    sx = torch.empty((T,), dtype=torch.float32, device=dev) if sx is None else sx
    if int8:
        rowsum = torch.empty((T,), dtype=torch.int32, device=dev) if rowsum is None else rowsum
        _need(rowsum, "rowsum", torch.int32, 1, dev)
    ids = torch.empty((T, k), dtype=torch.int32, device=dev) if ids is None else ids
    w = torch.empty((T, k), dtype=torch.float32, device=dev) if w is None else w
    offsets = torch.empty((E + 1,), dtype=torch.int32, device=dev) if offsets is None else offsets
    row_token = torch.empty((R,), dtype=torch.int32, device=dev) if row_token is None else row_token
    inv_pos = torch.empty((R,), dtype=torch.int32, device=dev) if inv_pos is None else inv_pos
    nbytes = w4a8_moe_permute_workspace_bytes(T, k, E)
    if workspace is None:
        workspace = torch.empty((max(nbytes, 4),), dtype=torch.uint8, device=dev)
    _need(qx, "qx", cdt, 2, dev)
    _need(sx, "sx", torch.float32, 1, dev)
    _need(ids, "ids", torch.int32, 2, dev)
    _need(w, "w", torch.float32, 2, dev)
    _need(offsets, "offsets", torch.int32, 1, dev)
    _need(row_token, "row_token", torch.int32, 1, dev)
    _need(inv_pos, "inv_pos", torch.int32, 1, dev)
    _need(workspace, "workspace", torch.uint8, 1, dev)
    if (tuple(qx.shape) != (T, H) or sx.numel() != T or tuple(ids.shape) != (T, k) or tuple(w.shape) != (T, k)
            or offsets.numel() != E + 1 or row_token.numel() != R or inv_pos.numel() != R):
        raise ValueError("output shapes do not match x [T, H], logits [T, E] and k")
    if int8:
        _check("w4a8_moe_front_i8", lib().w4a8_moe_front_i8(
            _p(x), T, H, H, _p(qx), _p(sx), _p(rowsum), _p(logits), E, k, int(bool(renormalize)), _p(ids),
            _p(w), _p(offsets), _p(row_token), _p(inv_pos), _p(workspace), workspace.numel(), _p(counter),
            _stream(dev)))
    else:
        _check("w4a8_moe_front", lib().w4a8_moe_front(
            _p(x), T, H, H, _p(qx), _p(sx), _p(logits), E, k, int(bool(renormalize)), _p(ids), _p(w),
            _p(offsets), _p(row_token), _p(inv_pos), _p(workspace), workspace.numel(), _p(counter), _stream(dev)))
    return qx, sx, rowsum if int8 else None, ids, w, offsets, row_token, inv_pos


def w4a8_moe_permute(ids: torch.Tensor, E: int, offsets=None, row_token=None, inv_pos=None, workspace=None):
    """ids int32 [T, k] -> (offsets int32 [E+1], row_token int32 [T*k], inv_pos int32 [T*k])."""
    _need(ids, "ids", torch.int32, 2)
    T, k = ids.shape
    dev = ids.device
    R = T * k
    offsets = torch.empty((E + 1,), dtype=torch.int32, device=dev) if offsets is None else offsets
    row_token = torch.empty((R,), dtype=torch.int32, device=dev) if row_token is None else row_token
    inv_pos = torch.empty((R,), dtype=torch.int32, device=dev) if inv_pos is None else inv_pos
    nbytes = w4a8_moe_permute_workspace_bytes(T, k, E)
    if workspace is None:
        workspace = torch.empty((max(nbytes, 4),), dtype=torch.uint8, device=dev)
    _need(offsets, "offsets", torch.int32, 1, dev)
    _need(row_token, "row_token", torch.int32, 1, dev)
    _need(inv_pos, "inv_pos", torch.int32, 1, dev)
    _need(workspace, "workspace", torch.uint8, 1, dev)
    if offsets.numel() != E + 1 or row_token.numel() != R or inv_pos.numel() != R:
        raise ValueError("offsets must be [E+1], row_token / inv_pos [T*k]")
    _check("w4a8_moe_permute", lib().w4a8_moe_permute(_p(ids), T, k, E, _p(offsets), _p(row_token), _p(inv_pos),
                                                      _p(workspace), workspace.numel(), _stream(dev)))
    return offsets, row_token, inv_pos


def w4a8_moe_permute_noalloc(ids: torch.Tensor, E: int, offsets=None, row_token=None, inv_pos=None):
    """w4a8_moe_permute with its workspace in the library's own device buffer (no allocation by the
    library; pass every output to allocate nothing here either) -> (offsets, row_token, inv_pos)."""
    _need(ids, "ids", torch.int32, 2)
    T, k = ids.shape
    dev = ids.device
    R = T * k
    offsets = torch.empty((E + 1,), dtype=torch.int32, device=dev) if offsets is None else offsets
    row_token = torch.empty((R,), dtype=torch.int32, device=dev) if row_token is None else row_token
    inv_pos = torch.empty((R,), dtype=torch.int32, device=dev) if inv_pos is None else inv_pos
    for t, n, size in ((offsets, "offsets", E + 1), (row_token, "row_token", R), (inv_pos, "inv_pos", R)):
        _need(t, n, torch.int32, 1, dev)
        if t.numel() != size:
            raise ValueError(f"{n} must have {size} entries")
    _check("w4a8_moe_permute_noalloc",
           lib().w4a8_moe_permute_noalloc(_p(ids), T, k, E, _p(offsets), _p(row_token), _p(inv_pos), _stream(dev)))
    return offsets, row_token, inv_pos


def w4a8_moe_swiglu(h: torch.Tensor, qa: torch.Tensor | None = None, sa: torch.Tensor | None = None):
    """fp32 [M, 2I] -> (E4M3 codes uint8 [M, I], per-row scales fp32 [M])."""
    _need(h, "h", torch.float32, 2)
    M, I2 = h.shape
    I = I2 // 2
    dev = h.device
    qa = torch.empty((M, I), dtype=torch.uint8, device=dev) if qa is None else qa
    sa = torch.empty((M,), dtype=torch.float32, device=dev) if sa is None else sa
    _need(qa, "qa", torch.uint8, 2, dev)
    _need(sa, "sa", torch.float32, 1, dev)
    if I2 % 2 or tuple(qa.shape) != (M, I) or tuple(sa.shape) != (M,):
        raise ValueError("h must be [M, 2I], qa [M, I], sa [M]")
    _check("w4a8_moe_swiglu", lib().w4a8_moe_swiglu(_p(h), M, I, _p(qa), _p(sa), _stream(dev)))
    return qa, sa


def w4a8_moe_unpermute(o: torch.Tensor, inv_pos: torch.Tensor, w: torch.Tensor,
                       y: torch.Tensor | None = None, y_dtype: torch.dtype = torch.float32):
    """o fp32 [T*k, H], inv_pos int32 [T*k], w fp32 [T, k] -> y [T, H] (fp32 or bf16)."""
    _need(o, "o", torch.float32, 2)
    dev = o.device
    _need(inv_pos, "inv_pos", torch.int32, 1, dev)
    _need(w, "w", torch.float32, 2, dev)
    T, k = w.shape
    H = o.shape[1]
    if inv_pos.numel() != T * k or o.shape[0] < T * k:
        raise ValueError("inv_pos must be [T*k] and o at least [T*k, H]")
    if y is None:
        y = torch.empty((T, H), dtype=y_dtype, device=dev)
    if y.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("y must be float32 or bfloat16")
    _need(y, "y", y.dtype, 2, dev)
    if tuple(y.shape) != (T, H):
        raise ValueError("y must be [T, H]")
    code = W4A8_Y_F32 if y.dtype == torch.float32 else W4A8_Y_BF16
    _check("w4a8_moe_unpermute", lib().w4a8_moe_unpermute(_p(o), _p(inv_pos), _p(w), T, k, H, _p(y), code,
                                                          _stream(dev)))
    return y


def w4a8_moe_quantize_weights(w: torch.Tensor, mse_clip: bool = True, w_packed: torch.Tensor | None = None,
                              w_scale: torch.Tensor | None = None):
    """fp32 [..., K] -> (packed int32 [..., K/8], group scales fp32 [..., K/128]).

    Every leading dimension is flattened into rows (experts x output channels)."""
    if not isinstance(w, torch.Tensor) or w.dim() < 1:
        raise TypeError("w must be a torch.Tensor with a K dimension")
    _need(w, "w", torch.float32, w.dim())
    K = w.shape[-1]
    lead = tuple(w.shape[:-1])
    rows = 1
    for d in lead:
        rows *= int(d)
    dev = w.device
    if K % 128:
        raise ValueError("K must be a multiple of 128")
    w_packed = torch.empty(lead + (K // 8,), dtype=torch.int32, device=dev) if w_packed is None else w_packed
    w_scale = torch.empty(lead + (K // 128,), dtype=torch.float32, device=dev) if w_scale is None else w_scale
    _need(w_packed, "w_packed", torch.int32, len(lead) + 1, dev)
    _need(w_scale, "w_scale", torch.float32, len(lead) + 1, dev)
    if tuple(w_packed.shape) != lead + (K // 8,) or tuple(w_scale.shape) != lead + (K // 128,):
        raise ValueError("w_packed must be [..., K/8] and w_scale [..., K/128]")
    _check("w4a8_moe_quantize_weights",
           lib().w4a8_moe_quantize_weights(_p(w), rows, K, 1 if mse_clip else 0, _p(w_packed), _p(w_scale),
                                           _stream(dev)))
    return w_packed, w_scale


# ---- the per-channel INT4 x per-token INT8 variant ------------------------
def w4a8_moe_quant_act_i8(x: torch.Tensor, qx=None, sx=None, rowsum=None):
    """bf16 [T, H] -> (int8 codes [T, H], scales fp32 [T], code row sums int32 [T])."""
    _need(x, "x", torch.bfloat16, 2)
    T, H = x.shape
    dev = x.device
    qx = torch.empty((T, H), dtype=torch.int8, device=dev) if qx is None else qx
    sx = torch.empty((T,), dtype=torch.float32, device=dev) if sx is None else sx
    rowsum = torch.empty((T,), dtype=torch.int32, device=dev) if rowsum is None else rowsum
    _need(qx, "qx", torch.int8, 2, dev)
    _need(sx, "sx", torch.float32, 1, dev)
    _need(rowsum, "rowsum", torch.int32, 1, dev)
    if tuple(qx.shape) != (T, H) or tuple(sx.shape) != (T,) or tuple(rowsum.shape) != (T,):
        raise ValueError("qx must be [T, H], sx and rowsum [T]")
    _check("w4a8_moe_quant_act_i8", lib().w4a8_moe_quant_act_i8(_p(x), T, H, H, _p(qx), _p(sx),
                                                                _p(rowsum), _stream(dev)))
    return qx, sx, rowsum


def w4a8_moe_swiglu_i8(h: torch.Tensor, qa=None, sa=None, rowsum=None):
    """fp32 [M, 2I] -> (int8 codes [M, I], scales fp32 [M], code row sums int32 [M])."""
    _need(h, "h", torch.float32, 2)
    M, I2 = h.shape
    I = I2 // 2
    dev = h.device
    qa = torch.empty((M, I), dtype=torch.int8, device=dev) if qa is None else qa
    sa = torch.empty((M,), dtype=torch.float32, device=dev) if sa is None else sa
    rowsum = torch.empty((M,), dtype=torch.int32, device=dev) if rowsum is None else rowsum
    _need(qa, "qa", torch.int8, 2, dev)
    _need(sa, "sa", torch.float32, 1, dev)
    _need(rowsum, "rowsum", torch.int32, 1, dev)
    if I2 % 2 or tuple(qa.shape) != (M, I) or tuple(sa.shape) != (M,) or tuple(rowsum.shape) != (M,):
        raise ValueError("h must be [M, 2I], qa [M, I], sa and rowsum [M]")
    _check("w4a8_moe_swiglu_i8", lib().w4a8_moe_swiglu_i8(_p(h), M, I, _p(qa), _p(sa), _p(rowsum), _stream(dev)))
    return qa, sa, rowsum


def w4a8_moe_quantize_weights_channel(w: torch.Tensor, w_packed=None, w_scale=None):
    """fp32 [..., K] -> (packed int32 [..., K/8], per-row scales fp32 [...])."""
    if not isinstance(w, torch.Tensor) or w.dim() < 1:
        raise TypeError("w must be a torch.Tensor with a K dimension")
    _need(w, "w", torch.float32, w.dim())
    K = w.shape[-1]
    lead = tuple(w.shape[:-1])
    rows = 1
    for d in lead:
        rows *= int(d)
    dev = w.device
    if K % 128:
        raise ValueError("K must be a multiple of 128")
    w_packed = torch.empty(lead + (K // 8,), dtype=torch.int32, device=dev) if w_packed is None else w_packed
    w_scale = torch.empty(lead, dtype=torch.float32, device=dev) if w_scale is None else w_scale
    _need(w_packed, "w_packed", torch.int32, len(lead) + 1, dev)
    _need(w_scale, "w_scale", torch.float32, len(lead), dev)
    if tuple(w_packed.shape) != lead + (K // 8,) or tuple(w_scale.shape) != lead:
        raise ValueError("w_packed must be [..., K/8] and w_scale [...]")
    _check("w4a8_moe_quantize_weights_channel",
           lib().w4a8_moe_quantize_weights_channel(_p(w), rows, K, _p(w_packed), _p(w_scale), _stream(dev)))
    return w_packed, w_scale


# ------------------------------------------------------------------ fused epilogues
def _act_out(M: int, I: int, dev, act, act_pmax):
    act = torch.empty((M, I), dtype=torch.float32, device=dev) if act is None else act
    act_pmax = torch.empty((M, I // 64), dtype=torch.float32, device=dev) if act_pmax is None else act_pmax
    _need(act, "act", torch.float32, 2, dev)
    _need(act_pmax, "act_pmax", torch.float32, 2, dev)
    if act.shape[0] < M or act.shape[1] != I or act_pmax.shape[0] < M or act_pmax.shape[1] != I // 64:
        raise ValueError("act must be at least [M_total, I] and act_pmax [M_total, I/64]")
    return act, act_pmax


def w4a8_moe_requant(act: torch.Tensor, act_pmax: torch.Tensor, qa=None, sa=None, M: int | None = None):
    """act fp32 [M, I] with its partial row maxima [M, I/64] -> (E4M3 codes uint8 [M, I], scales fp32 [M])."""
    _need(act, "act", torch.float32, 2)
    dev = act.device
    _need(act_pmax, "act_pmax", torch.float32, 2, dev)
    M = act.shape[0] if M is None else M
    I = act.shape[1]
    qa = torch.empty((M, I), dtype=torch.uint8, device=dev) if qa is None else qa
    sa = torch.empty((M,), dtype=torch.float32, device=dev) if sa is None else sa
    _need(qa, "qa", torch.uint8, 2, dev)
    _need(sa, "sa", torch.float32, 1, dev)
    if act.shape[0] < M or act_pmax.shape[0] < M or act_pmax.shape[1] != I // 64 or qa.shape[0] < M \
            or qa.shape[1] != I or sa.numel() < M:
        raise ValueError("act, act_pmax, qa and sa must hold M rows of I")
    _check("w4a8_moe_requant", lib().w4a8_moe_requant(_p(act), _p(act_pmax), M, I, _p(qa), _p(sa), _stream(dev)))
    return qa, sa


def w4a8_moe_requant_i8(act: torch.Tensor, act_pmax: torch.Tensor, qa=None, sa=None, rowsum=None,
                        M: int | None = None):
    """act fp32 [M, I] with its partial row maxima [M, I/64] -> (int8 codes, scales fp32 [M], code row sums [M])."""
    _need(act, "act", torch.float32, 2)
    dev = act.device
    _need(act_pmax, "act_pmax", torch.float32, 2, dev)
    M = act.shape[0] if M is None else M
    I = act.shape[1]
    qa = torch.empty((M, I), dtype=torch.int8, device=dev) if qa is None else qa
    sa = torch.empty((M,), dtype=torch.float32, device=dev) if sa is None else sa
    rowsum = torch.empty((M,), dtype=torch.int32, device=dev) if rowsum is None else rowsum
    _need(qa, "qa", torch.int8, 2, dev)
    _need(sa, "sa", torch.float32, 1, dev)
    _need(rowsum, "rowsum", torch.int32, 1, dev)
    if act.shape[0] < M or act_pmax.shape[0] < M or act_pmax.shape[1] != I // 64 or qa.shape[0] < M \
            or qa.shape[1] != I or sa.numel() < M or rowsum.numel() < M:
        raise ValueError("act, act_pmax, qa, sa and rowsum must hold M rows of I")
    _check("w4a8_moe_requant_i8", lib().w4a8_moe_requant_i8(_p(act), _p(act_pmax), M, I, _p(qa), _p(sa),
                                                            _p(rowsum), _stream(dev)))
    return qa, sa, rowsum


# ---- MXFP4 group-32 weights x per-token FP8 activations ---------------------
def w4a8_moe_quantize_weights_mxfp4(w: torch.Tensor, w_packed=None, w_scale=None):
    """fp32 [..., K] -> (E2M1 codes uint8 [..., K/2], E8M0 block scales uint8 [..., K/32]).

    Every leading dimension is flattened into rows (experts x output channels)."""
    if not isinstance(w, torch.Tensor) or w.dim() < 1:
        raise TypeError("w must be a torch.Tensor with a K dimension")
    _need(w, "w", torch.float32, w.dim())
    K = w.shape[-1]
    lead = tuple(w.shape[:-1])
    rows = 1
    for d in lead:
        rows *= int(d)
    dev = w.device
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    w_packed = torch.empty(lead + (K // 2,), dtype=torch.uint8, device=dev) if w_packed is None else w_packed
    w_scale = torch.empty(lead + (K // 32,), dtype=torch.uint8, device=dev) if w_scale is None else w_scale
    _need(w_packed, "w_packed", torch.uint8, len(lead) + 1, dev)
    _need(w_scale, "w_scale", torch.uint8, len(lead) + 1, dev)
    if tuple(w_packed.shape) != lead + (K // 2,) or tuple(w_scale.shape) != lead + (K // 32,):
        raise ValueError("w_packed must be [..., K/2] and w_scale [..., K/32]")
    _check("w4a8_moe_quantize_weights_mxfp4",
           lib().w4a8_moe_quantize_weights_mxfp4(_p(w), rows, K, _p(w_packed), _p(w_scale), _stream(dev)))
    return w_packed, w_scale


def w4a8_moe_prepack_int4(w_packed: torch.Tensor, w_scale: torch.Tensor | None = None, w_blk=None, s_blk=None):
    """Row-major INT4 experts (int32 [E, N, K/8], group scales fp32 [E, N, K/128] or None for per-channel
    scales) -> the GEMM storage (w_blk int32 [E, N/16, K/128, 16, 16], s_blk fp32 [E, K/128, N] or None)."""
    _need(w_packed, "w_packed", torch.int32, 3)
    dev = w_packed.device
    E, N, KW = w_packed.shape
    K = 8 * KW
    if N % 16 or K % 128:
        raise ValueError("w_packed must be [E, N, K/8] with N % 16 == 0 and K % 128 == 0")
    G = K // 128
    w_blk = torch.empty((E, N // 16, G, 16, 16), dtype=torch.int32, device=dev) if w_blk is None else w_blk
    _need(w_blk, "w_blk", torch.int32, 5, dev)
    if tuple(w_blk.shape) != (E, N // 16, G, 16, 16):
        raise ValueError("w_blk must be [E, N/16, K/128, 16, 16]")
    if w_scale is not None:
        _need(w_scale, "w_scale", torch.float32, 3, dev)
        if tuple(w_scale.shape) != (E, N, G):
            raise ValueError("w_scale must be [E, N, K/128]")
        s_blk = torch.empty((E, G, N), dtype=torch.float32, device=dev) if s_blk is None else s_blk
        _need(s_blk, "s_blk", torch.float32, 3, dev)
        if tuple(s_blk.shape) != (E, G, N):
            raise ValueError("s_blk must be [E, K/128, N]")
    else:
        s_blk = None
    _check("w4a8_moe_prepack_int4",
           lib().w4a8_moe_prepack_int4(_p(w_packed), _p(w_scale), E, N, K, _p(w_blk), _p(s_blk), _stream(dev)))
    return w_blk, s_blk


def w4a8_moe_prepack_mxfp4(w_packed: torch.Tensor, w_scale: torch.Tensor, w_blk=None, s_blk=None):
    """Row-major MXFP4 (codes uint8 [E, N, K/2], scales uint8 [E, N, K/32]) -> the GEMM storage
    (w_blk uint8 [E, N/16, K/128, 16, 64], s_blk uint8 [E, K/128, N, 4])."""
    _need(w_packed, "w_packed", torch.uint8, 3)
    dev = w_packed.device
    _need(w_scale, "w_scale", torch.uint8, 3, dev)
    E, N, KB = w_packed.shape
    K = 2 * KB
    if N % 16 or K % 128 or tuple(w_scale.shape) != (E, N, K // 32):
        raise ValueError("w_packed must be [E, N, K/2] with N % 16 == 0 and K % 128 == 0, w_scale [E, N, K/32]")
    G = K // 128
    w_blk = torch.empty((E, N // 16, G, 16, 64), dtype=torch.uint8, device=dev) if w_blk is None else w_blk
    s_blk = torch.empty((E, G, N, 4), dtype=torch.uint8, device=dev) if s_blk is None else s_blk
    _need(w_blk, "w_blk", torch.uint8, 5, dev)
    _need(s_blk, "s_blk", torch.uint8, 4, dev)
    if tuple(w_blk.shape) != (E, N // 16, G, 16, 64) or tuple(s_blk.shape) != (E, G, N, 4):
        raise ValueError("w_blk must be [E, N/16, K/128, 16, 64] and s_blk [E, K/128, N, 4]")
    _check("w4a8_moe_prepack_mxfp4",
           lib().w4a8_moe_prepack_mxfp4(_p(w_packed), _p(w_scale), E, N, K, _p(w_blk), _p(s_blk), _stream(dev)))
    return w_blk, s_blk




# ------------------------------------------------------------ grouped GEMMs
# Each GEMM exists twice: on the weights as stored (row-major: INT4 int32
# [E, N, K/8] uint4b8 words, MXFP4 uint8 [E, N, K/2] codes) and, with the
# suffix _prepacked, on the GEMM storage written by w4a8_moe_prepack_int4 /
# w4a8_moe_prepack_mxfp4 (INT4 int32 [E, N/16, K/128, 16, 16], MXFP4 uint8
# [E, N/16, K/128, 16, 64]), which the layer classes use.
def _int4_weights(w: torch.Tensor, name: str, dev, prepacked: bool) -> tuple[int, int, int]:
    """(E, N, K) of INT4 weights in either format."""
    if prepacked:
        return _int4_storage(w, name, dev)
    _need(w, name, torch.int32, 3, dev)
    E, N, KW = w.shape
    return E, N, 8 * KW


def _g128_scales(s: torch.Tensor, name: str, dev, E: int, N: int, K: int, prepacked: bool) -> None:
    _need(s, name, torch.float32, 3, dev)
    want = (E, K // 128, N) if prepacked else (E, N, K // 128)
    if tuple(s.shape) != want:
        raise ValueError(f"{name} must be {list(want)} ({'[E, K/128, N]' if prepacked else '[E, N, K/128]'})")


def _mx_weights(w: torch.Tensor, s: torch.Tensor, names, dev, prepacked: bool) -> tuple[int, int, int]:
    """(E, N, K) of MXFP4 weights: stored w [E, N, K/2] with s [E, N, K/32], or the GEMM
    storage w [E, N/16, K/128, 16, 64] with s [E, K/128, N, 4]."""
    if prepacked:
        _need(w, names[0], torch.uint8, 5, dev)
        _need(s, names[1], torch.uint8, 4, dev)
        E, NB, G, sixteen, sixtyfour = w.shape
        N, K = 16 * NB, 128 * G
        if (sixteen, sixtyfour) != (16, 64) or tuple(s.shape) != (E, G, N, 4):
            raise ValueError(f"{names[0]} [E,N/16,K/128,16,64] and {names[1]} [E,K/128,N,4] must match "
                             "(prepack_mxfp4 writes this storage)")
        return E, N, K
    _need(w, names[0], torch.uint8, 3, dev)
    _need(s, names[1], torch.uint8, 3, dev)
    E, N, KB = w.shape
    K = 2 * KB
    if tuple(s.shape) != (E, N, K // 32):
        raise ValueError(f"{names[0]} [E,N,K/2] and {names[1]} [E,N,K/32] must match")
    return E, N, K


def _gemm_inputs(a, a_scale, a_rows, offsets, M_total, a_dtype):
    _need(a, "a", a_dtype, 2)
    dev = a.device
    _need(a_scale, "a_scale", torch.float32, 1, dev)
    if a_rows is not None:
        _need(a_rows, "a_rows", torch.int32, 1, dev)
        if a_rows.numel() < M_total:
            raise ValueError("a_rows must hold M_total entries")
    elif a.shape[0] < M_total:
        raise ValueError("a must hold M_total rows when a_rows is None")
    _need(offsets, "offsets", torch.int32, 1, dev)
    if a_scale.numel() != a.shape[0]:
        raise ValueError("a_scale must have one entry per row of a")
    return dev


def _plain_out(out, M_total: int, N: int, dev):
    out = torch.empty((M_total, N), dtype=torch.float32, device=dev) if out is None else out
    _need(out, "out", torch.float32, 2, dev)
    if out.shape[0] < M_total or out.shape[1] != N:
        raise ValueError("out must be at least [M_total, N]")
    return out


def _row_dst(row_dst, M_total: int, out, dev):
    """The scatter forms: row_dst int32 [>= M_total], and an explicit out."""
    _need(row_dst, "row_dst", torch.int32, 1, dev)
    if row_dst.numel() < M_total:
        raise ValueError("row_dst must hold M_total entries")
    if out is None:
        raise ValueError("the scatter forms write into a given out (its rows are row_dst's targets)")


def _gemm_g128(prepacked, a, a_scale, a_rows, offsets, w_packed, w_scale, M_total, out, algo, row_dst=None):
    dev = _gemm_inputs(a, a_scale, a_rows, offsets, M_total, torch.uint8)
    E, N, K = _int4_weights(w_packed, "w_packed", dev, prepacked)
    _g128_scales(w_scale, "w_scale", dev, E, N, K, prepacked)
    if a.shape[1] != K or offsets.numel() != E + 1:
        raise ValueError("w_packed, w_scale and offsets [E+1] must match a [*, K]")
    if row_dst is not None:
        _row_dst(row_dst, M_total, out, dev)
    out = _plain_out(out, M_total, N, dev)
    if row_dst is not None:
        _check("w4a8_moe_grouped_gemm_scatter_prepacked", lib().w4a8_moe_grouped_gemm_scatter_prepacked(
            _p(a), _p(a_scale), _p(a_rows), M_total, _p(offsets), E, _p(w_packed), _p(w_scale), N, K, _p(row_dst),
            _p(out), algo, _stream(dev)))
        return out
    args = (_p(a), _p(a_scale), _p(a_rows), M_total, _p(offsets), E, _p(w_packed), _p(w_scale), N, K, _p(out))
    if prepacked:
        _check("w4a8_moe_grouped_gemm_prepacked", lib().w4a8_moe_grouped_gemm_prepacked(*args, algo, _stream(dev)))
    else:
        _check("w4a8_moe_grouped_gemm", lib().w4a8_moe_grouped_gemm(*args, _stream(dev)))
    return out


def w4a8_moe_grouped_gemm(a: torch.Tensor, a_scale: torch.Tensor, a_rows: torch.Tensor | None,
                          offsets: torch.Tensor, w_packed: torch.Tensor, w_scale: torch.Tensor, M_total: int,
                          out: torch.Tensor | None = None):
    """Grouped W4A8 GEMM on stored weights (int32 [E, N, K/8], fp32 [E, N, K/128]) -> fp32 [M_total, N]
    (rows of expert e: offsets[e]..offsets[e+1])."""
    return _gemm_g128(False, a, a_scale, a_rows, offsets, w_packed, w_scale, M_total, out, W4A8_GG_AUTO)


def w4a8_moe_grouped_gemm_prepacked(a: torch.Tensor, a_scale: torch.Tensor, a_rows: torch.Tensor | None,
                                    offsets: torch.Tensor, w_packed: torch.Tensor, w_scale: torch.Tensor,
                                    M_total: int, out: torch.Tensor | None = None, algo: int = W4A8_GG_AUTO):
    """The same on the GEMM storage (w4a8_moe_prepack_int4: int32 [E, N/16, K/128, 16, 16], fp32 [E, K/128, N])."""
    return _gemm_g128(True, a, a_scale, a_rows, offsets, w_packed, w_scale, M_total, out, algo)


def _gemm_i8(prepacked, a, a_scale, a_rowsum, a_rows, offsets, w_packed, w_scale, out, M_total, algo, row_dst=None):
    if M_total is None:
        M_total = a_rows.numel() if a_rows is not None else a.shape[0]
    dev = _gemm_inputs(a, a_scale, a_rows, offsets, M_total, torch.int8)
    _need(a_rowsum, "a_rowsum", torch.int32, 1, dev)
    E, N, K = _int4_weights(w_packed, "w_packed", dev, prepacked)
    _need(w_scale, "w_scale", torch.float32, 2, dev)
    if a.shape[1] != K or tuple(w_scale.shape) != (E, N) or offsets.numel() != E + 1:
        raise ValueError("a must be [*, K], w_scale [E, N], offsets [E+1]")
    if row_dst is not None:
        _row_dst(row_dst, M_total, out, dev)
    out = _plain_out(out, M_total, N, dev)
    if row_dst is not None:
        _check("w4a8_moe_grouped_gemm_scatter_i8_prepacked", lib().w4a8_moe_grouped_gemm_scatter_i8_prepacked(
            _p(a), _p(a_scale), _p(a_rowsum), _p(a_rows), M_total, _p(offsets), E, _p(w_packed), _p(w_scale), N, K,
            _p(row_dst), _p(out), algo, _stream(dev)))
        return out
    args = (_p(a), _p(a_scale), _p(a_rowsum), _p(a_rows), M_total, _p(offsets), E, _p(w_packed), _p(w_scale), N,
            K, _p(out))
    if prepacked:
        _check("w4a8_moe_grouped_gemm_i8_prepacked",
               lib().w4a8_moe_grouped_gemm_i8_prepacked(*args, algo, _stream(dev)))
    else:
        _check("w4a8_moe_grouped_gemm_i8", lib().w4a8_moe_grouped_gemm_i8(*args, _stream(dev)))
    return out


def w4a8_moe_grouped_gemm_i8(a: torch.Tensor, a_scale: torch.Tensor, a_rowsum: torch.Tensor,
                             a_rows: torch.Tensor | None, offsets: torch.Tensor, w_packed: torch.Tensor,
                             w_scale: torch.Tensor, out: torch.Tensor | None = None, M_total: int | None = None):
    """int8 [*, K] activations x per-channel INT4 experts as stored (int32 [E, N, K/8], scales [E, N])
    -> fp32 [M_total, N]."""
    return _gemm_i8(False, a, a_scale, a_rowsum, a_rows, offsets, w_packed, w_scale, out, M_total, W4A8_GG_AUTO)


def w4a8_moe_grouped_gemm_i8_prepacked(a: torch.Tensor, a_scale: torch.Tensor, a_rowsum: torch.Tensor,
                                       a_rows: torch.Tensor | None, offsets: torch.Tensor, w_packed: torch.Tensor,
                                       w_scale: torch.Tensor, out: torch.Tensor | None = None,
                                       M_total: int | None = None, algo: int = W4A8_GG_AUTO):
    """The same on the GEMM storage of the weights (int32 [E, N/16, K/128, 16, 16])."""
    return _gemm_i8(True, a, a_scale, a_rowsum, a_rows, offsets, w_packed, w_scale, out, M_total, algo)


def _act_out(M: int, I: int, dev, act, act_pmax):
    act = torch.empty((M, I), dtype=torch.float32, device=dev) if act is None else act
    act_pmax = torch.empty((M, I // 64), dtype=torch.float32, device=dev) if act_pmax is None else act_pmax
    _need(act, "act", torch.float32, 2, dev)
    _need(act_pmax, "act_pmax", torch.float32, 2, dev)
    if act.shape[0] < M or act.shape[1] != I or act_pmax.shape[0] < M or act_pmax.shape[1] != I // 64:
        raise ValueError("act must be at least [M_total, I] and act_pmax [M_total, I/64]")
    return act, act_pmax


def _gemm_swiglu(form, prepacked, a, a_scale, a_rowsum, a_rows, offsets, w13, s13, M_total, act, act_pmax, algo):
    dev = _gemm_inputs(a, a_scale, a_rows, offsets, M_total, torch.int8 if form == "i8" else torch.uint8)
    if form == "mxfp4":
        E, N2, K = _mx_weights(w13, s13, ("w13", "s13"), dev, prepacked)
    else:
        E, N2, K = _int4_weights(w13, "w13", dev, prepacked)
        if form == "i8":
            _need(a_rowsum, "a_rowsum", torch.int32, 1, dev)
            _need(s13, "s13", torch.float32, 2, dev)
            if tuple(s13.shape) != (E, N2):
                raise ValueError("s13 must be [E, 2I]")
        else:
            _g128_scales(s13, "s13", dev, E, N2, K, prepacked)
    if N2 % 2 or a.shape[1] != K or offsets.numel() != E + 1:
        raise ValueError("w13 must hold 2I rows of K, offsets [E+1], and a [*, K]")
    I = N2 // 2
    act, act_pmax = _act_out(M_total, I, dev, act, act_pmax)
    head = (_p(a), _p(a_scale)) + ((_p(a_rowsum),) if form == "i8" else ())
    args = head + (_p(a_rows), M_total, _p(offsets), E, _p(w13), _p(s13), I, K, _p(act), _p(act_pmax))
    name = "w4a8_moe_grouped_gemm_swiglu" + ("" if form == "g128" else "_" + form) + ("_prepacked" if prepacked else "")
    fn = getattr(lib(), name)
    _check(name, fn(*args, algo, _stream(dev)) if prepacked else fn(*args, _stream(dev)))
    return act, act_pmax


def w4a8_moe_grouped_gemm_swiglu(a: torch.Tensor, a_scale: torch.Tensor, a_rows: torch.Tensor | None,
                                 offsets: torch.Tensor, w13: torch.Tensor, s13: torch.Tensor, M_total: int,
                                 act: torch.Tensor | None = None, act_pmax: torch.Tensor | None = None):
    """Gate/up GEMM with SwiGLU in its epilogue on stored weights (int32 [E, 2I, K/8], fp32 [E, 2I, K/128])
    -> (act fp32 [M_total, I], partial row maxima of |act| [M_total, I/64])."""
    return _gemm_swiglu("g128", False, a, a_scale, None, a_rows, offsets, w13, s13, M_total, act, act_pmax,
                        W4A8_GG_AUTO)


def w4a8_moe_grouped_gemm_swiglu_prepacked(a: torch.Tensor, a_scale: torch.Tensor, a_rows: torch.Tensor | None,
                                           offsets: torch.Tensor, w13: torch.Tensor, s13: torch.Tensor,
                                           M_total: int, act: torch.Tensor | None = None,
                                           act_pmax: torch.Tensor | None = None, algo: int = W4A8_GG_AUTO):
    """The same on the GEMM storage (int32 [E, 2I/16, K/128, 16, 16], fp32 [E, K/128, 2I])."""
    return _gemm_swiglu("g128", True, a, a_scale, None, a_rows, offsets, w13, s13, M_total, act, act_pmax, algo)


def w4a8_moe_grouped_gemm_swiglu_i8(a: torch.Tensor, a_scale: torch.Tensor, a_rowsum: torch.Tensor,
                                    a_rows: torch.Tensor | None, offsets: torch.Tensor, w13: torch.Tensor,
                                    s13: torch.Tensor, M_total: int, act: torch.Tensor | None = None,
                                    act_pmax: torch.Tensor | None = None):
    """INT8 form of w4a8_moe_grouped_gemm_swiglu (stored w13 int32 [E, 2I, K/8], per-channel s13 [E, 2I])."""
    return _gemm_swiglu("i8", False, a, a_scale, a_rowsum, a_rows, offsets, w13, s13, M_total, act, act_pmax,
                        W4A8_GG_AUTO)


def w4a8_moe_grouped_gemm_swiglu_i8_prepacked(a: torch.Tensor, a_scale: torch.Tensor, a_rowsum: torch.Tensor,
                                              a_rows: torch.Tensor | None, offsets: torch.Tensor, w13: torch.Tensor,
                                              s13: torch.Tensor, M_total: int, act: torch.Tensor | None = None,
                                              act_pmax: torch.Tensor | None = None, algo: int = W4A8_GG_AUTO):
    """The same on the GEMM storage of w13."""
    return _gemm_swiglu("i8", True, a, a_scale, a_rowsum, a_rows, offsets, w13, s13, M_total, act, act_pmax, algo)


def _gemm_mx(prepacked, a, a_scale, a_rows, offsets, w_packed, w_scale, M_total, out, algo, row_dst=None):
    dev = _gemm_inputs(a, a_scale, a_rows, offsets, M_total, torch.uint8)
    E, N, K = _mx_weights(w_packed, w_scale, ("w_packed", "w_scale"), dev, prepacked)
    if a.shape[1] != K or offsets.numel() != E + 1:
        raise ValueError("w_packed, w_scale and offsets [E+1] must match a [*, K]")
    if row_dst is not None:
        _row_dst(row_dst, M_total, out, dev)
    out = _plain_out(out, M_total, N, dev)
    if row_dst is not None:
        _check("w4a8_moe_grouped_gemm_scatter_mxfp4_prepacked", lib().w4a8_moe_grouped_gemm_scatter_mxfp4_prepacked(
            _p(a), _p(a_scale), _p(a_rows), M_total, _p(offsets), E, _p(w_packed), _p(w_scale), N, K, _p(row_dst),
            _p(out), algo, _stream(dev)))
        return out
    args = (_p(a), _p(a_scale), _p(a_rows), M_total, _p(offsets), E, _p(w_packed), _p(w_scale), N, K, _p(out))
    if prepacked:
        _check("w4a8_moe_grouped_gemm_mxfp4_prepacked",
               lib().w4a8_moe_grouped_gemm_mxfp4_prepacked(*args, algo, _stream(dev)))
    else:
        _check("w4a8_moe_grouped_gemm_mxfp4", lib().w4a8_moe_grouped_gemm_mxfp4(*args, _stream(dev)))
    return out


def w4a8_moe_grouped_gemm_mxfp4(a: torch.Tensor, a_scale: torch.Tensor, a_rows: torch.Tensor | None,
                                offsets: torch.Tensor, w_packed: torch.Tensor, w_scale: torch.Tensor, M_total: int,
                                out: torch.Tensor | None = None):
    """Grouped FP8 x MXFP4 GEMM on stored weights (uint8 [E, N, K/2] codes, [E, N, K/32] E8M0 scales)
    -> out fp32 [M_total, N]."""
    return _gemm_mx(False, a, a_scale, a_rows, offsets, w_packed, w_scale, M_total, out, W4A8_GG_AUTO)


def w4a8_moe_grouped_gemm_mxfp4_prepacked(a: torch.Tensor, a_scale: torch.Tensor, a_rows: torch.Tensor | None,
                                          offsets: torch.Tensor, w_packed: torch.Tensor, w_scale: torch.Tensor,
                                          M_total: int, out: torch.Tensor | None = None,
                                          algo: int = W4A8_GG_AUTO):
    """The same on the GEMM storage (w4a8_moe_prepack_mxfp4)."""
    return _gemm_mx(True, a, a_scale, a_rows, offsets, w_packed, w_scale, M_total, out, algo)


# -------------------------------------------------- step 7 with the scatter in the down GEMM
def w4a8_moe_row_sources(inv_pos: torch.Tensor, w: torch.Tensor, a_scale: torch.Tensor, M_total: int,
                         row_src: torch.Tensor | None = None, row_scale: torch.Tensor | None = None):
    """inv_pos int32 [T*k], w fp32 [T, k], a_scale fp32 [>= M_total] -> (row_src int32 [M_total]: the routed
    index f of each row p, row_scale fp32 [M_total]: a_scale[p] * w[f])."""
    _need(inv_pos, "inv_pos", torch.int32, 1)
    dev = inv_pos.device
    _need(w, "w", torch.float32, 2, dev)
    _need(a_scale, "a_scale", torch.float32, 1, dev)
    T, k = w.shape
    if inv_pos.numel() != T * k or a_scale.numel() < M_total:
        raise ValueError("inv_pos must be [T*k] and a_scale hold M_total entries")
    row_src = torch.empty((M_total,), dtype=torch.int32, device=dev) if row_src is None else row_src
    row_scale = torch.empty((M_total,), dtype=torch.float32, device=dev) if row_scale is None else row_scale
    _need(row_src, "row_src", torch.int32, 1, dev)
    _need(row_scale, "row_scale", torch.float32, 1, dev)
    if row_src.numel() < M_total or row_scale.numel() < M_total:
        raise ValueError("row_src and row_scale must hold M_total entries")
    _check("w4a8_moe_row_sources", lib().w4a8_moe_row_sources(_p(inv_pos), _p(w), _p(a_scale), T, k, M_total,
                                                              _p(row_src), _p(row_scale), _stream(dev)))
    return row_src, row_scale


def w4a8_moe_grouped_gemm_scatter_prepacked(a: torch.Tensor, a_scale: torch.Tensor, a_rows: torch.Tensor | None,
                                            offsets: torch.Tensor, w_packed: torch.Tensor, w_scale: torch.Tensor,
                                            M_total: int, row_dst: torch.Tensor, out: torch.Tensor,
                                            algo: int = W4A8_GG_AUTO):
    """w4a8_moe_grouped_gemm_prepacked with row p of the result stored as row row_dst[p] of out."""
    return _gemm_g128(True, a, a_scale, a_rows, offsets, w_packed, w_scale, M_total, out, algo, row_dst)


def w4a8_moe_grouped_gemm_scatter_i8_prepacked(a: torch.Tensor, a_scale: torch.Tensor, a_rowsum: torch.Tensor,
                                               a_rows: torch.Tensor | None, offsets: torch.Tensor,
                                               w_packed: torch.Tensor, w_scale: torch.Tensor, M_total: int,
                                               row_dst: torch.Tensor, out: torch.Tensor, algo: int = W4A8_GG_AUTO):
    """w4a8_moe_grouped_gemm_i8_prepacked with row p of the result stored as row row_dst[p] of out."""
    return _gemm_i8(True, a, a_scale, a_rowsum, a_rows, offsets, w_packed, w_scale, out, M_total, algo, row_dst)


def w4a8_moe_grouped_gemm_scatter_mxfp4_prepacked(a: torch.Tensor, a_scale: torch.Tensor,
                                                  a_rows: torch.Tensor | None, offsets: torch.Tensor,
                                                  w_packed: torch.Tensor, w_scale: torch.Tensor, M_total: int,
                                                  row_dst: torch.Tensor, out: torch.Tensor,
                                                  algo: int = W4A8_GG_AUTO):
    """w4a8_moe_grouped_gemm_mxfp4_prepacked with row p of the result stored as row row_dst[p] of out."""
    return _gemm_mx(True, a, a_scale, a_rows, offsets, w_packed, w_scale, M_total, out, algo, row_dst)


def w4a8_moe_combine(o_tok: torch.Tensor, inv_pos: torch.Tensor, T: int, k: int, y: torch.Tensor | None = None,
                     y_dtype: torch.dtype = torch.float32):
    """o_tok fp32 [T*k, H] (token-major), inv_pos int32 [T*k] -> y [T, H]: each token's routed rows summed."""
    _need(o_tok, "o_tok", torch.float32, 2)
    dev = o_tok.device
    _need(inv_pos, "inv_pos", torch.int32, 1, dev)
    H = o_tok.shape[1]
    if inv_pos.numel() != T * k or o_tok.shape[0] < T * k:
        raise ValueError("inv_pos must be [T*k] and o_tok at least [T*k, H]")
    if y is None:
        y = torch.empty((T, H), dtype=y_dtype, device=dev)
    if y.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("y must be float32 or bfloat16")
    _need(y, "y", y.dtype, 2, dev)
    if tuple(y.shape) != (T, H):
        raise ValueError("y must be [T, H]")
    code = W4A8_Y_F32 if y.dtype == torch.float32 else W4A8_Y_BF16
    _check("w4a8_moe_combine", lib().w4a8_moe_combine(_p(o_tok), _p(inv_pos), T, k, H, _p(y), code, _stream(dev)))
    return y


def w4a8_moe_grouped_gemm_swiglu_mxfp4(a: torch.Tensor, a_scale: torch.Tensor, a_rows: torch.Tensor | None,
                                       offsets: torch.Tensor, w13: torch.Tensor, s13: torch.Tensor, M_total: int,
                                       act: torch.Tensor | None = None, act_pmax: torch.Tensor | None = None):
    """MXFP4 gate/up GEMM with SwiGLU in its epilogue on stored weights -> (act [M_total, I], row maxima)."""
    return _gemm_swiglu("mxfp4", False, a, a_scale, None, a_rows, offsets, w13, s13, M_total, act, act_pmax,
                        W4A8_GG_AUTO)


def w4a8_moe_grouped_gemm_swiglu_mxfp4_prepacked(a: torch.Tensor, a_scale: torch.Tensor,
                                                 a_rows: torch.Tensor | None, offsets: torch.Tensor,
                                                 w13: torch.Tensor, s13: torch.Tensor, M_total: int,
                                                 act: torch.Tensor | None = None,
                                                 act_pmax: torch.Tensor | None = None, algo: int = W4A8_GG_AUTO):
    """The same on the GEMM storage of w13 and s13."""
    return _gemm_swiglu("mxfp4", True, a, a_scale, None, a_rows, offsets, w13, s13, M_total, act, act_pmax, algo)
