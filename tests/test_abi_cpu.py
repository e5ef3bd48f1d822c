"""The C ABI library without a GPU: it loads, exports every declared symbol,
and rejects bad arguments on the host before touching a device.

Pointers passed here are never dereferenced: every call either fails a host
check or (on a machine without a gfx950) the device check.  The calls that
would pass every check are made only when no supported device is present.
"""
import ctypes
import os
import re
import subprocess

import pytest
import torch

from quantized_grouped_gemm_token_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a8_moe.h")

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_DEVICE, ERR_HIP, ERR_WORKSPACE = range(7)
P = 0x10000          # a fake, 64 KiB-aligned address (never dereferenced)


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(w4a8_moe_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return ops.lib()


@pytest.fixture(scope="module")
def no_device(L):
    return L.w4a8_moe_device_supported() == 0


def test_exports_every_declared_symbol(L):
    syms = declared_symbols()
    assert len(syms) >= 10
    for s in syms:
        assert hasattr(L, s), s
    out = subprocess.run(["nm", "-D", "--defined-only", ops.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (w4a8_moe_\w+)", out))
    assert set(syms) <= exported


def test_status_strings(L):
    names = [ops.status_string(i) for i in range(7)]
    assert names == ["W4A8_OK", "W4A8_ERR_NULL", "W4A8_ERR_SHAPE", "W4A8_ERR_ALIGN", "W4A8_ERR_DEVICE",
                     "W4A8_ERR_HIP", "W4A8_ERR_WORKSPACE"]
    assert ops.status_string(99) == "W4A8_ERR_UNKNOWN"


def test_quant_act_checks(L):
    f = L.w4a8_moe_quant_act
    assert f(P, 4, 100, 100, P, P, None) == ERR_SHAPE            # H % 128
    assert f(P, 4, 256, 200, P, P, None) == ERR_SHAPE            # ld < H
    assert f(P, 4, 256, 260, P, P, None) == ERR_SHAPE            # ld % 8
    assert f(P, -1, 256, 256, P, P, None) == ERR_SHAPE
    assert f(None, 4, 256, 256, P, P, None) == ERR_NULL
    assert f(P + 8, 4, 256, 256, P, P, None) == ERR_ALIGN        # x not 16-byte aligned
    assert f(P, 4, 256, 256, P + 4, P, None) == ERR_ALIGN        # qx not 8-byte aligned
    assert f(None, 0, 256, 256, None, None, None) == OK          # T = 0 is a no-op


def test_route_checks(L):
    f = L.w4a8_moe_route
    assert f(P, 4, 8, 9, 1, P, P, None) == ERR_SHAPE             # k > E
    assert f(P, 4, 2048, 8, 1, P, P, None) == ERR_SHAPE          # E > 1024
    assert f(P, 4, 8, 0, 1, P, P, None) == ERR_SHAPE
    assert f(P, 4, 8, 2, 1, None, P, None) == ERR_NULL
    assert f(P + 2, 4, 8, 2, 1, P, P, None) == ERR_ALIGN
    assert f(None, 0, 8, 2, 1, None, None, None) == OK


def test_permute_checks(L):
    ws = L.w4a8_moe_permute_workspace_bytes
    assert ws(128, 8, 256) == 256 * 4
    assert ws(16384, 8, 256) == 128 * 256 * 4
    assert ws(0, 8, 256) == 256 * 4
    assert ws(4, 9, 8) == -1
    f = L.w4a8_moe_permute
    need = ws(128, 8, 256)
    assert f(P, 128, 8, 256, P, P, P, P, need - 4, None) == ERR_WORKSPACE
    assert f(P, 128, 8, 256, None, P, P, P, need, None) == ERR_NULL
    assert f(P, 128, 8, 256, P, P, P, None, need, None) == ERR_NULL
    assert f(P, 128, 9, 8, P, P, P, P, need, None) == ERR_SHAPE
    assert f(P, 128, 8, 256, P + 1, P, P, P, need, None) == ERR_ALIGN


def test_permute_noalloc_checks(L, no_device):
    f = L.w4a8_moe_permute_noalloc
    assert f(P, 128, 9, 8, P, P, P, None) == ERR_SHAPE               # k > E
    assert f(P, -1, 8, 256, P, P, P, None) == ERR_SHAPE
    assert f(P, 128, 8, 256, None, P, P, None) == ERR_NULL
    assert f(P, 128, 8, 256, P, None, P, None) == ERR_NULL
    assert f(P, 128, 8, 256, P + 2, P, P, None) == ERR_ALIGN
    # more than the library's 1 MiB of scratch: refused, whatever the pointers
    assert L.w4a8_moe_permute_workspace_bytes(1 << 18, 8, 256) > (1 << 20)
    assert f(P, 1 << 18, 8, 256, P, P, P, None) == ERR_WORKSPACE
    assert "1048576" in ops.last_error()
    if no_device:
        assert f(P, 1 << 17, 8, 256, P, P, P, None) == ERR_DEVICE    # the largest size that fits


def test_grouped_gemm_checks(L):
    f = L.w4a8_moe_grouped_gemm                    # weights as stored: N % 16
    fp = L.w4a8_moe_grouped_gemm_prepacked         # GEMM storage: N % 64, and an algo
    good = dict(a=P, sa=P, rows=None, M=64, off=P, E=8, w=P, ws=P, N=256, K=256, out=P)

    def call(fn=f, algo=None, **kw):
        d = dict(good, **kw)
        args = (d["a"], d["sa"], d["rows"], d["M"], d["off"], d["E"], d["w"], d["ws"], d["N"], d["K"], d["out"])
        return fn(*args, None) if algo is None else fn(*args, algo, None)
    for fn, algo in ((f, None), (fp, 0)):
        assert call(fn, algo, N=24) == ERR_SHAPE          # N % 16
        assert call(fn, algo, N=0) == ERR_SHAPE
        assert call(fn, algo, K=192) == ERR_SHAPE         # K % 128
        assert call(fn, algo, E=0) == ERR_SHAPE
        assert call(fn, algo, E=2000) == ERR_SHAPE
        assert call(fn, algo, M=-1) == ERR_SHAPE
        assert call(fn, algo, w=None) == ERR_NULL
        assert call(fn, algo, off=None) == ERR_NULL
        assert call(fn, algo, a=P + 8) == ERR_ALIGN
        assert call(fn, algo, w=P + 4) == ERR_ALIGN
        assert call(fn, algo, out=P + 4) == ERR_ALIGN
        assert call(fn, algo, M=0, a=None, w=None) == OK  # no rows: no-op
    assert call(fp, 0, N=96) == ERR_SHAPE                 # the GEMM storage needs N % 64
    assert call(fp, 7) == ERR_SHAPE                       # unknown algo
    assert call(f, None, N=48, M=0, a=None, w=None) == OK  # stored weights: N % 16 is enough


def test_swiglu_unpermute_checks(L):
    assert L.w4a8_moe_swiglu(P, 4, 100, P, P, None) == ERR_SHAPE
    assert L.w4a8_moe_swiglu(P + 4, 4, 128, P, P, None) == ERR_ALIGN
    assert L.w4a8_moe_swiglu(None, 4, 128, P, P, None) == ERR_NULL
    assert L.w4a8_moe_swiglu(None, 0, 128, None, None, None) == OK
    u = L.w4a8_moe_unpermute
    assert u(P, P, P, 4, 2, 100, P, 0, None) == ERR_SHAPE
    assert u(P, P, P, 4, 2, 256, P, 5, None) == ERR_SHAPE        # bad y dtype
    assert u(P, P, P, 4, 0, 256, P, 0, None) == ERR_SHAPE
    assert u(P, P, P, 4, 2, 256, P + 8, 0, None) == ERR_ALIGN    # f32 y needs 16 bytes
    assert u(P, P, None, 4, 2, 256, P, 0, None) == ERR_NULL
    assert u(None, None, None, 0, 2, 256, None, 0, None) == OK


def test_quantize_weights_checks(L):
    q = L.w4a8_moe_quantize_weights
    assert q(P, 4, 100, 1, P, P, None) == ERR_SHAPE             # K % 128
    assert q(P, -1, 128, 1, P, P, None) == ERR_SHAPE
    assert q(None, 4, 128, 1, P, P, None) == ERR_NULL
    assert q(P + 4, 4, 128, 1, P, P, None) == ERR_ALIGN         # w not 8-byte aligned
    assert q(P, 4, 128, 1, P + 2, P, None) == ERR_ALIGN
    assert q(None, 0, 128, 1, None, None, None) == OK


def test_valid_calls_report_missing_device(L, no_device):
    if not no_device:
        pytest.skip("a supported GPU is present; these fake pointers must not reach it")
    assert L.w4a8_moe_quant_act(P, 4, 256, 256, P, P, None) == ERR_DEVICE
    assert "gfx950" in ops.last_error() or "device" in ops.last_error()
    assert L.w4a8_moe_route(P, 4, 8, 2, 1, P, P, None) == ERR_DEVICE
    assert L.w4a8_moe_permute(P, 4, 2, 8, P, P, P, P, 4096, None) == ERR_DEVICE
    assert L.w4a8_moe_grouped_gemm(P, P, None, 8, P, 8, P, P, 256, 256, P, None) == ERR_DEVICE
    assert L.w4a8_moe_swiglu(P, 4, 128, P, P, None) == ERR_DEVICE
    assert L.w4a8_moe_unpermute(P, P, P, 4, 2, 256, P, 0, None) == ERR_DEVICE
    assert L.w4a8_moe_quantize_weights(P, 4, 256, 1, P, P, None) == ERR_DEVICE
    assert L.w4a8_moe_device_supported() == 0


def test_last_error_is_per_call(L):
    assert L.w4a8_moe_swiglu(P, 4, 100, P, P, None) == ERR_SHAPE
    assert "I=100" in ops.last_error()
    assert L.w4a8_moe_swiglu(None, 0, 128, None, None, None) == OK
    assert ops.last_error() == ""


def test_binding_rejects_host_tensors():
    x = torch.zeros((4, 256), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ops.w4a8_moe_quant_act(x)
    with pytest.raises(TypeError):
        ops.w4a8_moe_quant_act(torch.zeros((4, 256), dtype=torch.float32))
    with pytest.raises(ValueError):
        ops.w4a8_moe_route(torch.zeros((4, 8), dtype=torch.float32), 2)


def test_binding_declares_every_symbol():
    # every entry point of the header has a ctypes signature in the binding, and no other
    assert set(declared_symbols()) == set(ops._SIGNATURES)


def test_int8_variant_checks(L):
    q = L.w4a8_moe_quant_act_i8
    assert q(P, 4, 100, 100, P, P, P, None) == ERR_SHAPE            # H % 128
    assert q(P, 4, 256, 256, P, P, None, None) == ERR_NULL          # row sums are required
    assert q(P + 8, 4, 256, 256, P, P, P, None) == ERR_ALIGN
    assert q(None, 0, 256, 256, None, None, None, None) == OK
    good = dict(a=P, sa=P, rs=P, rows=None, M=64, off=P, E=8, w=P, ws=P, N=256, K=256, out=P)

    def call(fn, algo=None, **kw):
        d = dict(good, **kw)
        args = (d["a"], d["sa"], d["rs"], d["rows"], d["M"], d["off"], d["E"], d["w"], d["ws"], d["N"], d["K"],
                d["out"])
        return fn(*args, None) if algo is None else fn(*args, algo, None)
    for fn, algo in ((L.w4a8_moe_grouped_gemm_i8, None), (L.w4a8_moe_grouped_gemm_i8_prepacked, 0)):
        assert call(fn, algo, K=(1 << 20) + 128) == ERR_SHAPE    # int32 sums could overflow
        assert call(fn, algo, N=24) == ERR_SHAPE
        assert call(fn, algo, rs=None) == ERR_NULL
        assert call(fn, algo, rows=P + 2) == ERR_ALIGN
        assert call(fn, algo, M=0, a=None, rs=None) == OK
    assert call(L.w4a8_moe_grouped_gemm_i8_prepacked, 0, N=96) == ERR_SHAPE
    assert call(L.w4a8_moe_grouped_gemm_i8_prepacked, 3) == ERR_SHAPE
    s = L.w4a8_moe_swiglu_i8
    assert s(P, 4, 100, P, P, P, None) == ERR_SHAPE
    assert s(P, 4, 128, P, P, None, None) == ERR_NULL
    assert s(P, 4, 128, P + 2, P, P, None) == ERR_ALIGN             # qa 4-byte
    assert s(None, 0, 128, None, None, None, None) == OK
    c = L.w4a8_moe_quantize_weights_channel
    assert c(P, 4, 100, P, P, None) == ERR_SHAPE
    assert c(P, 4, 128, None, P, None) == ERR_NULL
    assert c(P + 4, 4, 128, P, P, None) == ERR_ALIGN
    assert c(None, 0, 128, None, None, None) == OK


def test_fused_epilogue_checks(L):
    good = dict(a=P, sa=P, rows=None, M=64, off=P, E=8, w=P, s=P, I=128, K=256, act=P, pm=P)

    def call(fn, algo=None, **kw):
        d = dict(good, **kw)
        args = (d["a"], d["sa"], d["rows"], d["M"], d["off"], d["E"], d["w"], d["s"], d["I"], d["K"], d["act"],
                d["pm"])
        return fn(*args, None) if algo is None else fn(*args, algo, None)
    for fn, algo in ((L.w4a8_moe_grouped_gemm_swiglu, None), (L.w4a8_moe_grouped_gemm_swiglu_mxfp4, None),
                     (L.w4a8_moe_grouped_gemm_swiglu_prepacked, 0),
                     (L.w4a8_moe_grouped_gemm_swiglu_mxfp4_prepacked, 0)):
        assert call(fn, algo, I=64) == ERR_SHAPE                       # I % 128
        assert call(fn, algo, K=100) == ERR_SHAPE
        assert call(fn, algo, E=0) == ERR_SHAPE
        assert call(fn, algo, pm=None) == ERR_NULL
        assert call(fn, algo, act=P + 4) == ERR_ALIGN                  # act 16-byte
        assert call(fn, algo, pm=P + 2) == ERR_ALIGN
        assert call(fn, algo, M=0, a=None, w=None, act=None, pm=None) == OK
        if algo is not None:
            assert call(fn, 5) == ERR_SHAPE
    g = L.w4a8_moe_grouped_gemm_swiglu_i8
    assert g(P, P, None, None, 64, P, 8, P, P, 128, 256, P, P, None) == ERR_NULL      # row sums
    assert g(P, P, P, None, 64, P, 8, P, P, 128, (1 << 20) + 128, P, P, None) == ERR_SHAPE
    gp = L.w4a8_moe_grouped_gemm_swiglu_i8_prepacked
    assert gp(P, P, None, None, 64, P, 8, P, P, 128, 256, P, P, 0, None) == ERR_NULL
    assert gp(P, P, P, None, 64, P, 8, P, P, 128, 256, P, P, 4, None) == ERR_SHAPE
    r = L.w4a8_moe_requant
    assert r(P, P, 4, 100, P, P, None) == ERR_SHAPE
    assert r(P, None, 4, 128, P, P, None) == ERR_NULL
    assert r(P + 4, P, 4, 128, P, P, None) == ERR_ALIGN
    assert r(None, None, 0, 128, None, None, None) == OK
    r8 = L.w4a8_moe_requant_i8
    assert r8(P, P, 4, 128, P, P, None, None) == ERR_NULL
    assert r8(P, P, 4, 128, P, P, P + 2, None) == ERR_ALIGN
    assert r8(None, None, 0, 128, None, None, None, None) == OK


def test_prepack_and_mxfp4_checks(L):
    pi = L.w4a8_moe_prepack_int4
    assert pi(P, P, 2, 24, 256, P, P, None) == ERR_SHAPE            # N % 16
    assert pi(P, P, 2, 32, 200, P, P, None) == ERR_SHAPE            # K % 128
    assert pi(P, P, -1, 32, 256, P, P, None) == ERR_SHAPE
    assert pi(P, P, 2, 32, 256, P, None, None) == ERR_NULL          # scales: both or neither
    assert pi(P, None, 2, 32, 256, P, P, None) == ERR_NULL
    assert pi(P + 8, None, 2, 32, 256, P, None, None) == ERR_ALIGN
    assert pi(None, None, 0, 32, 256, None, None, None) == OK
    pm = L.w4a8_moe_prepack_mxfp4
    assert pm(P, P, 2, 24, 256, P, P, None) == ERR_SHAPE
    assert pm(P, None, 2, 32, 256, P, P, None) == ERR_NULL          # MXFP4 scales are required
    assert pm(P, P, 2, 32, 256, P + 8, P, None) == ERR_ALIGN
    assert pm(None, None, 0, 32, 256, None, None, None) == OK
    qm = L.w4a8_moe_quantize_weights_mxfp4
    assert qm(P, 4, 48, P, P, None) == ERR_SHAPE                    # K % 32
    assert qm(P, 4, 64, P, None, None) == ERR_NULL
    assert qm(P + 8, 4, 64, P, P, None) == ERR_ALIGN               # w 16-byte
    assert qm(P, 4, 64, P + 1, P, None) == ERR_ALIGN               # codes 2-byte
    assert qm(None, 0, 64, None, None, None) == OK
    gm = L.w4a8_moe_grouped_gemm_mxfp4
    assert gm(P, P, None, 64, P, 8, P, P, 24, 256, P, None) == ERR_SHAPE         # N % 16
    assert gm(P, P, None, 64, P, 8, P, P, 256, 192, P, None) == ERR_SHAPE        # K % 128
    assert gm(P, P, None, 64, P, 8, P, None, 256, 256, P, None) == ERR_NULL
    assert gm(P, P, None, 64, P, 8, P + 8, P, 256, 256, P, None) == ERR_ALIGN
    assert gm(None, None, None, 0, None, 8, None, None, 256, 256, None, None) == OK
    gmp = L.w4a8_moe_grouped_gemm_mxfp4_prepacked
    assert gmp(P, P, None, 64, P, 8, P, P, 96, 256, P, 0, None) == ERR_SHAPE     # N % 64
    assert gmp(P, P, None, 64, P, 8, P, P, 256, 256, P, 9, None) == ERR_SHAPE    # algo
    assert gmp(P, P, None, 64, P, 8, P, None, 256, 256, P, 0, None) == ERR_NULL
    assert gmp(None, None, None, 0, None, 8, None, None, 256, 256, None, 0, None) == OK


def test_later_calls_report_missing_device(L, no_device):
    if not no_device:
        pytest.skip("a supported GPU is present; these fake pointers must not reach it")
    assert L.w4a8_moe_quant_act_i8(P, 4, 256, 256, P, P, P, None) == ERR_DEVICE
    assert L.w4a8_moe_grouped_gemm_i8(P, P, P, None, 8, P, 8, P, P, 256, 256, P, None) == ERR_DEVICE
    assert L.w4a8_moe_grouped_gemm_i8_prepacked(P, P, P, None, 8, P, 8, P, P, 256, 256, P, 0, None) == ERR_DEVICE
    assert L.w4a8_moe_grouped_gemm_prepacked(P, P, None, 8, P, 8, P, P, 256, 256, P, 0, None) == ERR_DEVICE
    assert L.w4a8_moe_grouped_gemm(P, P, None, 8, P, 8, P, P, 48, 256, P, None) == ERR_DEVICE
    assert L.w4a8_moe_swiglu_i8(P, 4, 128, P, P, P, None) == ERR_DEVICE
    assert L.w4a8_moe_quantize_weights_channel(P, 4, 128, P, P, None) == ERR_DEVICE
    assert L.w4a8_moe_grouped_gemm_swiglu(P, P, None, 8, P, 8, P, P, 128, 256, P, P, None) == ERR_DEVICE
    assert L.w4a8_moe_grouped_gemm_swiglu_prepacked(P, P, None, 8, P, 8, P, P, 128, 256, P, P, 0, None) == ERR_DEVICE
    assert L.w4a8_moe_grouped_gemm_swiglu_i8(P, P, P, None, 8, P, 8, P, P, 128, 256, P, P, None) == ERR_DEVICE
    assert L.w4a8_moe_grouped_gemm_swiglu_i8_prepacked(P, P, P, None, 8, P, 8, P, P, 128, 256, P, P, 0,
                                                       None) == ERR_DEVICE
    assert L.w4a8_moe_requant(P, P, 4, 128, P, P, None) == ERR_DEVICE
    assert L.w4a8_moe_requant_i8(P, P, 4, 128, P, P, P, None) == ERR_DEVICE
    assert L.w4a8_moe_quantize_weights_mxfp4(P, 4, 64, P, P, None) == ERR_DEVICE
    assert L.w4a8_moe_prepack_int4(P, P, 2, 32, 256, P, P, None) == ERR_DEVICE
    assert L.w4a8_moe_prepack_mxfp4(P, P, 2, 32, 256, P, P, None) == ERR_DEVICE
    assert L.w4a8_moe_grouped_gemm_mxfp4(P, P, None, 8, P, 8, P, P, 256, 256, P, None) == ERR_DEVICE
    assert L.w4a8_moe_grouped_gemm_mxfp4_prepacked(P, P, None, 8, P, 8, P, P, 256, 256, P, 0, None) == ERR_DEVICE
    assert L.w4a8_moe_grouped_gemm_swiglu_mxfp4(P, P, None, 8, P, 8, P, P, 128, 256, P, P, None) == ERR_DEVICE
    assert L.w4a8_moe_grouped_gemm_swiglu_mxfp4_prepacked(P, P, None, 8, P, 8, P, P, 128, 256, P, P, 0,
                                                          None) == ERR_DEVICE


def test_front_checks(L, no_device):
    f = L.w4a8_moe_front
    need = L.w4a8_moe_permute_workspace_bytes(128, 8, 256)

    def call(fn=f, int8=False, **kw):
        d = dict(x=P, T=128, H=6144, ld=6144, qx=P, sx=P, rs=P, lg=P, E=256, k=8, ren=1, ids=P, w=P, off=P, rt=P,
                 inv=P, ws=P, nws=need, cnt=P)
        d.update(kw)
        if int8:
            return fn(d["x"], d["T"], d["H"], d["ld"], d["qx"], d["sx"], d["rs"], d["lg"], d["E"], d["k"], d["ren"],
                      d["ids"], d["w"], d["off"], d["rt"], d["inv"], d["ws"], d["nws"], d["cnt"], None)
        return fn(d["x"], d["T"], d["H"], d["ld"], d["qx"], d["sx"], d["lg"], d["E"], d["k"], d["ren"], d["ids"],
                  d["w"], d["off"], d["rt"], d["inv"], d["ws"], d["nws"], d["cnt"], None)
    assert call(H=100, ld=100) == ERR_SHAPE
    assert call(k=9, E=8) == ERR_SHAPE
    assert call(cnt=None) == ERR_NULL                          # the counter is required
    assert call(nws=need - 4) == ERR_WORKSPACE
    assert call(cnt=P + 2) == ERR_ALIGN
    assert call(qx=P + 4) == ERR_ALIGN                         # qx 8-byte
    g = L.w4a8_moe_front_i8
    assert call(g, True, rs=None) == ERR_NULL                  # row sums are required
    assert call(g, True, H=200, ld=200) == ERR_SHAPE
    if no_device:
        assert call() == ERR_DEVICE
        assert call(g, True) == ERR_DEVICE


def test_last_error_per_thread(L):
    # each thread sees the detail of its own last call, whatever the others do meanwhile
    import threading
    errors = []

    def worker(i):
        for r in range(200):
            bad_h = 128 * (i + 1) + 1
            if L.w4a8_moe_swiglu(P, 4, bad_h, P, P, None) != ERR_SHAPE or f"I={bad_h}" not in ops.last_error():
                errors.append((i, r))
            if L.w4a8_moe_swiglu(None, 0, 128, None, None, None) != OK or ops.last_error() != "":
                errors.append((i, r, "ok"))
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors[:5]


def test_scatter_combine_checks(L, no_device):
    """Step 7 with the routing weights applied in the down GEMM's epilogue: the
    scatter GEMMs take the prepacked forms' checks plus a row_dst, and the row
    sources and combine calls check their own shapes."""
    g = L.w4a8_moe_grouped_gemm_scatter_prepacked
    mx = L.w4a8_moe_grouped_gemm_scatter_mxfp4_prepacked
    i8 = L.w4a8_moe_grouped_gemm_scatter_i8_prepacked
    for fn in (g, mx):
        assert fn(P, P, None, 64, P, 8, P, P, 256, 256, None, P, 0, None) == ERR_NULL     # row_dst
        assert fn(P, P, None, 64, P, 8, P, P, 256, 256, P + 2, P, 0, None) == ERR_ALIGN  # row_dst
        assert fn(P, P, None, 64, P, 8, P, P, 96, 256, P, P, 0, None) == ERR_SHAPE       # N % 64
        assert fn(P, P, None, 64, P, 8, P, P, 256, 256, P, P, 7, None) == ERR_SHAPE      # algo
        assert fn(None, None, None, 0, None, 8, None, None, 256, 256, None, None, 0, None) == OK
    assert i8(P, P, P, None, 64, P, 8, P, P, 256, 256, None, P, 0, None) == ERR_NULL
    assert i8(P, P, P, None, 64, P, 8, P, P, 256, 256, P + 2, P, 0, None) == ERR_ALIGN
    assert i8(None, None, None, None, 0, None, 8, None, None, 256, 256, None, None, 0, None) == OK

    rs = L.w4a8_moe_row_sources
    assert rs(P, P, P, 4, 0, 4, P, P, None) == ERR_SHAPE            # k >= 1
    assert rs(P, P, P, 4, 2, 9, P, P, None) == ERR_SHAPE            # M_total <= T k
    assert rs(P, P, P, -1, 2, 0, P, P, None) == ERR_SHAPE
    assert rs(P, None, P, 4, 2, 8, P, P, None) == ERR_NULL
    assert rs(P, P, P, 4, 2, 8, P, P + 2, None) == ERR_ALIGN
    assert rs(None, None, None, 0, 2, 0, None, None, None) == OK

    c = L.w4a8_moe_combine
    assert c(P, P, 4, 2, 100, P, 0, None) == ERR_SHAPE               # H % 128
    assert c(P, P, 4, 2, 256, P, 5, None) == ERR_SHAPE               # y dtype
    assert c(P, P, 4, 0, 256, P, 0, None) == ERR_SHAPE
    assert c(P + 4, P, 4, 2, 256, P, 0, None) == ERR_ALIGN           # o_tok 16 bytes
    assert c(P, P, 4, 2, 256, P + 8, 0, None) == ERR_ALIGN           # f32 y 16 bytes
    assert c(P, None, 4, 2, 256, P, 0, None) == ERR_NULL
    assert c(None, None, 0, 2, 256, None, 0, None) == OK
    if no_device:
        assert g(P, P, None, 64, P, 8, P, P, 256, 256, P, P, 0, None) == ERR_DEVICE
        assert i8(P, P, P, None, 64, P, 8, P, P, 256, 256, P, P, 0, None) == ERR_DEVICE
        assert mx(P, P, None, 64, P, 8, P, P, 256, 256, P, P, 0, None) == ERR_DEVICE
        assert rs(P, P, P, 4, 2, 8, P, P, None) == ERR_DEVICE
        assert c(P, P, 4, 2, 256, P + 8, 1, None) == ERR_DEVICE      # bf16 y: 8 bytes suffice


def test_native_caller_without_device(no_device, tmp_path):
    """The native C++ caller (built with the library) links against it through a relative path and,
    on a host without a gfx950, exits with status 2 and the library's message before any allocation."""
    from quantized_grouped_gemm_token_amd import build as B
    assert os.path.exists(B.C_CALLER), "build the library first (it builds the native caller too)"
    if not no_device:
        pytest.skip("a supported GPU is present; the GPU tests run the caller")
    r = subprocess.run([B.C_CALLER, str(tmp_path), "4", "256", "128", "8", "2"], capture_output=True, text=True,
                       timeout=60)
    assert r.returncode == 2, (r.returncode, r.stderr)
    assert "no gfx950 device" in r.stderr
    r = subprocess.run([B.C_CALLER, str(tmp_path), "4", "200", "128", "8", "2"], capture_output=True, text=True,
                       timeout=60)
    assert r.returncode == 1 and "bad sizes" in r.stderr
