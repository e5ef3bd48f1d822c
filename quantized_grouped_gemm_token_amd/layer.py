"""The W4A8 MoE routed-expert layer: the seven library steps chained on one stream.

    quant_act -> route -> permute -> grouped_gemm(W13) -> swiglu ->
    grouped_gemm(W2) -> unpermute

With fused=True (the default) steps 4 and 5 run as grouped_gemm_swiglu (the
gate/up GEMM with SwiGLU in its epilogue, writing act = silu(gate) * up and
partial row maxima of |act|) and requant (the codes of act): the same results with half
the intermediate bytes.

With scatter=True step 7 moves into the down GEMM's epilogue: row_sources
gives each GEMM row p its routed index f = t k + j and the scale
a_scale[p] w[t, j], the GEMM stores row p as row f (token-major, the routing
weight applied), and combine sums each token's k contiguous rows in j order.
scatter=None takes that path from SCATTER_MIN_ROWS routed rows on.

Expert weights are given in the packed format (int32 [E][N][K/8] words of
uint4b8 nibbles and fp32 [E][N][K/128] group scales) and stay resident on the
GPU in the GEMM storage (prepack_int4, once at construction: 1 KB per 16 rows
x 128 K, group-major scales), which the _prepacked GEMM calls read.
W4A8MoEChannel is the per-channel INT4 x per-token INT8 variant: fp32 [E][N]
scales, INT8 activations.  W4A8MoEMxfp4 holds MXFP4 group-32 experts (E2M1
codes uint8 [E][N][K/2], E8M0 scales uint8 [E][N][K/32]) and uses the same
FP8 activations.
Intermediate buffers are allocated once per token count and reused, so a
forward pass enqueues kernels only: no allocation, no host synchronisation.
That also makes a step capturable: capture() records one forward into a HIP
graph, whose replay re-runs the whole step on the current contents of the
same x, logits and y tensors with a single launch.
"""
from __future__ import annotations

import torch

from . import ops


class W4A8MoE:
    K_PER_ITEM = 8                                        # K elements per item of a weight row (int32 words)
    GEMM = staticmethod(ops.w4a8_moe_grouped_gemm_prepacked)
    GEMM_SWIGLU = staticmethod(ops.w4a8_moe_grouped_gemm_swiglu_prepacked)
    GEMM_SCATTER = staticmethod(ops.w4a8_moe_grouped_gemm_scatter_prepacked)
    SCATTER_MIN_ROWS = 1 << 62                            # scatter=None: the gather combine at every size

    def __init__(self, w13: torch.Tensor, s13: torch.Tensor, w2: torch.Tensor, s2: torch.Tensor, k: int,
                 renormalize: bool = True, fused: bool = True, front: bool = True, scatter: bool | None = None):
        E, N13, KW13 = w13.shape
        E2, H, KW2 = w2.shape
        c = self.K_PER_ITEM
        if E2 != E or N13 % 2 or KW13 * c != H or KW2 * c * 2 != N13:
            raise ValueError(f"w13 must be [E, 2I, H/{c}] and w2 [E, H, I/{c}]")
        self.w13, self.s13, self.w2, self.s2 = self.prepack(w13, s13, w2, s2)
        self.E, self.H, self.I, self.k = E, H, N13 // 2, k
        self.renormalize = renormalize
        self.fused = fused
        self.scatter = scatter
        self.front = front                                # steps 1-3 as one call (w4a8_moe_front)
        self.steps = (("front",) if front else ("quant_act", "route", "permute")) + self.STEPS[3:]
        self._bufs: dict[int, dict] = {}

    def buffers(self, T: int) -> dict:
        """Intermediate buffers for T tokens (allocated on first use)."""
        if T not in self._bufs:
            dev = self.w13.device
            R = T * self.k
            nbytes = ops.w4a8_moe_permute_workspace_bytes(T, self.k, self.E)
            e = lambda shape, dt: torch.empty(shape, dtype=dt, device=dev)  # noqa: E731
            self._bufs[T] = dict(
                qx=e((T, self.H), torch.uint8), sx=e((T,), torch.float32),
                ids=e((T, self.k), torch.int32), w=e((T, self.k), torch.float32),
                offsets=e((self.E + 1,), torch.int32), row_token=e((R,), torch.int32),
                inv_pos=e((R,), torch.int32), workspace=e((max(nbytes, 4),), torch.uint8),
                counter=torch.zeros((1,), dtype=torch.int32, device=dev),   # the front call's counter
                qa=e((R, self.I), torch.uint8), sa=e((R,), torch.float32), o=e((R, self.H), torch.float32),
                row_src=e((R,), torch.int32), row_scale=e((R,), torch.float32),
            )
            if self.fused:
                self._bufs[T].update(act=e((R, self.I), torch.float32), pmax=e((R, self.I // 64), torch.float32))
            else:
                self._bufs[T].update(h=e((R, 2 * self.I), torch.float32))
        return self._bufs[T]

    @staticmethod
    def prepack(w13, s13, w2, s2):
        """The experts in the GEMM storage."""
        w13b, s13b = ops.w4a8_moe_prepack_int4(w13, s13)
        w2b, s2b = ops.w4a8_moe_prepack_int4(w2, s2)
        return w13b, s13b, w2b, s2b

    STEPS = ("quant_act", "route", "permute", "gemm_gate_up", "swiglu", "gemm_down", "unpermute")

    def uses_scatter(self, T: int) -> bool:
        """Whether a forward over T tokens folds the routing weights into the down GEMM."""
        return self.scatter if self.scatter is not None else T * self.k >= self.SCATTER_MIN_ROWS

    def forward(self, x: torch.Tensor, logits: torch.Tensor, y: torch.Tensor | None = None,
                y_dtype: torch.dtype = torch.float32, algo: int = ops.W4A8_GG_AUTO,
                events: dict | None = None) -> torch.Tensor:
        """x bf16 [T, H], router logits fp32 [T, E] -> y [T, H].

        events, if given, maps step names (self.steps) to (start, end) CUDA
        events that are recorded on the current stream around each step.
        """
        T = x.shape[0]
        b = self.buffers(T)
        R = T * self.k

        def step(name, fn, *args):
            ev = events.get(name) if events else None
            if ev:
                ev[0].record()
            r = fn(*args)
            if ev:
                ev[1].record()
            return r

        if self.front:
            step("front", ops.w4a8_moe_front, x, logits, self.k, b["counter"], self.renormalize, False, b["qx"],
                 b["sx"], None, b["ids"], b["w"], b["offsets"], b["row_token"], b["inv_pos"], b["workspace"])
        else:
            step("quant_act", ops.w4a8_moe_quant_act, x, b["qx"], b["sx"])
            step("route", ops.w4a8_moe_route, logits, self.k, self.renormalize, b["ids"], b["w"])
            step("permute", ops.w4a8_moe_permute, b["ids"], self.E, b["offsets"], b["row_token"], b["inv_pos"],
                 b["workspace"])
        if self.fused:
            step("gemm_gate_up", self.GEMM_SWIGLU, b["qx"], b["sx"], b["row_token"], b["offsets"],
                 self.w13, self.s13, R, b["act"], b["pmax"], algo)
            step("swiglu", ops.w4a8_moe_requant, b["act"], b["pmax"], b["qa"], b["sa"])
        else:
            step("gemm_gate_up", self.GEMM, b["qx"], b["sx"], b["row_token"], b["offsets"],
                 self.w13, self.s13, R, b["h"], algo)
            step("swiglu", ops.w4a8_moe_swiglu, b["h"], b["qa"], b["sa"])
        if self.uses_scatter(T):
            def down():
                ops.w4a8_moe_row_sources(b["inv_pos"], b["w"], b["sa"], R, b["row_src"], b["row_scale"])
                self.GEMM_SCATTER(b["qa"], b["row_scale"], None, b["offsets"], self.w2, self.s2, R, b["row_src"],
                                  b["o"], algo)
            step("gemm_down", down)
            return step("unpermute", ops.w4a8_moe_combine, b["o"], b["inv_pos"], T, self.k, y, y_dtype)
        step("gemm_down", self.GEMM, b["qa"], b["sa"], None, b["offsets"], self.w2, self.s2, R, b["o"], algo)
        return step("unpermute", ops.w4a8_moe_unpermute, b["o"], b["inv_pos"], b["w"], y, y_dtype)

    __call__ = forward

    def capture(self, x: torch.Tensor, logits: torch.Tensor, y: torch.Tensor,
                y_dtype: torch.dtype = torch.float32, algo: int = ops.W4A8_GG_AUTO) -> torch.cuda.CUDAGraph:
        """Record one forward on these tensors into a HIP graph and return it.

        One eager forward runs first (it allocates the per-T buffers, which the
        captured kernels then use); g.replay() then runs the step again on the
        tensors' current contents.  The step enqueues no memset and no copy,
        so the graph holds kernel nodes only."""
        self.forward(x, logits, y, y_dtype=y_dtype, algo=algo)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.forward(x, logits, y, y_dtype=y_dtype, algo=algo)
        torch.cuda.synchronize()
        return g


class W4A8MoEChannel(W4A8MoE):
    """The per-channel INT4 x per-token INT8 variant: s13 [E, 2I] and s2 [E, H]
    are per-channel scales; steps 1, 4, 5 and 6 use the INT8 calls."""

    @staticmethod
    def prepack(w13, s13, w2, s2):
        return ops.w4a8_moe_prepack_int4(w13)[0], s13, ops.w4a8_moe_prepack_int4(w2)[0], s2

    def buffers(self, T: int) -> dict:
        if T not in self._bufs:
            b = dict(super().buffers(T))
            dev = self.w13.device
            R = T * self.k
            b["qx"] = torch.empty((T, self.H), dtype=torch.int8, device=dev)
            b["rx"] = torch.empty((T,), dtype=torch.int32, device=dev)
            b["qa"] = torch.empty((R, self.I), dtype=torch.int8, device=dev)
            b["ra"] = torch.empty((R,), dtype=torch.int32, device=dev)
            self._bufs[T] = b
        return self._bufs[T]

    def forward(self, x: torch.Tensor, logits: torch.Tensor, y: torch.Tensor | None = None,
                y_dtype: torch.dtype = torch.float32, algo: int = ops.W4A8_GG_AUTO,
                events: dict | None = None) -> torch.Tensor:
        T = x.shape[0]
        b = self.buffers(T)
        R = T * self.k

        def step(name, fn, *args):
            ev = events.get(name) if events else None
            if ev:
                ev[0].record()
            r = fn(*args)
            if ev:
                ev[1].record()
            return r

        if self.front:
            step("front", ops.w4a8_moe_front, x, logits, self.k, b["counter"], self.renormalize, True, b["qx"],
                 b["sx"], b["rx"], b["ids"], b["w"], b["offsets"], b["row_token"], b["inv_pos"], b["workspace"])
        else:
            step("quant_act", ops.w4a8_moe_quant_act_i8, x, b["qx"], b["sx"], b["rx"])
            step("route", ops.w4a8_moe_route, logits, self.k, self.renormalize, b["ids"], b["w"])
            step("permute", ops.w4a8_moe_permute, b["ids"], self.E, b["offsets"], b["row_token"], b["inv_pos"],
                 b["workspace"])
        if self.fused:
            step("gemm_gate_up", ops.w4a8_moe_grouped_gemm_swiglu_i8_prepacked, b["qx"], b["sx"], b["rx"],
                 b["row_token"], b["offsets"], self.w13, self.s13, R, b["act"], b["pmax"], algo)
            step("swiglu", ops.w4a8_moe_requant_i8, b["act"], b["pmax"], b["qa"], b["sa"], b["ra"])
        else:
            step("gemm_gate_up", ops.w4a8_moe_grouped_gemm_i8_prepacked, b["qx"], b["sx"], b["rx"],
                 b["row_token"], b["offsets"], self.w13, self.s13, b["h"], R, algo)
            step("swiglu", ops.w4a8_moe_swiglu_i8, b["h"], b["qa"], b["sa"], b["ra"])
        if self.uses_scatter(T):
            def down():
                ops.w4a8_moe_row_sources(b["inv_pos"], b["w"], b["sa"], R, b["row_src"], b["row_scale"])
                ops.w4a8_moe_grouped_gemm_scatter_i8_prepacked(b["qa"], b["row_scale"], b["ra"], None, b["offsets"],
                                                              self.w2, self.s2, R, b["row_src"], b["o"], algo)
            step("gemm_down", down)
            return step("unpermute", ops.w4a8_moe_combine, b["o"], b["inv_pos"], T, self.k, y, y_dtype)
        step("gemm_down", ops.w4a8_moe_grouped_gemm_i8_prepacked, b["qa"], b["sa"], b["ra"], None, b["offsets"],
             self.w2, self.s2, b["o"], R, algo)
        return step("unpermute", ops.w4a8_moe_unpermute, b["o"], b["inv_pos"], b["w"], y, y_dtype)

    __call__ = forward


class W4A8MoEMxfp4(W4A8MoE):
    """MXFP4 group-32 experts given row-major (w13 uint8 [E, 2I, H/2], s13 uint8
    [E, 2I, H/32], w2 uint8 [E, H, I/2], s2 uint8 [E, H, I/32]) and kept in the
    GEMM storage (prepack_mxfp4, once at construction), with the FP8
    activations of the group-128 form: only the two GEMMs differ."""
    K_PER_ITEM = 2                                        # two E2M1 codes per byte
    GEMM = staticmethod(ops.w4a8_moe_grouped_gemm_mxfp4_prepacked)
    GEMM_SWIGLU = staticmethod(ops.w4a8_moe_grouped_gemm_swiglu_mxfp4_prepacked)
    GEMM_SCATTER = staticmethod(ops.w4a8_moe_grouped_gemm_scatter_mxfp4_prepacked)

    @staticmethod
    def prepack(w13, s13, w2, s2):
        w13b, s13b = ops.w4a8_moe_prepack_mxfp4(w13, s13)
        w2b, s2b = ops.w4a8_moe_prepack_mxfp4(w2, s2)
        return w13b, s13b, w2b, s2b
