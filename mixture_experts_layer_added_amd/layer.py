"""MoE layer object: owns the device buffers of one batch size and issues the five
C-ABI calls on the current stream.  Plumbing only (allocation and argument
marshalling); every step runs in libmoe's HIP kernels.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import _lib as L

_DT = {"f32": L.MOE_F32, "bf16": L.MOE_BF16, "e4m3": L.MOE_FP8_E4M3}


@dataclass
class Shape:
    T: int
    H: int
    E: int
    G: int
    M: int
    K: int
    J: int
    I: int
    S: int = 1
    act: str = "bf16"
    expert: str = "bf16"

    def problem(self) -> L.moe_problem:
        return L.problem(self.T, self.H, self.E, self.G, self.M, self.K, self.J, self.I, self.S,
                         _DT[self.act], _DT[self.expert])

    @property
    def R(self) -> int:
        return self.T * self.K + self.S * self.T


def quantize_weights_fp8(w: torch.Tensor, stream=None):
    """bf16 [batch, rows, cols] -> (E4M3 codes uint8 [batch, rows, cols],
    fp32 scales [batch, rows/128, cols/128])."""
    assert w.dtype == torch.bfloat16 and w.dim() == 3 and w.is_contiguous()
    b, r, c = w.shape
    q = torch.empty((b, r, c), dtype=torch.uint8, device=w.device)
    s = torch.empty((b, r // 128, c // 128), dtype=torch.float32, device=w.device)
    L.moe_quantize_weights_fp8(w, q, s, b, r, c, stream)
    return q, s


# batches up to this mean load per routed expert use the packed-weight GEMMs by default
PACKED_MAX_MEAN_ROWS = 160


class MoELayer:
    """Buffers for one batch of T tokens.

    Weights: w_router [E,H] fp32, bias [E] fp32 (updated in place by bias_step),
    w13 [E+S,2I,H] and w2 [E+S,H,I] in the expert dtype (uint8 E4M3 codes with
    w13_scale / w2_scale for the FP8 path).

    gather=False: permute writes x_sorted and the gate/up GEMM reads it.
    gather=True:  permute writes the index maps only (FP8: plus one quantisation of x
    per token) and the gate/up GEMM reads its rows from x through sorted_token; the
    results are identical and the permuted copy of x is never written.
    train=True (bf16 / fp32): the gate/up GEMM also keeps the pre-activations (au) and
    backward(dy) computes dx, dw_router, dw13 and dw2 (weight gradients in fp32).
    packed (bf16 and FP8 experts): the expert GEMMs run over copies of w13 and w2 in the
    library's packed layout, made once here (bf16: the same results bit for bit; with
    train, the backward input part also runs over packed copies of the transposed
    matrices, the same results bit for bit).  Default: on when the
    mean load per routed expert, T*K/E, is at most PACKED_MAX_MEAN_ROWS -- the packed
    kernels take at most 192 rows of an expert per tile (a larger expert streams its
    weights once per tile), the natural-layout kernels 256.
    """

    def __init__(self, shape: Shape, w_router, bias, w13, w2, w13_scale=None, w2_scale=None,
                 device="cuda", gather=False, train=False, packed=None):
        self.shape = shape
        self.gather = gather
        self.train = train
        can_pack = shape.act == "bf16" and shape.expert in ("bf16", "e4m3")
        if packed is None:
            packed = can_pack and shape.T * shape.K <= PACKED_MAX_MEAN_ROWS * shape.E
        self.packed = bool(packed)
        assert can_pack or not self.packed, "packed weights are built for the bf16 and FP8 paths"
        self._x = None
        self._xin = None
        self.p = shape.problem()
        self.w_router, self.bias = w_router, bias
        self.w13, self.w2, self.w13_scale, self.w2_scale = w13, w2, w13_scale, w2_scale
        self.w13p = self.w2p = self.w13tp = self.w2tp = None
        if self.packed:
            self.w13p, self.w2p = torch.empty_like(w13), torch.empty_like(w2)
            L.moe_pack_expert_weights(self.p, w13, w2, self.w13p, self.w2p)
            if train and shape.expert == "bf16":  # the backward's transposed copies
                self.w13tp, self.w2tp = torch.empty_like(w13), torch.empty_like(w2)
                L.moe_pack_expert_weights_transposed(self.p, w13, w2, self.w13tp, self.w2tp)
        T, H, E, K, R = shape.T, shape.H, shape.E, shape.K, shape.R
        act = torch.float32 if shape.act == "f32" else torch.bfloat16
        dev = torch.device(device)
        i32 = dict(dtype=torch.int32, device=dev)
        self.topk_idx = torch.empty((T, K), **i32)
        self.topk_gate = torch.empty((T, K), dtype=torch.float32, device=dev)
        self.counts = torch.empty((E,), **i32)
        self.logits = torch.empty((T, E), dtype=torch.float32, device=dev)
        self.offsets = torch.empty((E + shape.S + 1,), **i32)
        self.sorted_token = torch.empty((R,), **i32)
        self.inv_perm = torch.empty((T, K), **i32)
        rows = T if gather else R  # gather: x itself (FP8: its per-token codes)
        self.x_sorted = None
        if shape.expert == "e4m3":
            self.x_q = torch.empty((rows, H), dtype=torch.uint8, device=dev)
            self.x_scale = torch.empty((rows, H // 128), dtype=torch.float32, device=dev)
        else:
            self.x_q = None if gather else torch.empty((R, H), dtype=act, device=dev)
            self.x_scale = None
        if not gather:
            self.x_sorted = self.x_q
        if shape.expert == "e4m3":
            self.h = torch.empty((R, shape.I), dtype=torch.uint8, device=dev)
            self.h_scale = torch.empty((R, shape.I // 128), dtype=torch.float32, device=dev)
        else:
            self.h = torch.empty((R, shape.I), dtype=act, device=dev)
            self.h_scale = None
        self.y_sorted = torch.empty((R, H), dtype=act, device=dev)
        self.y = torch.empty((T, H), dtype=act, device=dev)
        if train:
            assert shape.expert != "e4m3", "the backward is built for the bf16 and fp32 paths"
            NG, I, f32 = E + shape.S, shape.I, torch.float32
            self.au = torch.empty((R, 2 * I), dtype=act, device=dev)
            self.dy_sorted = torch.empty((R, H), dtype=act, device=dev)
            self.dgate = torch.empty((T, K), dtype=f32, device=dev)
            self.dz = torch.empty((T, K), dtype=f32, device=dev)
            self.dx_router = torch.empty((T, H), dtype=f32, device=dev)
            self.dw_router = torch.empty((E, H), dtype=f32, device=dev)
            self.dau = torch.empty((R, 2 * I), dtype=act, device=dev)
            self.dx_sorted = torch.empty((R, H), dtype=act, device=dev)
            self.dw13 = torch.empty((NG, 2 * I, H), dtype=f32, device=dev)
            self.dw2 = torch.empty((NG, H, I), dtype=f32, device=dev)
            self.dx = torch.empty((T, H), dtype=act, device=dev)
        self.ws = {}
        for call in (L.MOE_CALL_ROUTE, L.MOE_CALL_PERMUTE):
            n = L.moe_workspace_bytes(self.p, call)
            if n == 0 and call != L.MOE_CALL_ROUTE:
                raise L.MoeError(L.MOE_ERR_INVALID_ARG, "moe_workspace_bytes", L.last_error())
            self.ws[call] = torch.empty((max(n, 256),), dtype=torch.uint8, device=dev)

    def _ws(self, call):
        t = self.ws[call]
        return t, t.numel()

    def route(self, x, stream=None):
        L.moe_route(self.p, x, self.w_router, self.bias, self.topk_idx, self.topk_gate,
                    self.counts, self.logits, None, 0, stream)

    def permute(self, x, stream=None):
        ws, n = self._ws(L.MOE_CALL_PERMUTE)
        if self.gather:
            L.moe_permute(self.p, x, self.topk_idx, self.offsets, self.sorted_token,
                          self.inv_perm, None, None, ws, n, stream)
            if self.shape.expert == "e4m3":
                L.moe_quantize_act_fp8(self.p, x, self.x_q, self.x_scale, stream)
            self._x = x
        else:
            L.moe_permute(self.p, x, self.topk_idx, self.offsets, self.sorted_token,
                          self.inv_perm, self.x_sorted, self.x_scale, ws, n, stream)
            self._xin = x

    def expert_ffn_up(self, stream=None):
        if self.packed:
            if self.shape.expert == "e4m3":
                xin, st = (self.x_q, self.sorted_token) if self.gather else (self.x_sorted, None)
            else:
                xin, st = (self._x, self.sorted_token) if self.gather else (self.x_sorted, None)
            L.moe_expert_ffn_up_packed(self.p, xin, self.x_scale, st, self.offsets, self.w13,
                                       self.w13p, self.w13_scale, self.h, self.h_scale,
                                       self.au if self.train else None, stream)
        elif self.train:
            xin, st = (self._x, self.sorted_token) if self.gather else (self.x_sorted, None)
            L.moe_expert_ffn_up_save(self.p, xin, st, self.offsets, self.w13, self.h, self.au,
                                     stream)
        elif self.gather:
            xin = self.x_q if self.shape.expert == "e4m3" else self._x
            L.moe_expert_ffn_up_gather(self.p, xin, self.x_scale, self.sorted_token,
                                       self.offsets, self.w13, self.w13_scale, self.h,
                                       self.h_scale, stream)
        else:
            L.moe_expert_ffn_up(self.p, self.x_sorted, self.x_scale, self.offsets, self.w13,
                                self.w13_scale, self.h, self.h_scale, stream)

    def expert_ffn_down(self, stream=None):
        if self.packed:
            L.moe_expert_ffn_down_packed(self.p, self.h, self.h_scale, self.offsets, self.w2p,
                                         self.w2_scale, self.y_sorted, stream)
            return
        L.moe_expert_ffn_down(self.p, self.h, self.h_scale, self.offsets, self.w2, self.w2_scale,
                              self.y_sorted, stream)

    def expert_ffn(self, stream=None):
        self.expert_ffn_up(stream)
        self.expert_ffn_down(stream)

    def combine(self, stream=None):
        L.moe_combine(self.p, self.y_sorted, self.inv_perm, self.topk_gate, self.y, stream)

    def forward(self, x, stream=None):
        """route -> permute -> expert FFN -> combine; returns self.y (overwritten by the
        next call)."""
        self.route(x, stream)
        self.permute(x, stream)
        self.expert_ffn(stream)
        self.combine(stream)
        return self.y

    def bias_step(self, gamma=0.01, stream=None):
        """Aux-loss-free bias update from this batch's expert counts (in place)."""
        L.moe_bias_update(self.p, self.counts, gamma, self.bias, stream)

    def expert_ffn_backward_input(self, stream=None):
        if self.w13tp is not None:
            L.moe_expert_ffn_backward_input_packed(self.p, self.offsets, self.w13tp, self.w2tp,
                                                   self.au, self.dy_sorted, self.dau,
                                                   self.dx_sorted, stream)
            return
        L.moe_expert_ffn_backward_input(self.p, self.offsets, self.w13, self.w2, self.au,
                                        self.dy_sorted, self.dau, self.dx_sorted, stream)

    def expert_ffn_backward_weight(self, stream=None):
        xin, st = (self._x, self.sorted_token) if self.gather else (self.x_sorted, None)
        L.moe_expert_ffn_backward_weight(self.p, xin, st, self.offsets, self.h, self.dy_sorted,
                                         self.dau, self.dw13, self.dw2, stream)

    def combine_backward(self, dy, stream=None):
        L.moe_combine_backward(self.p, dy, self.y_sorted, self.inv_perm, self.topk_gate,
                               self.dy_sorted, self.dgate, stream)

    def router_backward(self, stream=None):
        x = self._x if self.gather else self._xin
        L.moe_router_backward(self.p, x, self.w_router, self.logits, self.topk_idx,
                              self.topk_gate, self.dgate, self.offsets, self.sorted_token,
                              self.dz, self.dx_router, self.dw_router, stream)

    def unpermute_sum(self, stream=None):
        L.moe_unpermute_sum(self.p, self.dx_sorted, self.inv_perm, self.dx_router, self.dx,
                            stream)

    def backward(self, dy, stream=None):
        """Gradients of sum(dy * y) for the last forward (train=True): returns self.dx and
        fills dw_router, dw13, dw2 (fp32).  The routing bias has no gradient."""
        assert self.train, "construct the layer with train=True"
        self.combine_backward(dy, stream)
        self.router_backward(stream)
        self.expert_ffn_backward_input(stream)
        self.expert_ffn_backward_weight(stream)
        self.unpermute_sum(stream)
        return self.dx

    def step(self, x, gamma=0.01, stream=None):
        y = self.forward(x, stream)
        self.bias_step(gamma, stream)
        return y
