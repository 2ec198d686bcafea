"""Thin ctypes binding of libmoe.so: the C ABI's calls under the same names.

Argument marshalling only: every step of the layer runs in the HIP kernels behind
these calls.  Tensors are passed as device pointers (``tensor.data_ptr()``) with the
current torch stream.  There is no fallback: if the library is missing or the
device is not gfx950 the calls raise.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
MOE_F32, MOE_BF16, MOE_FP8_E4M3 = 0, 1, 2
MOE_CALL_ROUTE, MOE_CALL_PERMUTE, MOE_CALL_EXPERT_FFN = 0, 1, 2

EXPORTS = ("moe_route", "moe_permute", "moe_expert_ffn", "moe_expert_ffn_up",
           "moe_expert_ffn_up_gather", "moe_quantize_act_fp8", "moe_expert_ffn_down",
           "moe_combine", "moe_bias_update", "moe_quantize_weights_fp8", "moe_workspace_bytes",
           "moe_status_str", "moe_last_error", "moe_expert_ffn_up_save", "moe_combine_backward",
           "moe_router_backward", "moe_expert_ffn_backward_input",
           "moe_expert_ffn_backward_weight", "moe_unpermute_sum", "moe_permute_noalloc",
           "moe_count_invalid_ids",
           "moe_seq_load_stats", "moe_pack_expert_weights", "moe_expert_ffn_up_packed",
           "moe_expert_ffn_down_packed", "moe_pack_expert_weights_transposed",
           "moe_expert_ffn_backward_input_packed")


class MoeError(RuntimeError):
    def __init__(self, status: int, call: str, msg: str):
        super().__init__(f"{call} failed with status {status}: {msg}")
        self.status = status


class moe_problem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("H", ctypes.c_int32), ("E", ctypes.c_int32),
                ("G", ctypes.c_int32), ("M", ctypes.c_int32), ("K", ctypes.c_int32),
                ("J", ctypes.c_int32), ("I", ctypes.c_int32), ("S", ctypes.c_int32),
                ("act_dtype", ctypes.c_int32), ("expert_dtype", ctypes.c_int32)]


_lib = None


def lib():
    """Load libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m mixture_experts_layer_added_amd.build`")
        # libmoe and torch must share one HIP runtime.  torch ships its own copy under
        # the same soname (libamdhip64.so.7); the first copy loaded serves the whole
        # process, so torch's is loaded before libmoe resolves its dependency.
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i32, i64, f32 = (ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64,
                                 ctypes.c_float)
        pp = ctypes.POINTER(moe_problem)
        L.moe_route.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_permute.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_permute_noalloc.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.moe_count_invalid_ids.argtypes = [pp, vp, vp, vp]
        L.moe_seq_load_stats.argtypes = [pp, vp, vp, i32, vp, vp, vp, vp]
        L.moe_expert_ffn.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_expert_ffn_up.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.moe_expert_ffn_up_gather.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.moe_quantize_act_fp8.argtypes = [pp, vp, vp, vp, vp]
        L.moe_expert_ffn_up_save.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp]
        L.moe_combine_backward.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp]
        L.moe_router_backward.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.moe_expert_ffn_backward_input.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.moe_expert_ffn_backward_weight.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.moe_unpermute_sum.argtypes = [pp, vp, vp, vp, vp, vp]
        L.moe_expert_ffn_down.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp]
        L.moe_pack_expert_weights.argtypes = [pp, vp, vp, vp, vp, vp]
        L.moe_pack_expert_weights_transposed.argtypes = [pp, vp, vp, vp, vp, vp]
        L.moe_expert_ffn_backward_input_packed.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.moe_expert_ffn_up_packed.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.moe_expert_ffn_down_packed.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp]
        L.moe_combine.argtypes = [pp, vp, vp, vp, vp, vp]
        L.moe_bias_update.argtypes = [pp, vp, f32, vp, vp]
        L.moe_quantize_weights_fp8.argtypes = [vp, vp, vp, i64, i32, i32, vp]
        L.moe_workspace_bytes.argtypes = [pp, i32]
        L.moe_workspace_bytes.restype = sz
        L.moe_status_str.argtypes = [i32]
        L.moe_status_str.restype = ctypes.c_char_p
        L.moe_last_error.argtypes = []
        L.moe_last_error.restype = ctypes.c_char_p
        for n in ("moe_route", "moe_permute", "moe_expert_ffn", "moe_expert_ffn_up",
                  "moe_expert_ffn_up_gather", "moe_quantize_act_fp8", "moe_expert_ffn_down",
                  "moe_combine", "moe_bias_update", "moe_quantize_weights_fp8",
                  "moe_expert_ffn_up_save", "moe_combine_backward", "moe_router_backward",
                  "moe_expert_ffn_backward_input", "moe_expert_ffn_backward_weight",
                  "moe_unpermute_sum", "moe_permute_noalloc", "moe_count_invalid_ids",
                  "moe_seq_load_stats",
                  "moe_pack_expert_weights", "moe_expert_ffn_up_packed",
                  "moe_expert_ffn_down_packed", "moe_pack_expert_weights_transposed",
                  "moe_expert_ffn_backward_input_packed"):
            getattr(L, n).restype = i32
        _lib = L
    return _lib


def problem(T, H, E, G, M, K, J, I, S=1, act_dtype=MOE_BF16, expert_dtype=MOE_BF16) -> moe_problem:
    return moe_problem(T, H, E, G, M, K, J, I, S, act_dtype, expert_dtype)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, call: str):
    if status != MOE_OK:
        raise MoeError(status, call, lib().moe_last_error().decode())


def last_error() -> str:
    return lib().moe_last_error().decode()


def moe_workspace_bytes(p: moe_problem, which_call: int) -> int:
    return lib().moe_workspace_bytes(ctypes.byref(p), which_call)


def moe_route(p, x, w_router, bias, topk_idx, topk_gate, expert_counts, logits_out=None,
              ws=None, ws_bytes=0, stream=None):
    _check(lib().moe_route(ctypes.byref(p), _ptr(x), _ptr(w_router), _ptr(bias), _ptr(topk_idx),
                           _ptr(topk_gate), _ptr(expert_counts), _ptr(logits_out), _ptr(ws),
                           ws_bytes, _stream(stream)), "moe_route")


def moe_permute(p, x, topk_idx, offsets, sorted_token, inv_perm, x_sorted, x_sorted_scale=None,
                ws=None, ws_bytes=0, stream=None):
    _check(lib().moe_permute(ctypes.byref(p), _ptr(x), _ptr(topk_idx), _ptr(offsets),
                             _ptr(sorted_token), _ptr(inv_perm), _ptr(x_sorted),
                             _ptr(x_sorted_scale), _ptr(ws), ws_bytes, _stream(stream)),
           "moe_permute")


def moe_count_invalid_ids(p, topk_idx, n_invalid, stream=None):
    _check(lib().moe_count_invalid_ids(ctypes.byref(p), _ptr(topk_idx), _ptr(n_invalid),
                                       _stream(stream)), "moe_count_invalid_ids")


def moe_permute_noalloc(p, x, topk_idx, offsets, sorted_token, inv_perm, x_sorted,
                        x_sorted_scale=None, stream=None):
    _check(lib().moe_permute_noalloc(ctypes.byref(p), _ptr(x), _ptr(topk_idx), _ptr(offsets),
                                     _ptr(sorted_token), _ptr(inv_perm), _ptr(x_sorted),
                                     _ptr(x_sorted_scale), _stream(stream)),
           "moe_permute_noalloc")


def moe_seq_load_stats(p, topk_idx, seq_offsets, n_seq, seq_counts, seq_stats, seq_ratio,
                       stream=None):
    _check(lib().moe_seq_load_stats(ctypes.byref(p), _ptr(topk_idx), _ptr(seq_offsets), n_seq,
                                    _ptr(seq_counts), _ptr(seq_stats), _ptr(seq_ratio),
                                    _stream(stream)), "moe_seq_load_stats")


def moe_expert_ffn(p, x_sorted, x_sorted_scale, offsets, w13, w13_scale, w2, w2_scale, y_sorted,
                   ws=None, ws_bytes=0, stream=None):
    _check(lib().moe_expert_ffn(ctypes.byref(p), _ptr(x_sorted), _ptr(x_sorted_scale),
                                _ptr(offsets), _ptr(w13), _ptr(w13_scale), _ptr(w2),
                                _ptr(w2_scale), _ptr(y_sorted), _ptr(ws), ws_bytes,
                                _stream(stream)), "moe_expert_ffn")


def moe_expert_ffn_up(p, x_sorted, x_sorted_scale, offsets, w13, w13_scale, h, h_scale=None,
                      stream=None):
    _check(lib().moe_expert_ffn_up(ctypes.byref(p), _ptr(x_sorted), _ptr(x_sorted_scale),
                                   _ptr(offsets), _ptr(w13), _ptr(w13_scale), _ptr(h),
                                   _ptr(h_scale), _stream(stream)), "moe_expert_ffn_up")


def moe_expert_ffn_up_gather(p, x, x_scale, sorted_token, offsets, w13, w13_scale, h,
                             h_scale=None, stream=None):
    _check(lib().moe_expert_ffn_up_gather(ctypes.byref(p), _ptr(x), _ptr(x_scale),
                                          _ptr(sorted_token), _ptr(offsets), _ptr(w13),
                                          _ptr(w13_scale), _ptr(h), _ptr(h_scale),
                                          _stream(stream)), "moe_expert_ffn_up_gather")


def moe_quantize_act_fp8(p, x, x_q, x_scale, stream=None):
    _check(lib().moe_quantize_act_fp8(ctypes.byref(p), _ptr(x), _ptr(x_q), _ptr(x_scale),
                                      _stream(stream)), "moe_quantize_act_fp8")


def moe_expert_ffn_down(p, h, h_scale, offsets, w2, w2_scale, y_sorted, stream=None):
    _check(lib().moe_expert_ffn_down(ctypes.byref(p), _ptr(h), _ptr(h_scale), _ptr(offsets),
                                     _ptr(w2), _ptr(w2_scale), _ptr(y_sorted), _stream(stream)),
           "moe_expert_ffn_down")


def moe_combine(p, y_sorted, inv_perm, topk_gate, y, stream=None):
    _check(lib().moe_combine(ctypes.byref(p), _ptr(y_sorted), _ptr(inv_perm), _ptr(topk_gate),
                             _ptr(y), _stream(stream)), "moe_combine")


def moe_bias_update(p, expert_counts, gamma, bias, stream=None):
    _check(lib().moe_bias_update(ctypes.byref(p), _ptr(expert_counts), float(gamma), _ptr(bias),
                                 _stream(stream)), "moe_bias_update")


def moe_quantize_weights_fp8(w_bf16, w_fp8, scale, batch, rows, cols, stream=None):
    _check(lib().moe_quantize_weights_fp8(_ptr(w_bf16), _ptr(w_fp8), _ptr(scale), batch, rows,
                                          cols, _stream(stream)), "moe_quantize_weights_fp8")



def moe_pack_expert_weights(p, w13, w2, w13_packed, w2_packed, stream=None):
    _check(lib().moe_pack_expert_weights(ctypes.byref(p), _ptr(w13), _ptr(w2), _ptr(w13_packed),
                                         _ptr(w2_packed), _stream(stream)),
           "moe_pack_expert_weights")


def moe_expert_ffn_up_packed(p, x, x_scale, sorted_token, offsets, w13, w13_packed, w13_scale,
                             h, h_scale, au=None, stream=None):
    _check(lib().moe_expert_ffn_up_packed(ctypes.byref(p), _ptr(x), _ptr(x_scale),
                                          _ptr(sorted_token), _ptr(offsets), _ptr(w13),
                                          _ptr(w13_packed), _ptr(w13_scale), _ptr(h),
                                          _ptr(h_scale), _ptr(au), _stream(stream)),
           "moe_expert_ffn_up_packed")


def moe_expert_ffn_down_packed(p, h, h_scale, offsets, w2_packed, w2_scale, y_sorted,
                               stream=None):
    _check(lib().moe_expert_ffn_down_packed(ctypes.byref(p), _ptr(h), _ptr(h_scale),
                                            _ptr(offsets), _ptr(w2_packed), _ptr(w2_scale),
                                            _ptr(y_sorted), _stream(stream)),
           "moe_expert_ffn_down_packed")


def moe_expert_ffn_up_save(p, x, sorted_token, offsets, w13, h, au, stream=None):
    _check(lib().moe_expert_ffn_up_save(ctypes.byref(p), _ptr(x), _ptr(sorted_token),
                                        _ptr(offsets), _ptr(w13), _ptr(h), _ptr(au),
                                        _stream(stream)), "moe_expert_ffn_up_save")


def moe_combine_backward(p, dy, y_sorted, inv_perm, topk_gate, dy_sorted, dgate, stream=None):
    _check(lib().moe_combine_backward(ctypes.byref(p), _ptr(dy), _ptr(y_sorted), _ptr(inv_perm),
                                      _ptr(topk_gate), _ptr(dy_sorted), _ptr(dgate),
                                      _stream(stream)), "moe_combine_backward")


def moe_router_backward(p, x, w_router, logits, topk_idx, topk_gate, dgate, offsets,
                        sorted_token, dz, dx_router, dw_router, stream=None):
    _check(lib().moe_router_backward(ctypes.byref(p), _ptr(x), _ptr(w_router), _ptr(logits),
                                     _ptr(topk_idx), _ptr(topk_gate), _ptr(dgate),
                                     _ptr(offsets), _ptr(sorted_token), _ptr(dz),
                                     _ptr(dx_router), _ptr(dw_router), _stream(stream)),
           "moe_router_backward")


def moe_pack_expert_weights_transposed(p, w13, w2, w13t_packed, w2t_packed, stream=None):
    _check(lib().moe_pack_expert_weights_transposed(ctypes.byref(p), _ptr(w13), _ptr(w2),
                                                    _ptr(w13t_packed), _ptr(w2t_packed),
                                                    _stream(stream)),
           "moe_pack_expert_weights_transposed")


def moe_expert_ffn_backward_input_packed(p, offsets, w13t_packed, w2t_packed, au, dy_sorted,
                                         dau, dx_sorted, stream=None):
    _check(lib().moe_expert_ffn_backward_input_packed(
        ctypes.byref(p), _ptr(offsets), _ptr(w13t_packed), _ptr(w2t_packed), _ptr(au),
        _ptr(dy_sorted), _ptr(dau), _ptr(dx_sorted), _stream(stream)),
        "moe_expert_ffn_backward_input_packed")


def moe_expert_ffn_backward_input(p, offsets, w13, w2, au, dy_sorted, dau, dx_sorted,
                                  stream=None):
    _check(lib().moe_expert_ffn_backward_input(ctypes.byref(p), _ptr(offsets), _ptr(w13),
                                               _ptr(w2), _ptr(au), _ptr(dy_sorted), _ptr(dau),
                                               _ptr(dx_sorted), _stream(stream)),
           "moe_expert_ffn_backward_input")


def moe_expert_ffn_backward_weight(p, x, sorted_token, offsets, h, dy_sorted, dau, dw13, dw2,
                                   stream=None):
    _check(lib().moe_expert_ffn_backward_weight(ctypes.byref(p), _ptr(x), _ptr(sorted_token),
                                                _ptr(offsets), _ptr(h), _ptr(dy_sorted),
                                                _ptr(dau), _ptr(dw13), _ptr(dw2),
                                                _stream(stream)),
           "moe_expert_ffn_backward_weight")


def moe_unpermute_sum(p, dx_sorted, inv_perm, dx_router, dx, stream=None):
    _check(lib().moe_unpermute_sum(ctypes.byref(p), _ptr(dx_sorted), _ptr(inv_perm),
                                   _ptr(dx_router), _ptr(dx), _stream(stream)),
           "moe_unpermute_sum")
