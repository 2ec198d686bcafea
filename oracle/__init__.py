"""CPU oracle of the DeepSeekMoE layer forward with aux-loss-free balancing.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg of
the benchmark may import this package; the product path never does.  It wraps
``moe_oracle.c`` (plain C, built with gcc) through ctypes on numpy buffers and
composes the per-call routines into a whole-layer forward.  It shares no code
with the HIP library.

Dtype codes: 0 = float32, 1 = bfloat16 (stored as uint16 bit patterns),
2 = FP8 E4M3 (OCP "fn", stored as uint8 codes).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

F32, BF16, E4M3 = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")
_lib = None


def build() -> str:
    """Compile the oracle with gcc (no fast-math, no fp contraction)."""
    cmd = ["gcc", "-O2", "-std=gnu11", "-ffp-contract=off", "-fno-fast-math", "-mfma",
           "-fPIC", "-shared", "-pthread", "-Wall", "-Wno-unused-function",
           _SRC, "-o", _LIB_PATH + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        _lib = _declare(ctypes.CDLL(_LIB_PATH))
    return _lib


def _declare(L):
    c = ctypes
    vp, i64, i32, f32 = c.c_void_p, c.c_int64, c.c_int, c.c_float
    L.oracle_bf16_to_f32.argtypes = [c.c_uint16]; L.oracle_bf16_to_f32.restype = f32
    L.oracle_bf16_from_f64.argtypes = [c.c_double]; L.oracle_bf16_from_f64.restype = c.c_uint16
    L.oracle_f32_from_f64.argtypes = [c.c_double]; L.oracle_f32_from_f64.restype = f32
    L.oracle_e4m3_to_f32.argtypes = [c.c_uint8]; L.oracle_e4m3_to_f32.restype = f32
    L.oracle_e4m3_from_f32.argtypes = [f32]; L.oracle_e4m3_from_f32.restype = c.c_uint8
    L.oracle_exp_spec.argtypes = [f32]; L.oracle_exp_spec.restype = f32
    L.oracle_sigmoid.argtypes = [f32]; L.oracle_sigmoid.restype = f32
    L.oracle_router_logits.argtypes = [i64, i32, i32, i32, vp, vp, vp, i32]
    L.oracle_router_logits.restype = None
    L.oracle_select.argtypes = [i64, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, i32]
    L.oracle_select.restype = None
    L.oracle_count.argtypes = [i64, i32, i32, vp, vp]; L.oracle_count.restype = None
    L.oracle_route.argtypes = [i64, i32, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp,
                               vp, vp, i32]
    L.oracle_route.restype = i32
    L.oracle_quantize_act_fp8.argtypes = [i64, i32, i32, vp, vp, vp]
    L.oracle_quantize_act_fp8.restype = None
    L.oracle_quantize_weight_fp8.argtypes = [i32, i32, vp, vp, vp]
    L.oracle_quantize_weight_fp8.restype = None
    L.oracle_permute.argtypes = [i64, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, i32,
                                 vp, vp]
    L.oracle_permute.restype = i32
    L.oracle_expert_ffn.argtypes = [i64, i32, i32, i32, vp, vp, vp, vp, vp, vp, i32, vp, i32]
    L.oracle_expert_ffn_h.argtypes = [i64, i32, i32, i32, vp, vp, vp, vp, vp, vp, i32, vp, vp,
                                      vp, i32]
    L.oracle_expert_ffn_h.restype = i32
    L.oracle_expert_ffn.restype = i32
    L.oracle_combine.argtypes = [i64, i32, i32, i32, i32, vp, vp, vp, vp, i32]
    L.oracle_combine.restype = None
    L.oracle_bias_update.argtypes = [i32, i64, i32, vp, f32, vp]
    L.oracle_seq_load_stats.argtypes = [i64, i32, i32, vp, i32, vp, vp, vp, vp]
    L.oracle_seq_load_stats.restype = None
    L.oracle_bias_update.restype = None
    L.oracle_combine_backward.argtypes = [i64, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, i32]
    L.oracle_combine_backward.restype = None
    L.oracle_router_backward.argtypes = [i64, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp,
                                         vp, vp, i32]
    L.oracle_router_backward.restype = i32
    L.oracle_expert_backward.argtypes = [i64, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp,
                                         vp, i32]
    L.oracle_expert_backward.restype = i32
    L.oracle_unpermute_sum.argtypes = [i64, i32, i32, i32, i32, vp, vp, vp, vp, i32]
    L.oracle_unpermute_sum.restype = None
    for n in ("oracle_exp_spec_array", "oracle_sigmoid_array", "oracle_e4m3_from_f32_array",
              "oracle_bf16_from_f64_array"):
        getattr(L, n).argtypes = [i64, vp, vp]
        getattr(L, n).restype = None
    return L


def default_threads() -> int:
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        return max(1, min(16, os.cpu_count() or 1))


def _p(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    assert a.dtype == dtype, (a.dtype, dtype)
    return a


def act_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.uint8:
        return E4M3
    raise TypeError(f"unsupported dtype {a.dtype}")


# --- scalar formats -----------------------------------------------------------

def exp_spec(a: float) -> float:
    return lib().oracle_exp_spec(a)


def sigmoid(z: float) -> float:
    return lib().oracle_sigmoid(z)


def exp_spec_array(a):
    a = _c(a, np.float32)
    out = np.empty_like(a)
    lib().oracle_exp_spec_array(a.size, _p(a), _p(out))
    return out


def sigmoid_array(z):
    z = _c(z, np.float32)
    out = np.empty_like(z)
    lib().oracle_sigmoid_array(z.size, _p(z), _p(out))
    return out


def e4m3_from_f32_array(v):
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().oracle_e4m3_from_f32_array(v.size, _p(v), _p(out))
    return out


def bf16_from_f64_array(v):
    v = _c(np.asarray(v, dtype=np.float64), np.float64)
    out = np.empty(v.shape, np.uint16)
    lib().oracle_bf16_from_f64_array(v.size, _p(v), _p(out))
    return out


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_from_f64(v: float) -> int:
    return lib().oracle_bf16_from_f64(v)


def e4m3_to_f32(c: int) -> float:
    return lib().oracle_e4m3_to_f32(c)


def e4m3_from_f32(v: float) -> int:
    return lib().oracle_e4m3_from_f32(v)


# --- per-call routines --------------------------------------------------------

def router_logits(x, w_router, nthreads=None):
    T, H = x.shape
    E = w_router.shape[0]
    w_router = _c(w_router, np.float32)
    x = np.ascontiguousarray(x)
    z = np.empty((T, E), np.float32)
    lib().oracle_router_logits(T, H, E, act_code(x), _p(x), _p(w_router), _p(z),
                               nthreads or default_threads())
    return z


def select(z, bias, G, M, K, J, nthreads=None):
    z = _c(z, np.float32)
    bias = _c(bias, np.float32)
    T, E = z.shape
    idx = np.empty((T, K), np.int32)
    gate = np.empty((T, K), np.float32)
    counts = np.empty(E, np.int32)
    lib().oracle_select(T, E, G, M, K, J, _p(z), _p(bias), _p(idx), _p(gate), _p(counts),
                        nthreads or default_threads())
    return idx, gate, counts


def route(x, w_router, bias, G, M, K, J, nthreads=None, want_logits=False):
    """Returns (topk_idx [T,K] int32, topk_gate [T,K] f32, counts [E] int32, logits|None)."""
    x = np.ascontiguousarray(x)
    w_router = _c(w_router, np.float32)
    bias = _c(bias, np.float32)
    T, H = x.shape
    E = w_router.shape[0]
    idx = np.empty((T, K), np.int32)
    gate = np.empty((T, K), np.float32)
    counts = np.empty(E, np.int32)
    z = np.empty((T, E), np.float32) if want_logits else None
    rc = lib().oracle_route(T, H, E, G, M, K, J, act_code(x), _p(x), _p(w_router), _p(bias),
                            _p(idx), _p(gate), _p(counts), _p(z), nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle_route rejected the problem (code {rc})")
    return idx, gate, counts, z


def count(topk_idx, E):
    topk_idx = _c(topk_idx, np.int32)
    T, K = topk_idx.shape
    c = np.empty(E, np.int32)
    lib().oracle_count(T, E, K, _p(topk_idx), _p(c))
    return c


def quantize_act_fp8(a):
    a = np.ascontiguousarray(a)
    rows, cols = a.shape
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((rows, cols // 128), np.float32)
    lib().oracle_quantize_act_fp8(rows, cols, act_code(a), _p(a), _p(q), _p(s))
    return q, s


def quantize_weight_fp8(w):
    """w: [rows, cols] bf16 bits (uint16) -> (codes uint8 [rows, cols], scales [rows/128, cols/128])."""
    w = _c(w, np.uint16)
    rows, cols = w.shape
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((rows // 128, cols // 128), np.float32)
    lib().oracle_quantize_weight_fp8(rows, cols, _p(w), _p(q), _p(s))
    return q, s


def permute(x, topk_idx, counts, E, shared=1, out_dtype=None):
    """Returns (offsets [E+1+S], sorted_token [R], inv_perm [T,K], x_sorted, x_sorted_scale|None)."""
    x = np.ascontiguousarray(x)
    topk_idx = _c(topk_idx, np.int32)
    counts = _c(counts, np.int32)
    T, H = x.shape
    K = topk_idx.shape[1]
    S = 1 if shared else 0
    R = T * K + S * T
    xd = act_code(x)
    od = xd if out_dtype is None else out_dtype
    offsets = np.empty(E + 1 + S, np.int32)
    sorted_token = np.empty(R, np.int32)
    inv_perm = np.empty((T, K), np.int32)
    if od == E4M3:
        xs = np.empty((R, H), np.uint8)
        xsc = np.empty((R, H // 128), np.float32)
    else:
        xs = np.empty((R, H), x.dtype)
        xsc = None
    rc = lib().oracle_permute(T, H, E, K, S, xd, _p(x), _p(topk_idx), _p(counts), _p(offsets),
                              _p(sorted_token), _p(inv_perm), od, _p(xs), _p(xsc))
    if rc != 0:
        raise ValueError(f"oracle_permute rejected the input (code {rc})")
    return offsets, sorted_token, inv_perm, xs, xsc


def expert_ffn(x_rows, w13, w2, out_dtype, x_scale=None, w13_scale=None, w2_scale=None,
               nthreads=None, want_h=False):
    """One expert on a block of rows.  x_rows [n,H]; w13 [2I,H]; w2 [H,I].  Returns y,
    or with want_h (y, h, h_scale): h [n,I] as stored between the GEMMs (E4M3 codes and
    h_scale [n,I/128] for the FP8 path, else h_scale None)."""
    x_rows = np.ascontiguousarray(x_rows)
    w13 = np.ascontiguousarray(w13)
    w2 = np.ascontiguousarray(w2)
    n, H = x_rows.shape
    I = w2.shape[1]
    dt = act_code(x_rows)
    assert act_code(w13) == dt and act_code(w2) == dt
    y = np.empty((n, H), np.uint16 if out_dtype == BF16 else np.float32)
    if dt == E4M3:
        x_scale = _c(x_scale, np.float32)
        w13_scale = _c(w13_scale, np.float32)
        w2_scale = _c(w2_scale, np.float32)
    if not want_h:
        rc = lib().oracle_expert_ffn(n, H, I, dt, _p(x_rows), _p(x_scale), _p(w13),
                                     _p(w13_scale), _p(w2), _p(w2_scale), out_dtype, _p(y),
                                     nthreads or default_threads())
        if rc != 0:
            raise ValueError(f"oracle_expert_ffn rejected the input (code {rc})")
        return y
    h = np.empty((n, I), x_rows.dtype)
    h_scale = np.empty((n, I // 128), np.float32) if dt == E4M3 else None
    rc = lib().oracle_expert_ffn_h(n, H, I, dt, _p(x_rows), _p(x_scale), _p(w13),
                                   _p(w13_scale), _p(w2), _p(w2_scale), out_dtype, _p(y), _p(h),
                                   _p(h_scale), nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle_expert_ffn_h rejected the input (code {rc})")
    return y, h, h_scale


def combine(y_sorted, inv_perm, topk_gate, T, shared=1, nthreads=None):
    y_sorted = np.ascontiguousarray(y_sorted)
    inv_perm = _c(inv_perm, np.int32)
    topk_gate = _c(topk_gate, np.float32)
    H = y_sorted.shape[1]
    K = inv_perm.shape[1]
    y = np.empty((T, H), y_sorted.dtype)
    lib().oracle_combine(T, H, K, 1 if shared else 0, act_code(y_sorted), _p(y_sorted),
                         _p(inv_perm), _p(topk_gate), _p(y), nthreads or default_threads())
    return y


def bias_update(counts, T, K, gamma, bias):
    """Returns the updated bias (a new array)."""
    counts = _c(counts, np.int32)
    b = np.array(bias, dtype=np.float32, copy=True)
    lib().oracle_bias_update(len(counts), T, K, _p(counts), np.float32(gamma), _p(b))
    return b


# --- whole-layer composition ---------------------------------------------------

def seq_load_stats(topk_idx, E, seq_offsets):
    """Sequence-wise loads (mpbf.cn section 2.2, the sequence-level balance term; the
    pages give it no formula, so only its loads are computed).  Sequence s is tokens
    seq_offsets[s] .. seq_offsets[s+1]-1.  Returns counts [n_seq, E] int32 (chosen
    indices per sequence and expert), stats [n_seq, 3] int32 (max count, min count,
    experts with no token) and ratio [n_seq] fp32 = max / (L*K/E), 0 for an empty
    sequence."""
    idx = _c(topk_idx, np.int32)
    off = _c(np.asarray(seq_offsets, dtype=np.int32), np.int32)
    T, K = idx.shape
    n = len(off) - 1
    assert n >= 1 and off[0] == 0 and off[-1] == T and np.all(np.diff(off) >= 0)
    assert idx.min() >= 0 and idx.max() < E
    counts = np.empty((n, E), np.int32)
    stats = np.empty((n, 3), np.int32)
    ratio = np.empty((n,), np.float32)
    lib().oracle_seq_load_stats(T, E, K, _p(idx), n, _p(off), _p(counts), _p(stats), _p(ratio))
    return counts, stats, ratio


def forward(x, w_router, bias, w13, w2, G, M, K, J, shared=1, expert_dtype=None,
            w13_q=None, w13_s=None, w2_q=None, w2_s=None, nthreads=None):
    """Full layer forward: route -> permute -> per-expert FFN -> combine.

    x [T,H] (f32 or bf16 bits); w13 [E+S, 2I, H]; w2 [E+S, H, I] in the activation
    dtype.  With expert_dtype == E4M3 the expert operands are the given codes and
    block scales (w13_q/w13_s/w2_q/w2_s) and the output is bf16.
    Returns a dict with every intermediate.
    """
    T, H = x.shape
    E = w_router.shape[0]
    idx, gate, counts, _ = route(x, w_router, bias, G, M, K, J, nthreads)
    ad = act_code(x)
    ed = ad if expert_dtype is None else expert_dtype
    offsets, sorted_token, inv_perm, xs, xsc = permute(x, idx, counts, E, shared, out_dtype=ed)
    out_dtype = ad
    R = xs.shape[0]
    ys = np.empty((R, H), np.uint16 if out_dtype == BF16 else np.float32)
    for g in range(E + (1 if shared else 0)):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        if hi == lo:
            continue
        if ed == E4M3:
            ys[lo:hi] = expert_ffn(xs[lo:hi], w13_q[g], w2_q[g], out_dtype, xsc[lo:hi], w13_s[g],
                                   w2_s[g], nthreads)
        else:
            ys[lo:hi] = expert_ffn(xs[lo:hi], w13[g], w2[g], out_dtype, nthreads=nthreads)
    y = combine(ys, inv_perm, gate, T, shared, nthreads)
    return dict(topk_idx=idx, topk_gate=gate, counts=counts, offsets=offsets,
                sorted_token=sorted_token, inv_perm=inv_perm, x_sorted=xs,
                x_sorted_scale=xsc, y_sorted=ys, y=y)


# --- backward (the derivative of the forward; see moe_oracle.c) ----------------

def combine_backward(dy, y_sorted, inv_perm, topk_gate, shared=1, nthreads=None):
    """Returns (dY_sorted [R,H] act dtype, dgate [T,K] f32)."""
    dy = np.ascontiguousarray(dy)
    y_sorted = np.ascontiguousarray(y_sorted)
    inv_perm = _c(inv_perm, np.int32)
    topk_gate = _c(topk_gate, np.float32)
    T, H = dy.shape
    K = inv_perm.shape[1]
    dys = np.zeros_like(y_sorted)
    dg = np.empty((T, K), np.float32)
    lib().oracle_combine_backward(T, H, K, 1 if shared else 0, act_code(dy), _p(dy),
                                  _p(y_sorted), _p(inv_perm), _p(topk_gate), _p(dys), _p(dg),
                                  nthreads or default_threads())
    return dys, dg


def router_backward(x, w_router, logits, topk_idx, topk_gate, dgate, nthreads=None):
    """Returns (dz [T,K] f32, dx_router [T,H] f32, dw_router [E,H] f32)."""
    x = np.ascontiguousarray(x)
    w_router = _c(w_router, np.float32)
    logits = _c(logits, np.float32)
    topk_idx = _c(topk_idx, np.int32)
    topk_gate = _c(topk_gate, np.float32)
    dgate = _c(dgate, np.float32)
    T, H = x.shape
    E = w_router.shape[0]
    K = topk_idx.shape[1]
    dz = np.empty((T, K), np.float32)
    dxr = np.empty((T, H), np.float32)
    dwr = np.empty((E, H), np.float32)
    rc = lib().oracle_router_backward(T, H, E, K, act_code(x), _p(x), _p(w_router), _p(logits),
                                      _p(topk_idx), _p(topk_gate), _p(dgate), _p(dz), _p(dxr),
                                      _p(dwr), nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_router_backward rejected the input")
    return dz, dxr, dwr


def expert_backward(x_rows, w13, w2, dy_rows, nthreads=None, weights=True):
    """One expert on a block of rows.  Returns (h, dau, dx_rows, dw13 f32, dw2 f32);
    weights=False computes the input part only (dw13, dw2 are then None)."""
    x_rows = np.ascontiguousarray(x_rows)
    w13 = np.ascontiguousarray(w13)
    w2 = np.ascontiguousarray(w2)
    dy_rows = np.ascontiguousarray(dy_rows)
    n, H = x_rows.shape
    I = w2.shape[1]
    dt = act_code(x_rows)
    h = np.empty((n, I), x_rows.dtype)
    dau = np.empty((n, 2 * I), x_rows.dtype)
    dx = np.empty((n, H), x_rows.dtype)
    dw13 = np.empty((2 * I, H), np.float32) if weights else None
    dw2 = np.empty((H, I), np.float32) if weights else None
    rc = lib().oracle_expert_backward(n, H, I, dt, _p(x_rows), _p(w13), _p(w2), _p(dy_rows),
                                      _p(h), _p(dau), _p(dx), _p(dw13), _p(dw2),
                                      nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_expert_backward rejected the input")
    return h, dau, dx, dw13, dw2


def unpermute_sum(dx_sorted, inv_perm, dx_router, T, shared=1, nthreads=None):
    dx_sorted = np.ascontiguousarray(dx_sorted)
    inv_perm = _c(inv_perm, np.int32)
    H = dx_sorted.shape[1]
    K = inv_perm.shape[1]
    dxr = None if dx_router is None else _c(dx_router, np.float32)
    dx = np.empty((T, H), dx_sorted.dtype)
    lib().oracle_unpermute_sum(T, H, K, 1 if shared else 0, act_code(dx_sorted), _p(dx_sorted),
                               _p(inv_perm), _p(dxr), _p(dx), nthreads or default_threads())
    return dx


def backward(x, w_router, w13, w2, fwd, dy, logits, shared=1, nthreads=None):
    """Whole-layer backward from the forward's intermediates (the dict forward() returns)
    and the output gradient dy [T,H] (act dtype).  logits [T,E] f32 are the router
    logits of the forward.  Returns a dict: dx [T,H] act, dw_router [E,H] f32,
    dw13 [E+S,2I,H] f32, dw2 [E+S,H,I] f32 and the intermediates."""
    T, H = x.shape
    E = w_router.shape[0]
    S = 1 if shared else 0
    I = w2.shape[2]
    off = fwd["offsets"]
    dys, dg = combine_backward(dy, fwd["y_sorted"], fwd["inv_perm"], fwd["topk_gate"], shared,
                               nthreads)
    dz, dxr, dwr = router_backward(x, w_router, logits, fwd["topk_idx"], fwd["topk_gate"], dg,
                                   nthreads)
    xs = fwd["x_sorted"]
    R = xs.shape[0]
    dxs = np.zeros((R, H), xs.dtype)
    dau = np.zeros((R, 2 * I), xs.dtype)
    dw13 = np.zeros((E + S, 2 * I, H), np.float32)
    dw2 = np.zeros((E + S, H, I), np.float32)
    for g in range(E + S):
        lo, hi = int(off[g]), int(off[g + 1])
        if hi == lo:
            continue
        _, dau[lo:hi], dxs[lo:hi], dw13[g], dw2[g] = expert_backward(xs[lo:hi], w13[g], w2[g],
                                                                     dys[lo:hi], nthreads)
    dx = unpermute_sum(dxs, fwd["inv_perm"], dxr, T, shared, nthreads)
    return dict(dx=dx, dw_router=dwr, dw13=dw13, dw2=dw2, dy_sorted=dys, dgate=dg, dz=dz,
                dx_router=dxr, dau=dau, dx_sorted=dxs)
