"""Shared helpers for the GPU parity tests: problem cases, input generation through
the workloads module, comparisons with the oracle."""
from __future__ import annotations

import sys

import numpy as np

import oracle
import workloads

# name -> overrides of a base workload; small enough for the oracle to finish in
# seconds, large enough to span several GEMM tiles with ragged tails.
SMALL_CASES = {
    "tiny-fp32": ("tiny-fp32", {}),
    "tiny-fp32-T1": ("tiny-fp32", dict(T=1)),
    # from 2048 tokens the router logits run on the matrix cores: the fp32-activation
    # form with a ragged last token block and E = 48 (not a multiple of the 64 experts
    # of a workgroup); dense-bf16 and re4-ragged-bf16 below cover the bf16 form
    "mfma-fp32": ("tiny-fp32", dict(T=2100, E=48)),
    "ragged-bf16": ("v3-bf16", dict(T=1000, H=384, E=16, G=4, M=2, K=4, J=2, I=256)),
    # ~150 rows per expert: the grouped GEMMs' three-stage ring with A stages of up to
    # 160 rows (rows rounded up to 16), next to experts just above it
    "rows150-bf16": ("v3-bf16", dict(T=600, H=384, E=16, G=4, M=2, K=4, J=2, I=256)),
    "v3route-bf16": ("v3-bf16", dict(T=513, H=256, I=128)),
    "noshared-bf16": ("v3-bf16", dict(T=300, H=256, E=32, G=4, M=2, K=6, J=2, I=128, S=0)),
    "k1-j1-bf16": ("v3-bf16", dict(T=257, H=128, E=8, G=2, M=1, K=1, J=1, I=128)),
    "allgroups-bf16": ("v3-bf16", dict(T=200, H=256, E=64, G=8, M=8, K=8, J=3, I=128)),
    "maxE-bf16": ("v3-bf16", dict(T=130, H=128, E=512, G=64, M=4, K=16, J=8, I=128)),
    # T >= 2048 with a shared expert: its gate/up GEMM runs as a dense launch (ragged
    # last row tile; dense-fp8 below is the FP8 counterpart)
    "dense-bf16": ("v3-bf16", dict(T=2100, H=384, E=16, G=4, M=2, K=4, J=2, I=384)),
    # a ragged last 64-token block and E = 48 (router logits on the matrix cores, as
    # from 2048 tokens)
    "re4-ragged-bf16": ("v3-bf16", dict(T=3137, H=256, E=48, G=4, M=2, K=4, J=2, I=128)),
    "ragged-fp8": ("v3-fp8", dict(T=700, H=384, E=16, G=4, M=2, K=4, J=2, I=256)),
    "dense-fp8": ("v3-fp8", dict(T=2100, H=384, E=16, G=4, M=2, K=4, J=2, I=256)),
    "v3route-fp8": ("v3-fp8", dict(T=300, H=256, I=256)),
}

TOL = {"f32": 1e-4, "bf16": 2e-2, "e4m3": 1e-2}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def case(name):
    base, over = SMALL_CASES[name]
    return workloads.get(base, **over)


def make_cpu_inputs(w):
    W = workloads.make_weights(w)
    x = workloads.make_x(w)
    return dict(x=x, w_router=W["w_router"], bias=W["bias"], w13=W["w13"], w2=W["w2"])


def rel_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.abs(b).max()
    return float(np.abs(a - b).max() / (den if den > 0 else 1.0))


def as_f64(arr, act):
    """numpy array of act dtype (uint16 bf16 bits or float32) -> float64"""
    if act == "bf16":
        return (arr.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return arr.astype(np.float64)


def shape_of(w):
    from mixture_experts_layer_added_amd.layer import Shape
    return Shape(T=w.T, H=w.H, E=w.E, G=w.G, M=w.M, K=w.K, J=w.J, I=w.I, S=w.S, act=w.act,
                 expert=w.expert)


def token_reference(w, t, xn, wr, z, idx, gate, dyn, w13_of, w2_of):
    """Oracle backward of token t alone (its K expert rows and its shared row): the
    full problem restricted to one token.  w13_of(g), w2_of(g) give expert g's weights."""
    bf = oracle.BF16 if w.act == "bf16" else oracle.F32
    K = w.K
    groups = [int(e) for e in idx[t]] + ([w.E] if w.S else [])
    xt = np.ascontiguousarray(xn[t:t + 1])
    w13 = {g: w13_of(g) for g in groups}
    w2 = {g: w2_of(g) for g in groups}
    ys = np.concatenate([oracle.expert_ffn(xt, w13[g], w2[g], bf, nthreads=1) for g in groups])
    inv1 = np.arange(K, dtype=np.int32)[None, :]
    dys, dg = oracle.combine_backward(dyn[t:t + 1], ys, inv1, gate[t:t + 1], w.S, nthreads=1)
    dz, dxr, _ = oracle.router_backward(xt, wr, z[t:t + 1], idx[t:t + 1], gate[t:t + 1], dg,
                                        nthreads=1)
    dxs = np.empty((len(groups), w.H), xt.dtype)
    dau = np.empty((len(groups), 2 * w.I), xt.dtype)
    for i, g in enumerate(groups):
        _, dau[i:i + 1], dxs[i:i + 1], _, _ = oracle.expert_backward(xt, w13[g], w2[g],
                                                                     dys[i:i + 1], nthreads=1)
    dx = oracle.unpermute_sum(dxs, inv1, dxr, 1, w.S, nthreads=1)
    return dict(dgate=dg[0], dz=dz[0], dy_sorted=dys, dau=dau, dx=dx[0])


def slice_reference(w, g, n, xn, tokens, gates, dyn, w13_of, w2_of):
    """Oracle dW2[g][:, n], dW13[g][n, :], dW13[g][I+n, :] and [da|du][:, (n, I+n)] from
    the rows of expert g (tokens, their gates) with the weights cut to column n."""
    I = w.I
    w13 = w13_of(g)
    w13s = np.ascontiguousarray(w13[[n, I + n], :])
    w2s = np.ascontiguousarray(w2_of(g)[:, n:n + 1])
    m = len(tokens)
    inv1 = np.arange(m, dtype=np.int32)[:, None]
    dys, _ = oracle.combine_backward(np.ascontiguousarray(dyn[tokens]),
                                     np.zeros((m, w.H), dyn.dtype), inv1,
                                     np.ascontiguousarray(gates[:, None], np.float32), 0)
    _, dau, _, dw13s, dw2s = oracle.expert_backward(np.ascontiguousarray(xn[tokens]), w13s, w2s,
                                                    dys)
    return dict(dw2=dw2s[:, 0], dw13_a=dw13s[0], dw13_u=dw13s[1], dau=dau)
