"""Shared helpers for the GPU parity tests: problem cases, input generation through
the workloads module, comparisons with the oracle."""
from __future__ import annotations

import sys

import numpy as np

import workloads

# name -> overrides of a base workload; small enough for the oracle to finish in
# seconds, large enough to span several GEMM tiles with ragged tails.
SMALL_CASES = {
    "tiny-fp32": ("tiny-fp32", {}),
    "tiny-fp32-T1": ("tiny-fp32", dict(T=1)),
    "ragged-bf16": ("v3-bf16", dict(T=1000, H=384, E=16, G=4, M=2, K=4, J=2, I=256)),
    "v3route-bf16": ("v3-bf16", dict(T=513, H=256, I=128)),
    "noshared-bf16": ("v3-bf16", dict(T=300, H=256, E=32, G=4, M=2, K=6, J=2, I=128, S=0)),
    "k1-j1-bf16": ("v3-bf16", dict(T=257, H=128, E=8, G=2, M=1, K=1, J=1, I=128)),
    "allgroups-bf16": ("v3-bf16", dict(T=200, H=256, E=64, G=8, M=8, K=8, J=3, I=128)),
    "maxE-bf16": ("v3-bf16", dict(T=130, H=128, E=512, G=64, M=4, K=16, J=8, I=128)),
    "ragged-fp8": ("v3-fp8", dict(T=700, H=384, E=16, G=4, M=2, K=4, J=2, I=256)),
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
