"""Seeded synthetic workloads for the MoE layer.

This module only draws random inputs with the shapes and value distributions of
the layer the pages describe (DeepSeek-V3: hidden width 7168, 256 routed experts
plus one shared expert, top-8, experts in 8 groups of which at most 4 per token;
weights initialised with standard deviation 0.006).  It holds none of the
method's arithmetic, so both the CPU oracle and the HIP path can consume the same
tensors.

Workloads (the configurations the layer is tested and measured on):
  tiny-fp32     T=256,  H=256,  E=16 (4 groups, <=2 per token), K=4, I=128, fp32
  v3-bf16       T=4096, H=7168, E=256 (8 groups, <=4), K=8, I=2048, bf16
  v3-skew-loop  v3-bf16 shapes, T=8192, Zipf(1.2)-ranked logit offsets, 50 steps
  v3-fp8        v3-bf16 shapes with the FP8 E4M3 expert path
  v3-decode     v3-bf16 shapes, T=128
Every workload has one shared expert; the group score sums the top J=2 keys.
"""
from __future__ import annotations

import json
import math
import os
from dataclasses import dataclass, asdict, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    E: int
    G: int
    M: int
    K: int
    J: int
    I: int
    S: int
    act: str          # "f32" | "bf16"  (x, Y and y)
    expert: str       # "f32" | "bf16" | "e4m3"  (GEMM operands)
    bias_init: str    # "zero" | "uniform"  (U(-0.01, 0.01))
    seed_w: int = 0
    seed_x: int = 0
    gamma: float = 0.01
    steps: int = 1
    skew: bool = False

    def as_dict(self):
        return asdict(self)

    @property
    def R(self) -> int:
        return self.T * self.K + self.S * self.T


WORKLOADS = {
    "tiny-fp32": Workload("tiny-fp32", T=256, H=256, E=16, G=4, M=2, K=4, J=2, I=128, S=1,
                          act="f32", expert="f32", bias_init="zero", seed_w=0, seed_x=0),
    "v3-bf16": Workload("v3-bf16", T=4096, H=7168, E=256, G=8, M=4, K=8, J=2, I=2048, S=1,
                        act="bf16", expert="bf16", bias_init="uniform", seed_w=0, seed_x=1),
    "v3-skew-loop": Workload("v3-skew-loop", T=8192, H=7168, E=256, G=8, M=4, K=8, J=2, I=2048,
                             S=1, act="bf16", expert="bf16", bias_init="zero", seed_w=0,
                             seed_x=1000, steps=50, skew=True),
    "v3-fp8": Workload("v3-fp8", T=4096, H=7168, E=256, G=8, M=4, K=8, J=2, I=2048, S=1,
                       act="bf16", expert="e4m3", bias_init="uniform", seed_w=0, seed_x=1),
    "v3-decode": Workload("v3-decode", T=128, H=7168, E=256, G=8, M=4, K=8, J=2, I=2048, S=1,
                          act="bf16", expert="bf16", bias_init="uniform", seed_w=0, seed_x=2),
}

X_STD = 1.0
W_STD = 0.006        # init standard deviation of the pages' model
ROUTER_STD = 0.02
BIAS_HALF_RANGE = 0.01
ZIPF_S = 1.2


def get(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    return replace(w, **overrides) if overrides else w


def _torch():
    import torch
    return torch


def _gen(seed: int, device):
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal(shape, std, dtype, gen, device):
    torch = _torch()
    t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def act_dtype(w: Workload):
    torch = _torch()
    return torch.float32 if w.act == "f32" else torch.bfloat16


def weight_dtype(w: Workload):
    """Storage dtype of the expert weights as generated (e4m3 weights are made from bf16)."""
    torch = _torch()
    return torch.float32 if w.expert == "f32" else torch.bfloat16


def zipf_offsets(w: Workload, alpha: float) -> np.ndarray:
    """Per-expert logit offsets alpha * ln(p_rank) for a seeded random ranking of the
    experts, p_rank proportional to rank^-ZIPF_S (ranks 1..E)."""
    rng = np.random.default_rng(w.seed_w + 77)
    ranks = rng.permutation(w.E) + 1
    p = ranks.astype(np.float64) ** (-ZIPF_S)
    p /= p.sum()
    return (alpha * np.log(p)).astype(np.float32)


def skew_alpha() -> float:
    """Offset scale that gives the top 16 experts about half of all routings at step 0."""
    path = os.path.join(_HERE, "skew_alpha.json")
    with open(path) as f:
        return float(json.load(f)["alpha"])


def make_router(w: Workload, device="cpu"):
    """Router weight [E,H] fp32 and initial bias [E] fp32 (their own seeded streams)."""
    torch = _torch()
    g = _gen(w.seed_w, device)
    w_router = _normal((w.E, w.H), ROUTER_STD, torch.float32, g, device)
    if w.bias_init == "uniform":
        gb = _gen(w.seed_w + 2, device)
        bias = (torch.rand((w.E,), generator=gb, device=device, dtype=torch.float32) * 2 - 1)
        bias.mul_(BIAS_HALF_RANGE)
    else:
        bias = torch.zeros((w.E,), dtype=torch.float32, device=device)
    if w.skew:
        off = torch.from_numpy(zipf_offsets(w, skew_alpha())).to(device)
        w_router[:, 0] = off
    return w_router, bias


def make_experts(w: Workload, device="cpu"):
    """Expert weights w13 [E+S, 2I, H] (gate rows 0..I-1, up rows I..2I-1) and
    w2 [E+S, H, I]; the shared expert is the last slice.  Drawn one expert at a time
    so the full set can be made directly in device memory."""
    torch = _torch()
    g = _gen(w.seed_w + 1, device)
    wd = weight_dtype(w)
    ng = w.E + w.S
    w13 = torch.empty((ng, 2 * w.I, w.H), dtype=wd, device=device)
    w2 = torch.empty((ng, w.H, w.I), dtype=wd, device=device)
    for e in range(ng):
        w13[e] = _normal((2 * w.I, w.H), W_STD, wd, g, device)
        w2[e] = _normal((w.H, w.I), W_STD, wd, g, device)
    return w13, w2


def make_weights(w: Workload, device="cpu"):
    w_router, bias = make_router(w, device)
    w13, w2 = make_experts(w, device)
    return dict(w_router=w_router, w13=w13, w2=w2, bias=bias)


def make_x(w: Workload, step: int = 0, device="cpu", T: int | None = None):
    """Token activations [T,H] ~ N(0,1) in the activation dtype.  With skew, column 0
    is 1 so that the router's first product is exactly the expert's offset."""
    torch = _torch()
    g = _gen(w.seed_x + step, device)
    x = _normal((T or w.T, w.H), X_STD, act_dtype(w), g, device)
    if w.skew:
        x[:, 0] = 1.0
    return x


def make_dy(w: Workload, device="cpu"):
    """Output gradient [T,H] ~ N(0,1) in the activation dtype (its own seeded stream),
    for the backward."""
    g = _gen(w.seed_x + 1_000_003, device)
    return _normal((w.T, w.H), 1.0, act_dtype(w), g, device)


def make_y_sorted(w: Workload, seed: int, device="cpu"):
    """Random expert outputs [R,H] for testing the combine step on its own."""
    torch = _torch()
    g = _gen(seed, device)
    return _normal((w.R, w.H), 0.05, act_dtype(w), g, device)


def to_numpy(t):
    """torch tensor -> numpy, with bf16 given as uint16 bit patterns."""
    torch = _torch()
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.cpu().view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.cpu().view(torch.uint8).numpy()
    return t.cpu().numpy()


def zipf_top16_share(counts: np.ndarray) -> float:
    c = np.sort(np.asarray(counts))[::-1]
    return float(c[:16].sum() / c.sum())
