"""GPU parity of the layer backward (bf16 and fp32 paths) against the CPU oracle.

The oracle runs its own forward and backward on the same seeded inputs (no value
comes from the GPU); the GPU layer runs forward (keeping the gate/up pre-activations)
and backward.  Routing and the permutation are bit-exact (forward parity); gradients
are compared normwise: max |gpu - oracle| / max |oracle| within 1e-4 (fp32) or 2e-2
(bf16) for dgate, dz, dx, dw_router, dw13 and dw2.  Experts that received no tokens
must get exactly zero weight gradients.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_cases import TOL, as_f64, case, log, make_cpu_inputs, rel_err, shape_of

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

CASES = ["tiny-fp32", "tiny-fp32-T1", "ragged-bf16", "v3route-bf16", "noshared-bf16",
         "k1-j1-bf16", "maxE-bf16", "dense-bf16", "rows150-bf16"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mixture_experts_layer_added_amd import _lib
    _lib.lib()


def np_(t):
    return workloads.to_numpy(t)


def to_dev(t):
    return t.contiguous().cuda()


def vals(a, act):
    return as_f64(a, act) if a.dtype == np.uint16 else a.astype(np.float64)


@pytest.mark.parametrize("gather", [False, True])
@pytest.mark.parametrize("name", CASES)
def test_backward_matches_oracle(name, gather):
    from mixture_experts_layer_added_amd.layer import MoELayer
    log(f"[backward] {name} gather={gather}")
    w = case(name)
    inp = make_cpu_inputs(w)
    dyt = workloads.make_dy(w)
    dy = np_(dyt)
    xn, wr, bn = np_(inp["x"]), np_(inp["w_router"]), np_(inp["bias"])
    w13, w2 = np_(inp["w13"]), np_(inp["w2"])
    ref = oracle.forward(xn, wr, bn, w13, w2, w.G, w.M, w.K, w.J, shared=w.S)
    _, _, _, z = oracle.route(xn, wr, bn, w.G, w.M, w.K, w.J, want_logits=True)
    rb = oracle.backward(xn, wr, w13, w2, ref, dy, z, shared=w.S)

    layer = MoELayer(shape_of(w), to_dev(inp["w_router"]), to_dev(inp["bias"]),
                     to_dev(inp["w13"]), to_dev(inp["w2"]), gather=gather, train=True)
    x = to_dev(inp["x"])
    layer.forward(x)
    layer.backward(dyt.cuda())
    torch.cuda.synchronize()
    for k in ("topk_idx", "counts", "offsets", "sorted_token", "inv_perm"):
        assert np.array_equal(np_(getattr(layer, k)), ref[k]), k
    tol = TOL[w.expert]
    # keeping the pre-activations leaves the forward unchanged
    assert rel_err(vals(np_(layer.y), w.act), vals(ref["y"], w.act)) <= tol
    errs = {}
    for k, ok in (("dy_sorted", "dy_sorted"), ("dgate", "dgate"), ("dz", "dz"), ("dx", "dx"), ("dw_router", "dw_router"),
                  ("dw13", "dw13"), ("dw2", "dw2")):
        g, r = np_(getattr(layer, k)), rb[ok]
        errs[k] = rel_err(vals(g, w.act), vals(r, w.act))
    log("    " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()) + f" (bound {tol})")
    for k, v in errs.items():
        assert v <= tol, k
    # experts without tokens: exactly zero weight gradients
    empty = np.nonzero(ref["counts"] == 0)[0]
    if len(empty):
        assert not np.any(np_(layer.dw13)[empty]) and not np.any(np_(layer.dw2)[empty])
