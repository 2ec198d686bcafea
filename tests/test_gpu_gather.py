"""GPU parity of the gathered dispatch: the permute writes only the index maps (FP8:
plus one quantisation of x per token) and the gate/up GEMM reads its rows from x
through sorted_token.  Checked against the CPU oracle on the same seeded inputs
(routing, index maps and the per-token FP8 codes bit for bit; expert and combined
outputs within the per-dtype bound), and against the path that materialises x_sorted
(h, Y and y bit for bit: the two paths feed identical operands to identical kernels).
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_cases import SMALL_CASES, TOL, as_f64, case, log, make_cpu_inputs, rel_err, shape_of

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


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


def layers(w, inp):
    """(materialising layer, gathering layer) sharing the same device weights"""
    from mixture_experts_layer_added_amd.layer import MoELayer, quantize_weights_fp8
    wr, b = to_dev(inp["w_router"]), to_dev(inp["bias"])
    w13, w2 = to_dev(inp["w13"]), to_dev(inp["w2"])
    s13 = s2 = None
    if w.expert == "e4m3":
        w13, s13 = quantize_weights_fp8(w13)
        w2, s2 = quantize_weights_fp8(w2)
    return (MoELayer(shape_of(w), wr, b, w13, w2, s13, s2),
            MoELayer(shape_of(w), wr, b, w13, w2, s13, s2, gather=True))


@pytest.mark.parametrize("name", sorted(SMALL_CASES))
def test_gather_forward(name):
    log(f"[gather] {name}")
    w = case(name)
    inp = make_cpu_inputs(w)
    fp8 = w.expert == "e4m3"
    mat, gat = layers(w, inp)
    x = to_dev(inp["x"])
    mat.forward(x)
    gat.forward(x)
    torch.cuda.synchronize()
    # against the oracle
    xn = np_(inp["x"])
    idx, gate, counts, _ = oracle.route(xn, np_(inp["w_router"]), np_(inp["bias"]), w.G, w.M,
                                        w.K, w.J)
    off, st, inv, xs, xsc = oracle.permute(xn, idx, counts, w.E, w.S,
                                           out_dtype=oracle.E4M3 if fp8 else None)
    assert np.array_equal(np_(gat.topk_idx), idx)
    assert np.array_equal(np_(gat.offsets), off)
    assert np.array_equal(np_(gat.sorted_token), st)
    assert np.array_equal(np_(gat.inv_perm), inv)
    if fp8:
        q, s = oracle.quantize_act_fp8(xn)
        assert np.array_equal(np_(gat.x_q), q)
        assert np.array_equal(np_(gat.x_scale).view(np.uint32), s.view(np.uint32))
    # identical to the materialising path
    for k in ("h", "y_sorted", "y"):
        assert np.array_equal(np_(getattr(gat, k)).view(np.uint8),
                              np_(getattr(mat, k)).view(np.uint8)), k
    if fp8:
        assert np.array_equal(np_(gat.h_scale).view(np.uint32), np_(mat.h_scale).view(np.uint32))
    # expert outputs and combined output against the oracle
    out_dt = oracle.BF16 if w.act == "bf16" else oracle.F32
    ys = np.zeros((w.R, w.H), np.uint16 if w.act == "bf16" else np.float32)
    for g in range(w.E + w.S):
        rows = np.arange(off[g], off[g + 1])
        if len(rows) == 0:
            continue
        if fp8:
            a, sa = oracle.quantize_weight_fp8(np_(inp["w13"][g]))
            b, sb = oracle.quantize_weight_fp8(np_(inp["w2"][g]))
            ys[rows] = oracle.expert_ffn(xs[rows], a, b, out_dt, xsc[rows], sa, sb)
        else:
            ys[rows] = oracle.expert_ffn(xs[rows], np_(inp["w13"][g]), np_(inp["w2"][g]), out_dt)
    y_ref = oracle.combine(ys, inv, gate, w.T, w.S)
    ys_ref = as_f64(ys, w.act)
    e1 = rel_err(as_f64(np_(gat.y_sorted), w.act), ys_ref)
    e2 = float(np.abs(as_f64(np_(gat.y), w.act) - as_f64(y_ref, w.act)).max()
               / (2 * np.abs(ys_ref).max()))
    log(f"    y_sorted rel err {e1:.3e}, y err / (2 max|Y|) {e2:.3e} (bound {TOL[w.expert]})")
    assert e1 <= TOL[w.expert] and e2 <= TOL[w.expert]
