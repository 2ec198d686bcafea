"""GPU parity: every C-ABI call against the CPU oracle on identical seeded inputs.

Routing indices, gates, counts, logits, the permutation, the combine and the bias
update must match bit for bit; expert outputs within the per-dtype bound
(max |gpu - oracle| / max |oracle| <= 1e-4 fp32, 2e-2 bf16, 1e-2 fp8).
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


def from_np(a):
    """numpy -> torch with bf16 bit patterns (uint16) viewed as bfloat16"""
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(a)


def run_oracle_route(w, inp):
    return oracle.route(np_(inp["x"]), np_(inp["w_router"]), np_(inp["bias"]), w.G, w.M, w.K, w.J,
                        want_logits=True)


def gpu_layer(w, inp, w13=None, w2=None, s13=None, s2=None, packed=None):
    from mixture_experts_layer_added_amd.layer import MoELayer
    return MoELayer(shape_of(w), to_dev(inp["w_router"]), to_dev(inp["bias"]),
                    to_dev(inp["w13"]) if w13 is None else w13,
                    to_dev(inp["w2"]) if w2 is None else w2, s13, s2, packed=packed)


def fp8_weights(inp):
    q13, s13, q2, s2 = [], [], [], []
    for e in range(inp["w13"].shape[0]):
        a, b = oracle.quantize_weight_fp8(np_(inp["w13"][e]))
        q13.append(a), s13.append(b)
        a, b = oracle.quantize_weight_fp8(np_(inp["w2"][e]))
        q2.append(a), s2.append(b)
    return np.stack(q13), np.stack(s13), np.stack(q2), np.stack(s2)


CASES = sorted(SMALL_CASES)


@pytest.mark.parametrize("name", CASES)
def test_route_bitexact(name):
    log(f"[route] {name}")
    w = case(name)
    inp = make_cpu_inputs(w)
    idx, gate, counts, z = run_oracle_route(w, inp)
    layer = gpu_layer(w, inp)
    layer.route(to_dev(inp["x"]))
    torch.cuda.synchronize()
    assert np.array_equal(np_(layer.logits).view(np.uint32), z.view(np.uint32))
    assert np.array_equal(np_(layer.topk_idx), idx)
    assert np.array_equal(np_(layer.topk_gate).view(np.uint32), gate.view(np.uint32))
    assert np.array_equal(np_(layer.counts), counts)


@pytest.mark.parametrize("name", CASES)
def test_permute_bitexact(name):
    log(f"[permute] {name}")
    w = case(name)
    inp = make_cpu_inputs(w)
    idx, gate, counts, _ = run_oracle_route(w, inp)
    ed = oracle.E4M3 if w.expert == "e4m3" else None
    off, st, inv, xs, xsc = oracle.permute(np_(inp["x"]), idx, counts, w.E, w.S, out_dtype=ed)
    layer = gpu_layer(w, inp)
    layer.topk_idx.copy_(torch.from_numpy(idx))
    layer.permute(to_dev(inp["x"]))
    torch.cuda.synchronize()
    assert np.array_equal(np_(layer.offsets), off)
    assert np.array_equal(np_(layer.sorted_token), st)
    assert np.array_equal(np_(layer.inv_perm), inv)
    assert np.array_equal(np_(layer.x_sorted).view(np.uint8), xs.view(np.uint8))
    if xsc is not None:
        assert np.array_equal(np_(layer.x_scale).view(np.uint32), xsc.view(np.uint32))


@pytest.mark.parametrize("name", ["ragged-fp8", "v3route-fp8"])
def test_quantize_weights_bitexact(name):
    log(f"[quantize weights] {name}")
    w = case(name)
    inp = make_cpu_inputs(w)
    from mixture_experts_layer_added_amd.layer import quantize_weights_fp8
    q13, s13 = quantize_weights_fp8(to_dev(inp["w13"]))
    q2, s2 = quantize_weights_fp8(to_dev(inp["w2"]))
    torch.cuda.synchronize()
    o13, os13, o2, os2 = fp8_weights(inp)
    assert np.array_equal(np_(q13), o13) and np.array_equal(np_(s13).view(np.uint32), os13.view(np.uint32))
    assert np.array_equal(np_(q2), o2) and np.array_equal(np_(s2).view(np.uint32), os2.view(np.uint32))


FFN_CASES = ([(n, None) for n in CASES if n.endswith("-fp32") or "fp32-" in n] +
             [(n, pk) for n in CASES if n.endswith("-bf16") or n.endswith("-fp8")
              for pk in (True, False)])


@pytest.mark.parametrize("name,packed", FFN_CASES)
def test_expert_ffn_tolerance(name, packed):
    """bf16 and FP8 cases run twice: over packed weights and over the natural layout
    (the LDS-ring kernels)."""
    log(f"[expert_ffn] {name} packed={packed}")
    w = case(name)
    inp = make_cpu_inputs(w)
    idx, gate, counts, _ = run_oracle_route(w, inp)
    fp8 = w.expert == "e4m3"
    off, st, inv, xs, xsc = oracle.permute(np_(inp["x"]), idx, counts, w.E, w.S,
                                           out_dtype=oracle.E4M3 if fp8 else None)
    out_dt = oracle.BF16 if w.act == "bf16" else oracle.F32
    ref = np.empty((xs.shape[0], w.H), np.uint16 if w.act == "bf16" else np.float32)
    if fp8:
        q13, s13, q2, s2 = fp8_weights(inp)
        layer = gpu_layer(w, inp, torch.from_numpy(q13).cuda(), torch.from_numpy(q2).cuda(),
                          torch.from_numpy(s13).cuda(), torch.from_numpy(s2).cuda(), packed=packed)
        layer.x_scale.copy_(torch.from_numpy(xsc))
    else:
        layer = gpu_layer(w, inp, packed=packed)
        w13n, w2n = np_(inp["w13"]), np_(inp["w2"])
    for g in range(w.E + w.S):
        lo, hi = int(off[g]), int(off[g + 1])
        if hi == lo:
            continue
        if fp8:
            ref[lo:hi] = oracle.expert_ffn(xs[lo:hi], q13[g], q2[g], out_dt, xsc[lo:hi], s13[g], s2[g])
        else:
            ref[lo:hi] = oracle.expert_ffn(xs[lo:hi], w13n[g], w2n[g], out_dt)
    layer.offsets.copy_(torch.from_numpy(off))
    layer.x_sorted.copy_(from_np(xs))
    layer.expert_ffn()
    torch.cuda.synchronize()
    got = np_(layer.y_sorted)
    err = rel_err(as_f64(got, w.act), as_f64(ref, w.act))
    log(f"    max rel err {err:.3e} (bound {TOL[w.expert]})")
    assert err <= TOL[w.expert]


@pytest.mark.parametrize("name", CASES)
def test_combine_bitexact(name):
    log(f"[combine] {name}")
    w = case(name)
    inp = make_cpu_inputs(w)
    idx, gate, counts, _ = run_oracle_route(w, inp)
    _, _, inv, _, _ = oracle.permute(np_(inp["x"])[:, :128].copy(), idx, counts, w.E, w.S)
    ys = workloads.make_y_sorted(w, seed=5)
    ref = oracle.combine(np_(ys), inv, gate, w.T, w.S)
    layer = gpu_layer(w, inp)
    layer.inv_perm.copy_(torch.from_numpy(inv))
    layer.topk_gate.copy_(torch.from_numpy(gate))
    layer.y_sorted.copy_(ys)
    layer.combine()
    torch.cuda.synchronize()
    assert np.array_equal(np_(layer.y).view(np.uint8), ref.view(np.uint8))


@pytest.mark.parametrize("name", ["tiny-fp32", "v3route-bf16", "maxE-bf16"])
def test_bias_update_bitexact(name):
    log(f"[bias_update] {name}")
    w = case(name)
    rng = np.random.default_rng(3)
    counts = rng.multinomial(w.T * w.K, np.ones(w.E) / w.E).astype(np.int32)
    counts[0] = 0
    counts[1] += w.T * w.K - counts.sum() if counts.sum() != w.T * w.K else 0
    mean_hits = (counts.astype(np.int64) * w.E == w.T * w.K).sum()
    bias = rng.uniform(-0.05, 0.05, w.E).astype(np.float32)
    ref = oracle.bias_update(counts, w.T, w.K, 0.01, bias)
    from mixture_experts_layer_added_amd import _lib as L
    p = shape_of(w).problem()
    dc = torch.from_numpy(counts).cuda()
    db = torch.from_numpy(bias).cuda()
    L.moe_bias_update(p, dc, 0.01, db)
    torch.cuda.synchronize()
    assert np.array_equal(np_(db).view(np.uint32), ref.view(np.uint32))
    log(f"    experts exactly at the mean: {mean_hits}")


@pytest.mark.parametrize("name", CASES)
def test_forward_end_to_end(name):
    log(f"[forward] {name}")
    w = case(name)
    inp = make_cpu_inputs(w)
    fp8 = w.expert == "e4m3"
    args = (np_(inp["x"]), np_(inp["w_router"]), np_(inp["bias"]), np_(inp["w13"]), np_(inp["w2"]),
            w.G, w.M, w.K, w.J)
    if fp8:
        q13, s13, q2, s2 = fp8_weights(inp)
        ref = oracle.forward(*args, shared=w.S, expert_dtype=oracle.E4M3, w13_q=q13, w13_s=s13,
                             w2_q=q2, w2_s=s2)
        from mixture_experts_layer_added_amd.layer import quantize_weights_fp8
        g13, gs13 = quantize_weights_fp8(to_dev(inp["w13"]))
        g2, gs2 = quantize_weights_fp8(to_dev(inp["w2"]))
        layer = gpu_layer(w, inp, g13, g2, gs13, gs2)
    else:
        ref = oracle.forward(*args, shared=w.S)
        layer = gpu_layer(w, inp)
    y = layer.forward(to_dev(inp["x"]))
    torch.cuda.synchronize()
    for k in ("topk_idx", "counts", "offsets", "sorted_token", "inv_perm"):
        assert np.array_equal(np_(getattr(layer, k)), ref[k]), k
    assert np.array_equal(np_(layer.topk_gate).view(np.uint32), ref["topk_gate"].view(np.uint32))
    assert np.array_equal(np_(layer.x_sorted).view(np.uint8), ref["x_sorted"].view(np.uint8))
    ys_ref = as_f64(ref["y_sorted"], w.act)
    e1 = rel_err(as_f64(np_(layer.y_sorted), w.act), ys_ref)
    # y = Y_shared + sum_k g_k Y_k with sum_k g_k = 1, so an expert-output error of at
    # most tol*max|Y| moves y by at most 2*tol*max|Y|
    y_ref = as_f64(ref["y"], w.act)
    dy = np.abs(as_f64(np_(y), w.act) - y_ref).max()
    e2 = float(dy / (2 * np.abs(ys_ref).max()))
    # y's own normwise error (reported, not bounded: with FP8 experts it can exceed the
    # expert-output tolerance because y is smaller than the rows it sums)
    e3 = float(dy / np.abs(y_ref).max())
    log(f"    y_sorted rel err {e1:.3e}, y err / (2 max|Y|) {e2:.3e} (bound {TOL[w.expert]}); "
        f"y err / max|y| {e3:.3e}")
    assert e1 <= TOL[w.expert] and e2 <= TOL[w.expert]


@pytest.mark.parametrize("name", ["ragged-bf16", "ragged-fp8", "tiny-fp32"])
def test_forward_deterministic(name):
    log(f"[determinism] {name}")
    w = case(name)
    inp = make_cpu_inputs(w)
    if w.expert == "e4m3":
        from mixture_experts_layer_added_amd.layer import quantize_weights_fp8
        g13, gs13 = quantize_weights_fp8(to_dev(inp["w13"]))
        g2, gs2 = quantize_weights_fp8(to_dev(inp["w2"]))
        layer = gpu_layer(w, inp, g13, g2, gs13, gs2)
    else:
        layer = gpu_layer(w, inp)
    x = to_dev(inp["x"])
    outs = []
    for _ in range(2):
        layer.forward(x)
        torch.cuda.synchronize()
        outs.append({k: np_(getattr(layer, k)).copy() for k in
                     ("topk_idx", "topk_gate", "counts", "offsets", "sorted_token", "inv_perm",
                      "x_sorted", "y_sorted", "y")})
    for k in outs[0]:
        assert np.array_equal(outs[0][k].view(np.uint8), outs[1][k].view(np.uint8)), k


def test_checker_detects_planted_oracle_mistakes():
    """The comparisons above are live: a single flipped index, count or bias bit in the
    expected values (planted on the CPU side) makes them fail."""
    w = case("v3route-bf16")
    inp = make_cpu_inputs(w)
    idx, gate, counts, z = run_oracle_route(w, inp)
    layer = gpu_layer(w, inp)
    layer.route(to_dev(inp["x"]))
    torch.cuda.synchronize()
    got_idx = np_(layer.topk_idx)
    assert np.array_equal(got_idx, idx)
    bad = idx.copy()
    bad[7, 3] = (bad[7, 3] + 1) % w.E
    assert not np.array_equal(got_idx, bad)
    badc = counts.copy()
    badc[5] += 1
    assert not np.array_equal(np_(layer.counts), badc)
    badg = gate.copy()
    badg.view(np.uint32)[3, 2] ^= 1
    assert not np.array_equal(np_(layer.topk_gate).view(np.uint32), badg.view(np.uint32))
