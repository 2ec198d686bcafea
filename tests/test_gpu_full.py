"""GPU parity at the full DeepSeek-V3 layer shape (hidden 7168, 256 routed experts + 1
shared, top-8 of 8 groups with at most 4 per token, SwiGLU width 2048), in the launch
configuration the benchmark times.

The oracle recomputes everything it can at full size: routing of every token (logits,
indices, gates, counts bit for bit) and the permutation; the expert FFN and the combine
are checked on sampled tokens, which the oracle computes one by one from the inputs and
its own routing.  The skewed balancing loop compares the bias bit for bit at each of 50
steps.
"""
import concurrent.futures as cf

import numpy as np
import pytest

import oracle
import workloads
from gpu_cases import TOL, as_f64, log, shape_of

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mixture_experts_layer_added_amd import _lib
    _lib.lib()
    yield
    torch.cuda.empty_cache()


def np_(t):
    return workloads.to_numpy(t)


def build(w, fp8=False, gather=False):
    from mixture_experts_layer_added_amd.layer import MoELayer, quantize_weights_fp8
    dev = torch.device("cuda")
    wr, b = workloads.make_router(w, dev)
    w13, w2 = workloads.make_experts(w, dev)
    s13 = s2 = None
    if fp8:
        q13, s13 = quantize_weights_fp8(w13)
        q2, s2 = quantize_weights_fp8(w2)
        return MoELayer(shape_of(w), wr, b, q13, q2, s13, s2, gather=gather), (w13, w2)
    return MoELayer(shape_of(w), wr, b, w13, w2, gather=gather), (w13, w2)


def check_routing(w, layer, x):
    """Full-size routing and permutation against the oracle (bit for bit).
    Returns the oracle's routing."""
    xn = np_(x)
    idx, gate, counts, z = oracle.route(xn, np_(layer.w_router), np_(layer.bias), w.G, w.M, w.K,
                                        w.J, want_logits=True)
    assert np.array_equal(np_(layer.logits).view(np.uint32), z.view(np.uint32))
    assert np.array_equal(np_(layer.topk_idx), idx)
    assert np.array_equal(np_(layer.topk_gate).view(np.uint32), gate.view(np.uint32))
    assert np.array_equal(np_(layer.counts), counts)
    fp8 = w.expert == "e4m3"
    off, st, inv, xs, xsc = oracle.permute(xn, idx, counts, w.E, w.S,
                                           out_dtype=oracle.E4M3 if fp8 else None)
    assert np.array_equal(np_(layer.offsets), off)
    assert np.array_equal(np_(layer.sorted_token), st)
    assert np.array_equal(np_(layer.inv_perm), inv)
    rng = np.random.default_rng(0)
    if layer.gather:
        # no x_sorted; FP8 codes per token (the oracle's permuted rows of those tokens)
        if fp8:
            tok = np.unique(np.concatenate([rng.integers(0, w.T, 500), [0, w.T - 1]]))
            rows = w.T * w.K + tok  # shared-expert rows hold token t at T*K + t
            g = torch.from_numpy(tok).cuda()
            assert np.array_equal(np_(layer.x_q[g]), xs[rows])
            assert np.array_equal(np_(layer.x_scale[g]).view(np.uint32),
                                  xsc[rows].view(np.uint32))
    else:
        rows = np.unique(np.concatenate([rng.integers(0, w.R, 3000), [0, w.R - 1, w.T * w.K]]))
        got = np_(layer.x_sorted[torch.from_numpy(rows).cuda()])
        assert np.array_equal(got.view(np.uint8), xs[rows].view(np.uint8))
        if fp8:
            gsc = np_(layer.x_scale[torch.from_numpy(rows).cuda()])
            assert np.array_equal(gsc.view(np.uint32), xsc[rows].view(np.uint32))
    log(f"    routing/permutation bit-exact for all {w.T} tokens; "
        f"loads min/max {counts.min()}/{counts.max()} (mean {w.T * w.K / w.E:.1f})")
    return idx, gate, counts, inv, xs, xsc


def sampled_tokens(w, n, seed=0):
    rng = np.random.default_rng(seed)
    t = rng.choice(w.T, size=min(n, w.T), replace=False)
    return np.unique(np.concatenate([t, [0, w.T - 1]]))[: n + 2]


def check_sampled_outputs(w, layer, idx, gate, inv, xs, xsc, wts, tokens):
    """Oracle expert outputs and combined outputs of the sampled tokens vs the GPU's."""
    fp8 = w.expert == "e4m3"
    groups = sorted(set(int(e) for t in tokens for e in idx[t]) | {w.E})
    out_dt = oracle.BF16 if w.act == "bf16" else oracle.F32
    # oracle rows: (t, group) -> row of x_sorted
    work = {}
    for t in tokens:
        for k in range(w.K):
            work.setdefault(int(idx[t, k]), []).append(int(inv[t, k]))
        work.setdefault(w.E, []).append(w.T * w.K + int(t))
    if fp8:
        w13b, w2b = wts

    def one(g):
        rows = np.array(work[g])
        if fp8:
            a, sa = oracle.quantize_weight_fp8(np_(w13b[g]))
            b, sb = oracle.quantize_weight_fp8(np_(w2b[g]))
            assert np.array_equal(np_(layer.w13[g]), a)
            assert np.array_equal(np_(layer.w13_scale[g]).view(np.uint32), sa.view(np.uint32))
            assert np.array_equal(np_(layer.w2[g]), b)
            assert np.array_equal(np_(layer.w2_scale[g]).view(np.uint32), sb.view(np.uint32))
            y = oracle.expert_ffn(xs[rows], a, b, out_dt, xsc[rows], sa, sb, nthreads=1)
        else:
            y = oracle.expert_ffn(xs[rows], np_(layer.w13[g]), np_(layer.w2[g]), out_dt, nthreads=1)
        return g, rows, y

    ref_rows = {}
    with cf.ThreadPoolExecutor(oracle.default_threads()) as ex:
        for g, rows, y in ex.map(one, groups):
            for r, yr in zip(rows, y):
                ref_rows[int(r)] = yr
    allrows = np.array(sorted(ref_rows))
    ref = np.stack([ref_rows[r] for r in allrows])
    got = np_(layer.y_sorted[torch.from_numpy(allrows).cuda()])
    e1 = float(np.abs(as_f64(got, w.act) - as_f64(ref, w.act)).max() / np.abs(as_f64(ref, w.act)).max())
    # combine of the sampled tokens from the oracle's rows, in the oracle's order
    n = len(tokens)
    mini = np.zeros((n * w.K + n, w.H), ref.dtype)
    mini_inv = np.zeros((n, w.K), np.int32)
    for i, t in enumerate(tokens):
        for k in range(w.K):
            mini[i * w.K + k] = ref_rows[int(inv[t, k])]
            mini_inv[i, k] = i * w.K + k
        mini[n * w.K + i] = ref_rows[w.T * w.K + int(t)]
    yref = oracle.combine(mini, mini_inv, np.ascontiguousarray(gate[tokens]), n, w.S)
    ygot = np_(layer.y[torch.from_numpy(tokens).cuda()])
    dy = np.abs(as_f64(ygot, w.act) - as_f64(yref, w.act)).max()
    e2 = float(dy / (2 * np.abs(as_f64(ref, w.act)).max()))
    log(f"    sampled {n} tokens ({len(allrows)} expert rows): y_sorted rel err {e1:.3e}, "
        f"y err / (2 max|Y|) {e2:.3e} (bound {TOL[w.expert]})")
    assert e1 <= TOL[w.expert] and e2 <= TOL[w.expert]


@pytest.mark.parametrize("name,n_tok,gather", [("v3-bf16", 10, False), ("v3-decode", 8, False),
                                               ("v3-fp8", 6, False), ("v3-bf16", 6, True),
                                               ("v3-fp8", 4, True), ("v3-decode", 6, True)])
def test_full_shape_forward(name, n_tok, gather):
    w = workloads.get(name)
    log(f"[full] {name}: T={w.T} H={w.H} E={w.E}+{w.S} K={w.K} I={w.I} expert={w.expert} "
        f"gather={gather}")
    layer, wts = build(w, fp8=w.expert == "e4m3", gather=gather)
    x = workloads.make_x(w, device="cuda")
    layer.forward(x)
    torch.cuda.synchronize()
    idx, gate, counts, inv, xs, xsc = check_routing(w, layer, x)
    check_sampled_outputs(w, layer, idx, gate, inv, xs, xsc, wts, sampled_tokens(w, n_tok))
    del layer, wts, x
    torch.cuda.empty_cache()


def _load_stats(layer, w):
    """Batch load statistics of the last routing from the GPU: moe_seq_load_stats with
    the batch as one sequence (max, min, experts without tokens, max/mean)."""
    from mixture_experts_layer_added_amd import _lib as L
    dev = layer.counts.device
    off = torch.tensor([0, w.T], dtype=torch.int32, device=dev)
    c = torch.empty((1, w.E), dtype=torch.int32, device=dev)
    st = torch.empty((1, 3), dtype=torch.int32, device=dev)
    r = torch.empty((1,), dtype=torch.float32, device=dev)
    L.moe_seq_load_stats(layer.p, layer.topk_idx, off, 1, c, st, r)
    return c, st, r


def test_skew_loop_bias_trajectory(tmp_path):
    """50 forward + bias-update steps on fresh seeded x with Zipf-skewed router logits:
    the GPU and oracle biases agree bit for bit after every step.  Each step also logs
    one JSON line of load statistics (max/mean, min, experts without tokens, bias range;
    the pages follow expert utilisation as training goes, mpbf.cn section 6.2), taken on
    the GPU and equal to the oracle's.  Then the run is resumed from a checkpoint: the
    bias bits after step 25 are saved to a file, restored into the layer, and steps 25..49
    repeated must end at the same bias bit for bit."""
    import json
    w = workloads.get("v3-skew-loop")
    log(f"[skew loop] T={w.T}, {w.steps} steps, gamma={w.gamma}")
    layer, _ = build(w)
    wr = np_(layer.w_router)
    b_ref = np_(layer.bias).copy()
    ratios = []
    half = w.steps // 2
    ckpt = tmp_path / "bias_state.json"
    for step in range(w.steps):
        x = workloads.make_x(w, step=step, device="cuda")
        layer.step(x, w.gamma)
        _, _, counts, _ = oracle.route(np_(x), wr, b_ref, w.G, w.M, w.K, w.J)
        b_ref = oracle.bias_update(counts, w.T, w.K, w.gamma, b_ref)
        c, st, r = _load_stats(layer, w)
        torch.cuda.synchronize()
        assert np.array_equal(np_(layer.counts), counts), step
        assert np.array_equal(np_(layer.bias).view(np.uint32), b_ref.view(np.uint32)), step
        rc, rs, rr = oracle.seq_load_stats(np_(layer.topk_idx), w.E, [0, w.T])
        assert np.array_equal(np_(c), rc) and np.array_equal(np_(st), rs), step
        assert np_(r).view(np.uint32)[0] == rr.view(np.uint32)[0], step
        ratios.append(float(rr[0]))
        log(json.dumps({"step": step, "max_over_mean": round(float(rr[0]), 4),
                        "max_load": int(rs[0, 0]), "min_load": int(rs[0, 1]),
                        "zero_load_experts": int(rs[0, 2]),
                        "top16_share": round(workloads.zipf_top16_share(counts), 4),
                        "bias_min": float(b_ref.min()), "bias_max": float(b_ref.max())}))
        if step == half - 1:
            ckpt.write_text(json.dumps({"step": half,
                                        "bias_bits": np_(layer.bias).view(np.uint32).tolist()}))
    b_final = np_(layer.bias).copy()
    # the balancing pushes the load toward uniform (the pages describe this qualitatively)
    assert ratios[-1] < ratios[0]
    # resume from the checkpoint
    state = json.loads(ckpt.read_text())
    layer.bias.copy_(torch.from_numpy(np.array(state["bias_bits"], np.uint32).view(np.float32)))
    for step in range(state["step"], w.steps):
        layer.step(workloads.make_x(w, step=step, device="cuda"), w.gamma)
    torch.cuda.synchronize()
    assert np.array_equal(np_(layer.bias).view(np.uint32), b_final.view(np.uint32))
    log(f"    resumed from step {state['step']}: final bias bit-identical to the straight run")
    del layer
    torch.cuda.empty_cache()
