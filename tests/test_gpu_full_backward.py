"""GPU parity of the layer backward at the full DeepSeek-V3 layer shape (hidden 7168,
256 routed experts + 1 shared, top-8 of 8 groups with at most 4 per token, SwiGLU width
2048, bf16), in the dispatch form the benchmark times; also at the decode size (T=128,
most experts with a few rows or none) and on the skewed T=8192 batch (the most loaded
experts span many row tiles).

The oracle cannot run the whole backward at this size, so it computes what is local:
  * every gradient of a sampled token -- dgate, dz, the rows of dY and [da|du] that
    belong to it, and dx -- from a one-token problem (the token's K expert rows and
    its shared row), which is exactly the full problem restricted to that token;
  * sampled columns n of dW2[g] and rows n, I+n of dW13[g] for sampled experts g, from
    the expert's rows with its weights cut to the column pair (n, I+n) of the SwiGLU
    width -- h[:, n], da[:, n] and du[:, n] depend on nothing else.
The router weight gradient is checked as a property that holds at any size: row e
equals the sum over the rows of expert e of dz * x (fp64), with the GPU's own dz (the
sampled dz are pinned to the oracle above).  Experts without tokens get exactly zero
weight gradients.
"""
import concurrent.futures as cf

import numpy as np
import pytest

import oracle
import workloads
from gpu_cases import (TOL, as_f64, log, rel_err, shape_of, slice_reference,
                       token_reference)

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


def rows_of(layer, name, rows):
    return np_(getattr(layer, name)[torch.from_numpy(np.asarray(rows, np.int64)).cuda()])


@pytest.mark.parametrize("name,n_tok,gather", [("v3-bf16", 6, True), ("v3-decode", 6, False),
                                               ("v3-skew-loop", 4, True)])
def test_full_shape_backward(name, n_tok, gather):
    from mixture_experts_layer_added_amd.layer import MoELayer
    w = workloads.get(name)
    log(f"[full backward] {name}: T={w.T} H={w.H} E={w.E}+{w.S} K={w.K} I={w.I} "
        f"gather={gather}")
    dev = torch.device("cuda")
    wr_t, b_t = workloads.make_router(w, dev)
    w13_t, w2_t = workloads.make_experts(w, dev)
    layer = MoELayer(shape_of(w), wr_t, b_t, w13_t, w2_t, gather=gather, train=True)
    x = workloads.make_x(w, device="cuda")
    dy = workloads.make_dy(w, device="cuda")
    layer.forward(x)
    layer.backward(dy)
    torch.cuda.synchronize()
    xn, dyn, wr = np_(x), np_(dy), np_(layer.w_router)
    idx, gate, counts, z = oracle.route(xn, wr, np_(layer.bias), w.G, w.M, w.K, w.J,
                                        want_logits=True)
    assert np.array_equal(np_(layer.topk_idx), idx)
    assert np.array_equal(np_(layer.counts), counts)
    off, st, inv, _, _ = oracle.permute(xn, idx, counts, w.E, w.S)
    assert np.array_equal(np_(layer.offsets), off)
    assert np.array_equal(np_(layer.sorted_token), st)
    tol = TOL[w.expert]
    w13g = lambda g: np_(layer.w13[g])  # noqa: E731
    w2g = lambda g: np_(layer.w2[g])  # noqa: E731

    # --- sampled tokens: everything local to a token -------------------------
    rng = np.random.default_rng(5)
    tokens = np.unique(np.concatenate([rng.choice(w.T, n_tok, replace=False), [0, w.T - 1]]))
    with cf.ThreadPoolExecutor(oracle.default_threads()) as ex:
        refs = list(ex.map(lambda t: token_reference(w, t, xn, wr, z, idx, gate, dyn, w13g, w2g),
                           tokens))
    tk = torch.from_numpy(tokens.astype(np.int64)).cuda()
    got = {k: np_(getattr(layer, k)[tk]) for k in ("dgate", "dz", "dx")}
    errs = {}
    for k in ("dgate", "dz", "dx"):
        r = np.stack([ref[k] for ref in refs])
        errs[k] = rel_err(as_f64(got[k], w.act) if got[k].dtype == np.uint16 else got[k],
                          as_f64(r, w.act) if r.dtype == np.uint16 else r)
    rows = [list(inv[t]) + ([w.T * w.K + int(t)] if w.S else []) for t in tokens]
    for k in ("dy_sorted", "dau"):
        g_ = np.concatenate([rows_of(layer, k, r) for r in rows])
        r_ = np.concatenate([ref[k] for ref in refs])
        errs[k] = rel_err(as_f64(g_, w.act), as_f64(r_, w.act))
    log(f"    {len(tokens)} tokens: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= tol, k

    # --- weight-gradient slices of sampled experts ---------------------------
    loaded = np.nonzero(counts > 0)[0]
    experts = sorted({int(np.argmax(counts)), int(rng.choice(loaded)), int(rng.choice(loaded))})
    if w.S:
        experts.append(w.E)
    cols = [0, w.I - 1, int(rng.integers(1, w.I - 1))]
    work = []
    for g in experts:
        r0, r1 = int(off[g]), int(off[g + 1])
        toks = st[r0:r1].astype(np.int64)
        if g < w.E:
            kk = np.argmax(idx[toks] == g, axis=1)
            gates = gate[toks, kk]
        else:
            gates = np.ones(len(toks), np.float32)
        for n in cols:
            work.append((g, n, toks, gates, np.arange(r0, r1)))
    with cf.ThreadPoolExecutor(oracle.default_threads()) as ex:
        srefs = list(ex.map(lambda a: slice_reference(w, a[0], a[1], xn, a[2], a[3], dyn, w13g, w2g),
                            work))
    worst = {"dw2": 0.0, "dw13": 0.0, "dau": 0.0}
    for (g, n, toks, gates, rws), ref in zip(work, srefs):
        e_w2 = rel_err(np_(layer.dw2[g, :, n]), ref["dw2"])
        e_a = rel_err(np_(layer.dw13[g, n, :]), ref["dw13_a"])
        e_u = rel_err(np_(layer.dw13[g, w.I + n, :]), ref["dw13_u"])
        dau_g = rows_of(layer, "dau", rws)[:, [n, w.I + n]]
        e_d = rel_err(as_f64(dau_g, w.act), as_f64(ref["dau"], w.act))
        worst["dw2"] = max(worst["dw2"], e_w2)
        worst["dw13"] = max(worst["dw13"], e_a, e_u)
        worst["dau"] = max(worst["dau"], e_d)
        assert max(e_w2, e_a, e_u, e_d) <= tol, (g, n)
    log(f"    experts {experts} x columns {cols}: worst " +
        ", ".join(f"{k} {v:.2e}" for k, v in worst.items()) + f" (bound {tol})")

    # --- router weight gradient: sum over each expert's rows of dz * x --------
    dz = np_(layer.dz).astype(np.float64)
    dwr = np_(layer.dw_router)
    ref = np.zeros((w.E, w.H))
    xf = as_f64(xn, w.act)
    for k in range(w.K):
        np.add.at(ref, idx[:, k], dz[:, k:k + 1] * xf)
    e_r = rel_err(dwr, ref)
    log(f"    dw_router vs sum of dz x over each expert's rows: {e_r:.2e} (bound 1e-4)")
    assert e_r <= 1e-4

    # --- experts without tokens --------------------------------------------
    empty = np.nonzero(counts == 0)[0]
    for g in empty[:8]:
        assert not np.any(np_(layer.dw13[int(g)])) and not np.any(np_(layer.dw2[int(g)]))
        assert not np.any(dwr[g])
    log(f"    {len(empty)} experts without tokens: zero weight gradients")
    del layer, x, dy, w13_t, w2_t
    torch.cuda.empty_cache()
