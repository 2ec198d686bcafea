"""Pins of the oracle's layer backward (CPU).

The backward is the derivative of the forward (the pages only fix that the routing
bias takes no gradient and that gradients accumulate at high precision), so it is
pinned by what calculus fixes, independently of the oracle's own code:
  - central finite differences of an fp64 numpy forward of the same layer (routing
    frozen at the oracle's choice) along random directions, for dx, dW_r, dW13, dW2;
  - renormalised gates are invariant to scaling all chosen affinities, so the
    affinity gradient satisfies sum_j s_j ds_j = 0;
  - the bias only selects: two biases that select the same experts give identical
    gradients, bit for bit;
  - dy = 0 gives zero gradients; a token whose chosen logits are clamped (|z| > 80)
    passes no gradient to the router.
"""
import numpy as np
import pytest

import oracle

G, M, K, J = 2, 2, 3, 2


def make(seed=0, T=12, H=64, E=8, I=32):
    rng = np.random.default_rng(seed)
    x = rng.normal(0, 1, (T, H)).astype(np.float32)
    wr = rng.normal(0, 0.5, (E, H)).astype(np.float32)
    bias = rng.uniform(-0.01, 0.01, E).astype(np.float32)
    w13 = rng.normal(0, 0.3, (E + 1, 2 * I, H)).astype(np.float32)
    w2 = rng.normal(0, 0.3, (E + 1, H, I)).astype(np.float32)
    dy = rng.normal(0, 1, (T, H)).astype(np.float32)
    return x, wr, bias, w13, w2, dy


def oracle_grads(x, wr, bias, w13, w2, dy):
    fwd = oracle.forward(x, wr, bias, w13, w2, G, M, K, J)
    _, _, _, z = oracle.route(x, wr, bias, G, M, K, J, want_logits=True)
    return fwd, oracle.backward(x, wr, w13, w2, fwd, dy, z)


def np_loss(x, wr, w13, w2, idx, dy):
    """fp64 layer forward with the routing frozen at idx; returns sum(dy * y)."""
    x, wr, w13, w2, dy = (np.asarray(a, np.float64) for a in (x, wr, w13, w2, dy))
    E = wr.shape[0]
    I = w2.shape[2]
    s = 1.0 / (1.0 + np.exp(-(x @ wr.T)))
    sel = np.take_along_axis(s, idx, axis=1)
    g = sel / sel.sum(axis=1, keepdims=True)

    def ffn(e, rows):
        a = rows @ w13[e, :I].T
        u = rows @ w13[e, I:].T
        return (a / (1.0 + np.exp(-a)) * u) @ w2[e].T

    y = ffn(E, x)  # shared expert
    for k in range(idx.shape[1]):
        for e in np.unique(idx[:, k]):
            t = np.nonzero(idx[:, k] == e)[0]
            y[t] += g[t, k:k + 1] * ffn(e, x[t])
    return float((dy * y).sum())


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_backward_matches_finite_differences(seed):
    x, wr, bias, w13, w2, dy = make(seed)
    fwd, b = oracle_grads(x, wr, bias, w13, w2, dy)
    idx = fwd["topk_idx"]
    rng = np.random.default_rng(100 + seed)
    args = dict(x=x, wr=wr, w13=w13, w2=w2)
    grads = dict(x=b["dx"], wr=b["dw_router"], w13=b["dw13"], w2=b["dw2"])
    for name in args:
        v = rng.normal(0, 1, args[name].shape)
        eps = 1e-4
        plus = dict(args); plus[name] = args[name] + eps * v
        minus = dict(args); minus[name] = args[name] - eps * v
        fd = (np_loss(plus["x"], plus["wr"], plus["w13"], plus["w2"], idx, dy)
              - np_loss(minus["x"], minus["wr"], minus["w13"], minus["w2"], idx, dy)) / (2 * eps)
        an = float((grads[name].astype(np.float64) * v).sum())
        assert abs(an - fd) <= 1e-5 * max(1.0, abs(fd)), (name, an, fd)


def test_affinity_gradient_is_scale_invariant():
    x, wr, bias, w13, w2, dy = make(3)
    fwd, b = oracle_grads(x, wr, bias, w13, w2, dy)
    _, _, _, z = oracle.route(x, wr, bias, G, M, K, J, want_logits=True)
    # the fp32 affinities the gates were built from (the sigmoid is pinned elsewhere)
    s = oracle.sigmoid_array(np.take_along_axis(z, fwd["topk_idx"], axis=1)).astype(np.float64)
    ds = b["dz"].astype(np.float64) / (s * (1 - s))
    scale = np.abs(s * ds).sum(axis=1)
    assert np.all(np.abs((s * ds).sum(axis=1)) <= 1e-5 * np.maximum(scale, 1e-30))


def test_bias_has_no_gradient_path():
    x, wr, bias, w13, w2, dy = make(4)
    fwd1, b1 = oracle_grads(x, wr, bias, w13, w2, dy)
    bias2 = (bias + np.float32(1e-4)).astype(np.float32)  # uniform shift: same selection
    fwd2, b2 = oracle_grads(x, wr, bias2, w13, w2, dy)
    assert np.array_equal(fwd1["topk_idx"], fwd2["topk_idx"])
    for k in ("dx", "dw_router", "dw13", "dw2", "dz"):
        assert np.array_equal(b1[k].view(np.uint8), b2[k].view(np.uint8)), k


def test_zero_output_gradient():
    x, wr, bias, w13, w2, dy = make(5)
    _, b = oracle_grads(x, wr, bias, w13, w2, np.zeros_like(dy))
    for k in ("dx", "dw_router", "dw13", "dw2", "dz", "dgate"):
        assert not np.any(b[k].astype(np.float64)), k


def test_clamped_logits_pass_no_router_gradient():
    x, wr, bias, w13, w2, dy = make(6)
    x[0] *= 0.0
    x[0, 0] = 1.0
    wr[:, 0] = 200.0  # every logit of token 0 is 200 > 80: sigmoid clamped
    fwd, b = oracle_grads(x, wr, bias, w13, w2, dy)
    assert not np.any(b["dz"][0])
    assert np.any(b["dz"][1:])


def test_bf16_backward_tracks_f32():
    """The bf16 path rounds the stored tensors (dY, [da|du], the permuted input
    gradient, dx) to bf16; on bf16-representable inputs its gradients stay within
    bf16 rounding of the fp32 path's."""
    x, wr, bias, w13, w2, dy = make(7)

    def to_bf16(a):
        return np.array([oracle.bf16_from_f64(float(v)) for v in a.ravel()],
                        np.uint16).reshape(a.shape)

    xb, w13b, w2b, dyb = (to_bf16(a) for a in (x, w13, w2, dy))
    xf, w13f, w2f, dyf = (oracle.bf16_to_f32(a) for a in (xb, w13b, w2b, dyb))
    _, bf = oracle_grads(xf, wr, bias, w13f, w2f, dyf)
    _, bb = oracle_grads(xb, wr, bias, w13b, w2b, dyb)
    for k in ("dx", "dw_router", "dw13", "dw2"):
        a = bb[k]
        a = oracle.bf16_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)
        ref = bf[k].astype(np.float64)
        assert np.abs(a - ref).max() <= 2e-2 * np.abs(ref).max(), k


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_local_decompositions_match_full_backward(act):
    """The full-size GPU test checks the backward through one-token problems and
    column-sliced expert problems; both must equal the full oracle backward exactly
    (same arithmetic on the same values), here on a small layer."""
    from gpu_cases import slice_reference, token_reference
    from types import SimpleNamespace
    x, wr, bias, w13, w2, dy = make(seed=4, T=20, H=128, E=8, I=16)
    if act == "bf16":
        cv = lambda a: oracle.bf16_from_f64_array(a.astype(np.float64))  # noqa: E731
        x, w13, w2, dy = cv(x), cv(w13), cv(w2), cv(dy)
    fwd, bw = oracle_grads(x, wr, bias, w13, w2, dy)
    _, _, _, z = oracle.route(x, wr, bias, G, M, K, J, want_logits=True)
    E, I, T = wr.shape[0], w2.shape[2], x.shape[0]
    w = SimpleNamespace(T=T, H=x.shape[1], E=E, K=K, I=I, S=1, act=act)
    idx, gate, inv = fwd["topk_idx"], fwd["topk_gate"], fwd["inv_perm"]
    for t in (0, 7, T - 1):
        r = token_reference(w, t, x, wr, z, idx, gate, dy, lambda g: w13[g], lambda g: w2[g])
        assert np.array_equal(r["dgate"].view(np.uint32), bw["dgate"][t].view(np.uint32))
        assert np.array_equal(r["dz"].view(np.uint32), bw["dz"][t].view(np.uint32))
        rows = list(inv[t]) + [T * K + t]
        assert np.array_equal(r["dy_sorted"], bw["dy_sorted"][rows])
        assert np.array_equal(r["dau"], bw["dau"][rows])
        assert np.array_equal(r["dx"], bw["dx"][t])
    off, st = fwd["offsets"], fwd["sorted_token"]
    for g in (int(np.argmax(fwd["counts"])), E):
        toks = st[off[g]:off[g + 1]].astype(np.int64)
        gates = (gate[toks, np.argmax(idx[toks] == g, axis=1)] if g < E
                 else np.ones(len(toks), np.float32))
        for n in (0, 5, I - 1):
            r = slice_reference(w, g, n, x, toks, gates, dy, lambda e: w13[e], lambda e: w2[e])
            assert np.array_equal(r["dw2"], bw["dw2"][g][:, n])
            assert np.array_equal(r["dw13_a"], bw["dw13"][g][n])
            assert np.array_equal(r["dw13_u"], bw["dw13"][g][I + n])
            assert np.array_equal(r["dau"], bw["dau"][off[g]:off[g + 1]][:, [n, I + n]])


def test_input_part_alone_equals_the_full_expert_backward():
    """expert_backward(weights=False) skips the weight gradients only: h, [da|du] and dx
    are bit for bit those of the full call."""
    rng = np.random.default_rng(21)
    n, H, I = 7, 256, 128
    for act in ("f32", "bf16"):
        def mk(shape, std):
            v = rng.standard_normal(shape) * std
            return (oracle.bf16_from_f64_array(v).reshape(shape) if act == "bf16"
                    else v.astype(np.float32))
        x, dy = mk((n, H), 1.0), mk((n, H), 1.0)
        w13, w2 = mk((2 * I, H), 0.05), mk((H, I), 0.05)
        full = oracle.expert_backward(x, w13, w2, dy)
        part = oracle.expert_backward(x, w13, w2, dy, weights=False)
        assert part[3] is None and part[4] is None
        for a, b in zip(full[:3], part[:3]):
            assert np.array_equal(a, b)
