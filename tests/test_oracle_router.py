"""Pins for the oracle's routing: logits, selection, gates, counts.

Selection follows the aux-loss-free, group-limited rule (mpbf.cn DeepSeek-V3 report
summary, section 2.2): key = sigmoid(z) + bias decides the choice, groups are ranked
by the sum of their top-J keys, the M best groups are kept, the K largest keys among
their experts win, and gates are the unbiased scores renormalised over the chosen K.
"""
import itertools

import numpy as np
import pytest

F32 = np.float32


# --------------------------------------------------------------------------- logits

def test_logits_one_hot_and_zero(orc):
    rng = np.random.default_rng(0)
    H, E, T = 64, 12, 5
    w = rng.standard_normal((E, H)).astype(F32)
    x = np.zeros((T, H), F32)
    for t in range(T):
        x[t, (7 * t + 3) % H] = 1.0
    z = orc.router_logits(x, w)
    for t in range(T):
        assert np.array_equal(z[t], w[:, (7 * t + 3) % H])
    assert np.array_equal(orc.router_logits(np.zeros((T, H), F32), w), np.zeros((T, E), F32))


def test_logits_float64_bound(orc):
    rng = np.random.default_rng(1)
    T, H, E = 37, 512, 20
    x = rng.standard_normal((T, H)).astype(F32)
    w = (rng.standard_normal((E, H)) * 0.02).astype(F32)
    z = orc.router_logits(x, w).astype(np.float64)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    bound = H * 2.0 ** -24 * (np.abs(x).astype(np.float64) @ np.abs(w).astype(np.float64).T)
    assert np.all(np.abs(z - ref) <= bound + 1e-30)


def test_logits_sequential_order_from_h0(orc):
    # x = [1,1,1], w = [2^24, 1, -2^24]: a chain from h=0 gives 2^24 -> 2^24 (1 is lost
    # to rounding) -> 0, while any other grouping keeps the 1.
    x = np.ones((1, 3), F32)
    w = np.array([[2.0 ** 24, 1.0, -2.0 ** 24]], F32)
    assert orc.router_logits(x, w)[0, 0] == 0.0
    w2 = np.array([[-2.0 ** 24, 2.0 ** 24, 1.0]], F32)
    assert orc.router_logits(x, w2)[0, 0] == 1.0


def test_logits_fused_single_rounding(orc):
    # h0: 1 * -1 = -1; h1: (1+2^-12)^2 - 1 = 2^-11 + 2^-24 exactly with one rounding;
    # a separate multiply would round the product to 1 + 2^-11 first and give 2^-11.
    a = F32(1.0 + 2.0 ** -12)
    x = np.array([[1.0, a]], F32)
    w = np.array([[-1.0, a]], F32)
    assert orc.router_logits(x, w)[0, 0] == F32(2.0 ** -11 + 2.0 ** -24)


def test_logits_bf16_input_equals_widened(orc):
    rng = np.random.default_rng(2)
    xb = orc.bf16_from_f64_array(rng.standard_normal((9, 128)))
    w = rng.standard_normal((7, 128)).astype(F32)
    assert np.array_equal(orc.router_logits(xb, w), orc.router_logits(orc.bf16_to_f32(xb), w))


# --------------------------------------------------------------------------- selection

def brute_select(z, bias, G, M, K, J, sig):
    """Independent restatement with Python sorting of tuples (value desc, index asc)."""
    T, E = z.shape
    gs = E // G
    idx = np.zeros((T, K), np.int32)
    gate = np.zeros((T, K), F32)
    for t in range(T):
        s = sig(z[t])
        key = (s + bias).astype(F32)
        gscore = []
        for g in range(G):
            members = sorted(range(g * gs, (g + 1) * gs), key=lambda e: (-float(key[e]), e))
            acc = F32(0.0)
            for e in members[:J]:
                acc = F32(acc + key[e])
            gscore.append(acc)
        kept = sorted(range(G), key=lambda g: (-float(gscore[g]), g))[:M]
        cand = [e for e in range(E) if e // gs in kept]
        chosen = sorted(cand, key=lambda e: (-float(key[e]), e))[:K]
        tot = F32(0.0)
        for e in chosen:
            tot = F32(tot + s[e])
        idx[t] = chosen
        gate[t] = [F32(s[e] / tot) for e in chosen]
    return idx, gate


@pytest.mark.parametrize("E,G,M,K,J", [(8, 4, 2, 2, 1), (8, 4, 2, 3, 2), (12, 3, 2, 4, 2),
                                       (16, 4, 2, 4, 2), (16, 4, 3, 7, 3), (32, 8, 4, 8, 2),
                                       (16, 1, 1, 5, 4), (16, 16, 3, 3, 1)])
def test_select_matches_brute_force(orc, E, G, M, K, J):
    rng = np.random.default_rng(E * 100 + G * 10 + K)
    T = 60
    z = (rng.standard_normal((T, E)) * 1.7).astype(F32)
    bias = rng.uniform(-0.05, 0.05, E).astype(F32)
    # integer logits for many exact ties
    z[T // 2:] = rng.integers(-2, 3, (T - T // 2, E)).astype(F32)
    bias[: E // 2] = 0.0
    idx, gate, counts = orc.select(z, bias, G, M, K, J)
    bidx, bgate = brute_select(z, bias, G, M, K, J, orc.sigmoid_array)
    assert np.array_equal(idx, bidx)
    assert np.array_equal(gate.view(np.uint32), bgate.view(np.uint32))
    assert np.array_equal(counts, np.bincount(idx.ravel(), minlength=E))


@pytest.mark.parametrize("E,K", [(16, 4), (64, 8), (256, 8)])
def test_select_all_groups_is_plain_topk(orc, E, K):
    # With every group kept (M = G) the rule is a plain top-K of the keys.
    rng = np.random.default_rng(E)
    T = 40
    z = (rng.standard_normal((T, E)) * 2).astype(F32)
    bias = rng.uniform(-0.01, 0.01, E).astype(F32)
    for G in (1, 4):
        idx, _, _ = orc.select(z, bias, G, G, K, 1)
        key = (orc.sigmoid_array(z) + bias).astype(F32)
        for t in range(T):
            order = np.lexsort((np.arange(E), -key[t].astype(np.float64)))
            assert np.array_equal(idx[t], order[:K])


def test_select_invariants_v3_shape(orc):
    rng = np.random.default_rng(5)
    T, E, G, M, K, J = 300, 256, 8, 4, 8, 2
    z = (rng.standard_normal((T, E)) * 1.7).astype(F32)
    bias = rng.uniform(-0.01, 0.01, E).astype(F32)
    idx, gate, counts = orc.select(z, bias, G, M, K, J)
    key = (orc.sigmoid_array(z) + bias).astype(F32)
    gs = E // G
    for t in range(T):
        groups = set(int(e) // gs for e in idx[t])
        assert len(groups) <= M
        assert len(set(idx[t].tolist())) == K
        chosen = set(idx[t].tolist())
        kmin = min(key[t, e] for e in chosen)
        for g in groups:
            for e in range(g * gs, (g + 1) * gs):
                if e not in chosen:
                    assert key[t, e] <= kmin
        # rank order: keys non-increasing
        ks = key[t, idx[t]]
        assert np.all(ks[:-1] >= ks[1:])
    assert np.all(np.abs(gate.astype(np.float64).sum(1) - 1.0) <= K * 2.0 ** -24)
    assert counts.sum() == T * K


def test_select_all_equal_keys_lowest_index(orc):
    # every key equal: groups 0..M-1 win on index, then experts 0..K-1 in order
    T, E, G, M, K = 3, 16, 4, 2, 6
    z = np.full((T, E), 0.25, F32)
    idx, gate, _ = orc.select(z, np.zeros(E, F32), G, M, K, 2)
    assert np.array_equal(idx, np.tile(np.arange(K, dtype=np.int32), (T, 1)))
    assert np.all(gate == gate[0, 0])


def test_select_hand_worked_example(orc):
    # E=8 in G=4 groups of 2, keep M=2 groups, K=2, group score = top-2 sum (J=2).
    # Logits chosen so the single two best keys (experts 0 and 2) sit in groups whose
    # pair sums lose: group sums are g0: s(3)+s(-3)=1, g1: s(2.5)+s(-3),
    # g2: s(1)+s(1) = 1.462, g3: s(0.5)+s(0.9) = 1.333.  Groups 2 and 3 win, so the
    # picks are experts 4 and 5 (equal logits 1: index order), not 0 and 2.
    z = np.array([[3.0, -3.0, 2.5, -3.0, 1.0, 1.0, 0.5, 0.9]], F32)
    idx, gate, _ = orc.select(z, np.zeros(8, F32), 4, 2, 2, 2)
    assert idx.tolist() == [[4, 5]]
    assert gate.tolist() == [[0.5, 0.5]]
    # with J=1 the group score is the best key: groups 0 and 1 win -> experts 0 and 2
    idx, gate, _ = orc.select(z, np.zeros(8, F32), 4, 2, 2, 1)
    assert idx.tolist() == [[0, 2]]
    s0, s2 = orc.sigmoid(3.0), orc.sigmoid(2.5)
    tot = F32(F32(s0) + F32(s2))
    assert gate[0].tolist() == [float(F32(s0) / tot), float(F32(s2) / tot)]


def test_bias_steers_choice_not_gate(orc):
    rng = np.random.default_rng(7)
    T, E, G, M, K, J = 50, 32, 4, 2, 4, 2
    z = (rng.standard_normal((T, E)) * 1.5).astype(F32)
    b = rng.uniform(-0.01, 0.01, E).astype(F32)
    idx, gate, _ = orc.select(z, b, G, M, K, J)
    # raise the bias of every expert each token already chose, per token: same choice,
    # bitwise the same gates
    for t in range(T):
        b2 = b.copy()
        b2[idx[t]] += 5.0
        i2, g2, _ = orc.select(z[t:t + 1], b2, G, M, K, J)
        assert set(i2[0].tolist()) == set(idx[t].tolist())
        order = [list(i2[0]).index(e) for e in idx[t]]
        assert np.array_equal(g2[0][order].view(np.uint32), gate[t].view(np.uint32))
    # a large bias forces an expert in, yet its gate stays its unbiased share
    b3 = np.zeros(E, F32)
    b3[17] = 10.0
    i3, g3, _ = orc.select(z, b3, G, M, K, J)
    assert np.all((i3 == 17).any(1))
    s = orc.sigmoid_array(z)
    for t in range(T):
        k = list(i3[t]).index(17)
        tot = F32(0.0)
        for e in i3[t]:
            tot = F32(tot + s[t, e])
        assert g3[t, k] == F32(s[t, 17] / tot)


def test_route_composes_logits_and_select(orc):
    rng = np.random.default_rng(8)
    T, H, E = 33, 256, 16
    x = rng.standard_normal((T, H)).astype(F32)
    w = (rng.standard_normal((E, H)) * 0.02).astype(F32)
    b = rng.uniform(-0.01, 0.01, E).astype(F32)
    idx, gate, counts, z = orc.route(x, w, b, 4, 2, 4, 2, want_logits=True)
    assert np.array_equal(z, orc.router_logits(x, w))
    i2, g2, c2 = orc.select(z, b, 4, 2, 4, 2)
    assert np.array_equal(idx, i2) and np.array_equal(gate, g2) and np.array_equal(counts, c2)


def test_route_rejects_bad_problems(orc):
    x = np.zeros((4, 128), F32)
    w = np.zeros((16, 128), F32)
    b = np.zeros(16, F32)
    for G, M, K, J in [(5, 2, 2, 1), (4, 5, 2, 1), (4, 2, 9, 1), (4, 2, 2, 5), (4, 0, 2, 1)]:
        with pytest.raises(ValueError):
            orc.route(x, w, b, G, M, K, J)


def test_threaded_equals_single_thread(orc):
    rng = np.random.default_rng(9)
    T, H, E = 200, 384, 32
    x = orc.bf16_from_f64_array(rng.standard_normal((T, H)))
    w = (rng.standard_normal((E, H)) * 0.02).astype(F32)
    b = rng.uniform(-0.01, 0.01, E).astype(F32)
    r1 = orc.route(x, w, b, 4, 2, 6, 2, nthreads=1, want_logits=True)
    r8 = orc.route(x, w, b, 4, 2, 6, 2, nthreads=8, want_logits=True)
    for a, c in zip(r1, r8):
        assert np.array_equal(a.view(np.uint8), c.view(np.uint8))
