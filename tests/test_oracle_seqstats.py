"""Pins of the oracle's sequence-wise load statistic (mpbf.cn "DeepSeek-V3技术报告",
section 2.2: a sequence-level balance term with a very small weight guards against
extreme imbalance within one sequence; the pages print no formula for it, so the
oracle computes only the loads it would be built from).

Independent checks: per-sequence numpy bincount; the sequences' counts add up to the
whole batch's counts from the routing; one sequence spanning the batch reproduces the
batch histogram; closed forms of max / mean for a perfectly balanced sequence (1) and
for a sequence whose tokens all choose the same K experts (E/K); empty sequences."""
import numpy as np
import pytest

import oracle


def _bincount_ref(idx, off, E):
    return np.stack([np.bincount(idx[off[s]:off[s + 1]].ravel(), minlength=E)
                     for s in range(len(off) - 1)]).astype(np.int32)


@pytest.mark.parametrize("T,E,K,n_seq,seed", [(256, 16, 4, 1, 0), (1000, 64, 6, 7, 1),
                                              (513, 32, 8, 40, 2), (64, 8, 1, 64, 3)])
def test_counts_equal_bincount_per_sequence(T, E, K, n_seq, seed):
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.choice(E, size=K, replace=False) for _ in range(T)]).astype(np.int32)
    cuts = np.sort(rng.integers(0, T + 1, size=n_seq - 1))
    off = np.concatenate([[0], cuts, [T]]).astype(np.int32)
    counts, stats, ratio = oracle.seq_load_stats(idx, E, off)
    ref = _bincount_ref(idx, off, E)
    assert np.array_equal(counts, ref)
    assert np.array_equal(stats[:, 0], ref.max(axis=1))
    assert np.array_equal(stats[:, 1], ref.min(axis=1))
    assert np.array_equal(stats[:, 2], (ref == 0).sum(axis=1))
    # the sequences partition the batch: their counts add up to the batch histogram
    assert np.array_equal(counts.sum(axis=0), oracle.count(idx, E))
    L = np.diff(off).astype(np.float64)
    mean = L * K / E
    want = np.where(L > 0, ref.max(axis=1) / np.where(mean > 0, mean, 1), 0.0)
    # within one float32 rounding of the exact quotient
    assert np.all(np.abs(ratio.astype(np.float64) - want) <= np.abs(want) * 2.0 ** -23)


def test_single_sequence_is_the_batch_histogram():
    """Routing from the oracle itself on a tiny layer: one sequence over the whole
    batch gives the batch counts."""
    rng = np.random.default_rng(5)
    T, H, E, G, M, K, J = 300, 64, 32, 4, 2, 6, 2
    x = rng.standard_normal((T, H)).astype(np.float32)
    wr = (0.02 * rng.standard_normal((E, H))).astype(np.float32)
    b = np.zeros(E, np.float32)
    idx, _, counts, _ = oracle.route(x, wr, b, G, M, K, J)
    c, stats, ratio = oracle.seq_load_stats(idx, E, [0, T])
    assert np.array_equal(c[0], counts)
    assert stats[0, 0] == counts.max() and stats[0, 1] == counts.min()
    assert stats[0, 2] == int((counts == 0).sum())
    assert c.sum() == T * K


def test_closed_forms():
    E, K = 16, 4
    # balanced: 8 tokens cycling through the experts in blocks of K -> every expert
    # chosen exactly twice; max = min = mean, ratio exactly 1
    bal = np.array([[(4 * t + k) % E for k in range(K)] for t in range(8)], np.int32)
    # concentrated: 10 tokens all choosing experts 3, 5, 7, 9 -> max = 10, ratio = E/K
    conc = np.tile(np.array([3, 5, 7, 9], np.int32), (10, 1))
    idx = np.concatenate([bal, conc])
    counts, stats, ratio = oracle.seq_load_stats(idx, E, [0, 8, 8, 18])
    assert np.all(counts[0] == 2) and stats[0].tolist() == [2, 2, 0] and ratio[0] == 1.0
    # the empty middle sequence
    assert np.all(counts[1] == 0) and stats[1].tolist() == [0, 0, E] and ratio[1] == 0.0
    assert stats[2].tolist() == [10, 0, E - K] and ratio[2] == np.float32(E / K)
    assert counts[2, [3, 5, 7, 9]].tolist() == [10] * 4
