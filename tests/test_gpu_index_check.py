"""GPU: moe_count_invalid_ids counts the (token, slot) pairs of a caller-built topk_idx
that lie outside [0,E) -- the pairs moe_permute's precondition excludes -- exactly, and
clears its count on every call."""
import numpy as np
import pytest

from gpu_cases import log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mixture_experts_layer_added_amd import _lib
    _lib.lib()


# (T, K, E, G, M, number of planted out-of-range pairs, seed)
CASES = [(1000, 4, 16, 4, 2, 0, 0), (1000, 4, 16, 4, 2, 37, 1), (70000, 8, 256, 8, 4, 1, 2),
         (257, 8, 256, 8, 4, 2056, 3)]


@pytest.mark.parametrize("T,K,E,G,M,n_bad,seed", CASES)
def test_count_invalid_ids(T, K, E, G, M, n_bad, seed):
    from mixture_experts_layer_added_amd import _lib as L
    log(f"[index check] T={T} K={K} E={E} planted={n_bad}")
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, E, size=(T, K)).astype(np.int32)
    if n_bad:
        pos = rng.choice(T * K, n_bad, replace=False)
        bad = np.array([-1, E, E + 5, -(2 ** 31), 2 ** 31 - 1], np.int64)
        idx.flat[pos] = rng.choice(bad, n_bad).astype(np.int32)
    expect = int(((idx < 0) | (idx >= E)).sum())
    assert expect == n_bad
    p = L.problem(T, 256, E, G, M, K, 2, 128, 1, L.MOE_BF16, L.MOE_BF16)
    d_idx = torch.from_numpy(idx).cuda()
    n = torch.full((4,), 12345, dtype=torch.int32, device="cuda")
    L.moe_count_invalid_ids(p, d_idx, n)
    torch.cuda.synchronize()
    assert int(n[0]) == expect
    # a second call on valid indices clears the count
    d_idx.clamp_(0, E - 1)
    L.moe_count_invalid_ids(p, d_idx, n)
    torch.cuda.synchronize()
    assert int(n[0]) == 0
    assert n[1:].tolist() == [12345] * 3  # nothing past the one count is written
