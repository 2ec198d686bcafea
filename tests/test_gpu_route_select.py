"""GPU parity of the routing selection (sigmoid, bias-steered group-limited top-K, gates,
counts) on both selection kernels: the group-per-lane kernel (G a power of two from 2
to 64, E/G a multiple of 4 and at most 32) and the one-wave-per-token kernel that takes
every other shape.  Indices, gates, counts and logits must equal the oracle's bit for
bit, also where many keys, and group scores, are exactly equal (duplicated router rows),
and on a 262,144-token batch at the DeepSeek-V3 router shape, whose selection is
checked against the oracle's selection of the same logits."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_cases import log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mixture_experts_layer_added_amd import _lib
    _lib.lib()


# name -> (T, H, E, G, M, K, J, tied router rows: 0 = none, else rows repeat mod this)
CASES = {
    # one wave per token: a single group, G not a power of two, E/G not a multiple of 4,
    # E/G above 32
    "g1": (300, 128, 16, 1, 1, 4, 2, 0),
    "g3": (300, 128, 48, 3, 2, 4, 2, 0),
    "gs5": (300, 128, 20, 4, 2, 3, 2, 0),
    "gs40": (300, 128, 80, 2, 1, 6, 3, 0),
    "gs40-ties": (300, 128, 80, 2, 1, 6, 3, 7),
    # group per lane: two groups, the V3 grouping, 64 groups with K = 16, ties
    "g2": (257, 128, 8, 2, 1, 3, 2, 0),
    "v3-ties": (513, 128, 256, 8, 4, 8, 2, 5),
    "v3-ties-j3": (513, 128, 256, 8, 4, 8, 3, 3),
    "g64-ties": (130, 128, 512, 64, 4, 16, 8, 6),
    # 16- and 32-lane segments (the rounds' DPP row mirror, then one shuffle stage)
    "g16-ties": (300, 128, 128, 16, 4, 8, 2, 6),
    "g32": (200, 128, 256, 32, 8, 12, 3, 0),
    "g8-k16": (200, 128, 128, 8, 3, 16, 4, 0),
}


def _route_gpu(T, H, E, G, M, K, J, x, wr, b):
    from mixture_experts_layer_added_amd import _lib as L
    dev = "cuda"
    p = L.problem(T, H, E, G, M, K, J, 128, 1, L.MOE_BF16, L.MOE_BF16)
    idx = torch.empty((T, K), dtype=torch.int32, device=dev)
    gate = torch.empty((T, K), dtype=torch.float32, device=dev)
    counts = torch.empty((E,), dtype=torch.int32, device=dev)
    z = torch.empty((T, E), dtype=torch.float32, device=dev)
    n = L.moe_workspace_bytes(p, L.MOE_CALL_ROUTE)
    ws = torch.empty((max(n, 256),), dtype=torch.uint8, device=dev)
    L.moe_route(p, x, wr, b, idx, gate, counts, z, ws, ws.numel())
    torch.cuda.synchronize()
    return [workloads.to_numpy(t) for t in (idx, gate, counts, z)]


@pytest.mark.parametrize("name", sorted(CASES))
def test_select_bitexact(name):
    T, H, E, G, M, K, J, tie = CASES[name]
    log(f"[select] {name} T={T} E={E} G={G} M={M} K={K} J={J} tie={tie}")
    w = workloads.get("v3-bf16", T=T, H=H, E=E, G=G, M=M, K=K, J=J, I=128)
    wr, b = workloads.make_router(w)
    x = workloads.make_x(w)
    if tie:
        # rows repeat with period `tie`: equal logits; equal biases make equal keys
        wr = wr[torch.arange(E) % tie].contiguous()
        b = b[torch.arange(E) % tie].contiguous()
    idx, gate, counts, z = oracle.route(workloads.to_numpy(x), workloads.to_numpy(wr),
                                        workloads.to_numpy(b), G, M, K, J, want_logits=True)
    g_idx, g_gate, g_counts, g_z = _route_gpu(T, H, E, G, M, K, J, x.cuda(), wr.cuda(),
                                              b.cuda())
    assert np.array_equal(g_z.view(np.uint32), z.view(np.uint32))
    assert np.array_equal(g_idx, idx)
    assert np.array_equal(g_gate.view(np.uint32), gate.view(np.uint32))
    assert np.array_equal(g_counts, counts)


def test_select_large_batch():
    """T = 262,144 at the V3 router shape (the batch the selection is measured at): the GPU
    selection of the GPU logits against the oracle's selection of the same logits."""
    T = 262144
    w = workloads.get("v3-bf16", T=T)
    log(f"[select] large batch T={T} E={w.E} G={w.G} M={w.M} K={w.K} J={w.J}")
    wr, b = workloads.make_router(w, "cuda")
    x = workloads.make_x(w, device="cuda")
    g_idx, g_gate, g_counts, g_z = _route_gpu(T, w.H, w.E, w.G, w.M, w.K, w.J, x, wr, b)
    del x
    idx, gate, counts = oracle.select(g_z, workloads.to_numpy(b), w.G, w.M, w.K, w.J)
    assert np.array_equal(g_idx, idx)
    assert np.array_equal(g_gate.view(np.uint32), gate.view(np.uint32))
    assert np.array_equal(g_counts, counts)
    assert int(g_counts.sum()) == T * w.K
