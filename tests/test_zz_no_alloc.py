"""moe_permute_noalloc (the permute with its scratch in a fixed device array inside the
library) against moe_permute on the same inputs, through the C ABI: every output bit
for bit, on two calls in a row with the second problem smaller than the first (the
array keeps the first call's contents), in the index-only, materialised bf16 and
materialised FP8 forms."""
import numpy as np
import pytest

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


def _routing(w, seed):
    """Indices from moe_route on seeded inputs (the permutation's input)."""
    from mixture_experts_layer_added_amd import _lib as L
    dev = torch.device("cuda")
    wr, b = workloads.make_router(w, dev)
    x = workloads.make_x(w, step=seed, device=dev)
    p = L.problem(w.T, w.H, w.E, w.G, w.M, w.K, w.J, w.I, w.S,
                  L.MOE_BF16 if w.act == "bf16" else L.MOE_F32,
                  {"f32": L.MOE_F32, "bf16": L.MOE_BF16, "e4m3": L.MOE_FP8_E4M3}[w.expert])
    idx = torch.empty((w.T, w.K), dtype=torch.int32, device=dev)
    gate = torch.empty((w.T, w.K), dtype=torch.float32, device=dev)
    counts = torch.empty((w.E,), dtype=torch.int32, device=dev)
    logits = torch.empty((w.T, w.E), dtype=torch.float32, device=dev)
    L.moe_route(p, x, wr, b, idx, gate, counts, logits)
    return p, x, idx


def _outputs(w, form, dev):
    i32 = dict(dtype=torch.int32, device=dev)
    out = dict(offsets=torch.full((w.E + w.S + 1,), -7, **i32),
               sorted_token=torch.full((w.R,), -7, **i32),
               inv_perm=torch.full((w.T, w.K), -7, **i32), x_sorted=None, scale=None)
    if form == "bf16":
        out["x_sorted"] = torch.zeros((w.R, w.H), dtype=torch.bfloat16, device=dev)
    elif form == "fp8":
        out["x_sorted"] = torch.zeros((w.R, w.H), dtype=torch.uint8, device=dev)
        out["scale"] = torch.zeros((w.R, w.H // 128), dtype=torch.float32, device=dev)
    return out


def _run(w, form, seed):
    from mixture_experts_layer_added_amd import _lib as L
    dev = torch.device("cuda")
    p, x, idx = _routing(w, seed)
    ref, got = _outputs(w, form, dev), _outputs(w, form, dev)
    n = L.moe_workspace_bytes(p, L.MOE_CALL_PERMUTE)
    ws = torch.empty((n,), dtype=torch.uint8, device=dev)
    L.moe_permute(p, x, idx, ref["offsets"], ref["sorted_token"], ref["inv_perm"],
                  ref["x_sorted"], ref["scale"], ws, n)
    L.moe_permute_noalloc(p, x, idx, got["offsets"], got["sorted_token"], got["inv_perm"],
                          got["x_sorted"], got["scale"])
    torch.cuda.synchronize()
    for k in ("offsets", "sorted_token", "inv_perm", "x_sorted", "scale"):
        if ref[k] is None:
            continue
        a, b = ref[k].cpu(), got[k].cpu()
        if a.dtype == torch.bfloat16:
            a, b = a.view(torch.int16), b.view(torch.int16)
        if a.dtype == torch.float32:
            a, b = a.view(torch.int32), b.view(torch.int32)
        assert torch.equal(a, b), (w.T, form, k)
    return int(ref["offsets"][-1].item())


@pytest.mark.parametrize("form", ["index", "bf16", "fp8"])
def test_noalloc_permute_matches_workspace_permute(form):
    base = "v3-fp8" if form == "fp8" else "v3-bf16"
    # first call: 8192 tokens at the V3 routing shape; second: a smaller batch with fewer
    # experts, so the array still holds the larger call's ranks and block counts
    big = workloads.get(base, T=8192, H=256, I=128)
    small = workloads.get(base, T=777, H=384, E=64, G=8, M=4, K=6, J=2, I=128)
    for w, seed in ((big, 11), (small, 12)):
        rows = _run(w, form, seed)
        log(f"    {form}: T={w.T} E={w.E} K={w.K}: {rows} rows bit-identical to moe_permute")
