"""The expert GEMMs over packed weights (moe_pack_expert_weights,
moe_expert_ffn_up_packed, moe_expert_ffn_down_packed), bf16 and FP8.

- The packed layout is checked bit for bit against a numpy statement of it (the
  layout is documented in include/moe.h's terms: blocks of 64 weight rows, 64-deep k
  steps, 8 instructions x 64 lanes x 8 elements).
- The packed kernels multiply the same 16-deep k slices in the same order as the
  natural-layout kernels, so h, the pre-activations and y_sorted must be bit-identical
  to the natural-layout calls (which are pinned to the oracle): on small shapes that
  reach every row-subtile count, the shared expert's dense launch, the materialised and
  gathered forms and the pre-activation store, and on the whole DeepSeek-V3 layer at
  T=4096 (experts of 73..193 rows) and on the skewed T=8192 batch (experts of several
  hundred rows, split into 192-row tiles).
The FP8 kernels promote the same per-block partial sums (two 64-deep MFMAs per
128-deep scale block) with the same scale product as the natural-layout FP8 kernels,
so their h codes, h scales and Y must also equal those bit for bit.
The oracle comparison of the packed path itself is test_gpu_parity's expert FFN test.
"""
import numpy as np
import pytest

import workloads
from gpu_cases import case, log, make_cpu_inputs, shape_of

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


def pack13_np(w13, I, H):
    NG = w13.shape[0]
    a = w13.reshape(NG, 2, I // 32, 32, H // 64, 4, 2, 8)   # g n b c kt s h e
    return np.ascontiguousarray(a.transpose(0, 2, 4, 1, 5, 6, 3, 7)).reshape(w13.shape)


def pack2_np(w2, I, H):
    NG = w2.shape[0]
    a = w2.reshape(NG, H // 64, 2, 32, I // 64, 4, 2, 8)     # g b n c kt s h e
    return np.ascontiguousarray(a.transpose(0, 1, 4, 2, 5, 6, 3, 7)).reshape(w2.shape)


@pytest.mark.parametrize("H,I,E,S", [(384, 256, 3, 1), (256, 128, 5, 0), (128, 384, 2, 1)])
def test_pack_layout_bitexact(H, I, E, S):
    from mixture_experts_layer_added_amd import _lib as L
    rng = np.random.default_rng(H + I + E)
    NG = E + S
    w13 = rng.integers(0, 1 << 16, size=(NG, 2 * I, H), dtype=np.uint16)
    w2 = rng.integers(0, 1 << 16, size=(NG, H, I), dtype=np.uint16)
    d13 = torch.from_numpy(w13.view(np.int16)).cuda()
    d2 = torch.from_numpy(w2.view(np.int16)).cuda()
    p13, p2 = torch.full_like(d13, -1), torch.full_like(d2, -1)
    p = L.problem(64, H, E, 1, 1, 1, 1, I, S, L.MOE_BF16, L.MOE_BF16)
    L.moe_pack_expert_weights(p, d13, d2, p13, p2)
    torch.cuda.synchronize()
    assert np.array_equal(p13.cpu().numpy().view(np.uint16), pack13_np(w13, I, H))
    assert np.array_equal(p2.cpu().numpy().view(np.uint16), pack2_np(w2, I, H))
    # one matrix alone
    p2b = torch.full_like(d2, -1)
    L.moe_pack_expert_weights(p, None, d2, None, p2b)
    torch.cuda.synchronize()
    assert np.array_equal(p2b.cpu().numpy().view(np.uint16), pack2_np(w2, I, H))


def pack13_fp8_np(w13, I, H):
    NG = w13.shape[0]
    a = w13.reshape(NG, 2, I // 32, 32, H // 128, 2, 2, 2, 16)   # g n b c kt u h v e
    return np.ascontiguousarray(a.transpose(0, 2, 4, 1, 5, 7, 6, 3, 8)).reshape(w13.shape)


def pack2_fp8_np(w2, I, H):
    NG = w2.shape[0]
    a = w2.reshape(NG, H // 64, 2, 32, I // 128, 2, 2, 2, 16)     # g b n c kt u h v e
    return np.ascontiguousarray(a.transpose(0, 1, 4, 2, 5, 7, 6, 3, 8)).reshape(w2.shape)


@pytest.mark.parametrize("H,I,E,S", [(384, 256, 3, 1), (128, 384, 2, 0)])
def test_pack_layout_fp8_bitexact(H, I, E, S):
    from mixture_experts_layer_added_amd import _lib as L
    rng = np.random.default_rng(7 * H + I)
    NG = E + S
    w13 = rng.integers(0, 256, size=(NG, 2 * I, H), dtype=np.uint8)
    w2 = rng.integers(0, 256, size=(NG, H, I), dtype=np.uint8)
    d13, d2 = torch.from_numpy(w13).cuda(), torch.from_numpy(w2).cuda()
    p13, p2 = torch.zeros_like(d13), torch.zeros_like(d2)
    p = L.problem(64, H, E, 1, 1, 1, 1, I, S, L.MOE_BF16, L.MOE_FP8_E4M3)
    L.moe_pack_expert_weights(p, d13, d2, p13, p2)
    torch.cuda.synchronize()
    assert np.array_equal(p13.cpu().numpy(), pack13_fp8_np(w13, I, H))
    assert np.array_equal(p2.cpu().numpy(), pack2_fp8_np(w2, I, H))


def _pair(w, wr, b, w13, w2, gather, train, s13=None, s2=None):
    from mixture_experts_layer_added_amd.layer import MoELayer
    sh = shape_of(w)
    return (MoELayer(sh, wr, b, w13, w2, s13, s2, gather=gather, train=train, packed=True),
            MoELayer(sh, wr, b, w13, w2, s13, s2, gather=gather, train=train, packed=False))


def _same(a, b, tag):
    ea, eb = np_(a), np_(b)
    if not np.array_equal(ea, eb):
        bad = np.argwhere(ea != eb)
        raise AssertionError(f"{tag}: {len(bad)} elements differ, first at {bad[:3].tolist()}")


def _compare(w, x, pk, nat, tag):
    for layer in (pk, nat):
        layer.route(x)
        layer.permute(x)
        layer.expert_ffn()
    torch.cuda.synchronize()
    _same(pk.h, nat.h, tag + " h")
    if pk.h_scale is not None:
        _same(pk.h_scale, nat.h_scale, tag + " h_scale")
    _same(pk.y_sorted, nat.y_sorted, tag + " y_sorted")
    if pk.train:
        _same(pk.au, nat.au, tag + " au")


@pytest.mark.parametrize("name", ["ragged-bf16", "rows150-bf16", "v3route-bf16", "noshared-bf16",
                                  "k1-j1-bf16", "maxE-bf16", "dense-bf16"])
@pytest.mark.parametrize("gather,train", [(True, False), (False, False), (True, True)])
def test_packed_equals_natural_small(name, gather, train):
    w = case(name)
    inp = make_cpu_inputs(w)
    dev = lambda t: t.contiguous().cuda()  # noqa: E731
    pk, nat = _pair(w, dev(inp["w_router"]), dev(inp["bias"]), dev(inp["w13"]), dev(inp["w2"]),
                    gather, train)
    _compare(w, dev(inp["x"]), pk, nat, f"{name} gather={gather} train={train}")
    counts = np_(pk.counts)
    log(f"    {name} gather={gather} train={train}: bit-identical; rows per expert "
        f"{counts.min()}..{counts.max()}")


@pytest.mark.parametrize("name,T", [("v3-bf16", 4096), ("v3-skew-loop", 8192)])
def test_packed_equals_natural_v3(name, T):
    w = workloads.get(name, T=T)
    dev = torch.device("cuda")
    wr, b = workloads.make_router(w, dev)
    w13, w2 = workloads.make_experts(w, dev)
    x = workloads.make_x(w, device=dev)
    pk, nat = _pair(w, wr, b, w13, w2, True, False)
    _compare(w, x, pk, nat, name)
    counts = np_(pk.counts)
    log(f"[packed vs natural] {name} T={T}: h [{w.R}x{w.I}] and y_sorted [{w.R}x{w.H}] "
        f"bit-identical; rows per expert {counts.min()}..{counts.max()}")
    del pk, nat
    torch.cuda.empty_cache()


def _fp8_weights(w13, w2):
    from mixture_experts_layer_added_amd.layer import quantize_weights_fp8
    q13, s13 = quantize_weights_fp8(w13)
    q2, s2 = quantize_weights_fp8(w2)
    return q13, q2, s13, s2


@pytest.mark.parametrize("name", ["ragged-fp8", "dense-fp8", "v3route-fp8"])
@pytest.mark.parametrize("gather", [True, False])
def test_packed_equals_natural_fp8_small(name, gather):
    w = case(name)
    inp = make_cpu_inputs(w)
    dev = lambda t: t.contiguous().cuda()  # noqa: E731
    q13, q2, s13, s2 = _fp8_weights(dev(inp["w13"]), dev(inp["w2"]))
    pk, nat = _pair(w, dev(inp["w_router"]), dev(inp["bias"]), q13, q2, gather, False, s13, s2)
    _compare(w, dev(inp["x"]), pk, nat, f"{name} gather={gather}")
    counts = np_(pk.counts)
    log(f"    {name} gather={gather}: bit-identical; rows per expert "
        f"{counts.min()}..{counts.max()}")


def test_packed_equals_natural_fp8_v3():
    w = workloads.get("v3-fp8")
    dev = torch.device("cuda")
    wr, b = workloads.make_router(w, dev)
    w13, w2 = workloads.make_experts(w, dev)
    q13, q2, s13, s2 = _fp8_weights(w13, w2)
    del w13, w2
    x = workloads.make_x(w, device=dev)
    pk, nat = _pair(w, wr, b, q13, q2, True, False, s13, s2)
    _compare(w, x, pk, nat, "v3-fp8")
    counts = np_(pk.counts)
    log(f"[packed vs natural] v3-fp8 T={w.T}: h codes, h scales and y_sorted bit-identical; "
        f"rows per expert {counts.min()}..{counts.max()}")
    del pk, nat
    torch.cuda.empty_cache()


def packT_np(w):
    """Packed layout of the transposes W[g]^T for W [NG, Kd, Nout]: the down layout with
    Nout rows and k over Kd (moe_pack_expert_weights_transposed)."""
    t = np.ascontiguousarray(w.transpose(0, 2, 1))   # [NG, Nout, Kd]
    return pack2_np(t, t.shape[2], t.shape[1])


@pytest.mark.parametrize("H,I,E,S", [(384, 256, 3, 1), (256, 128, 5, 0)])
def test_pack_transposed_layout_bitexact(H, I, E, S):
    from mixture_experts_layer_added_amd import _lib as L
    rng = np.random.default_rng(3 * H + I + E)
    NG = E + S
    w13 = rng.integers(0, 1 << 16, size=(NG, 2 * I, H), dtype=np.uint16)
    w2 = rng.integers(0, 1 << 16, size=(NG, H, I), dtype=np.uint16)
    d13 = torch.from_numpy(w13.view(np.int16)).cuda()
    d2 = torch.from_numpy(w2.view(np.int16)).cuda()
    p13, p2 = torch.full_like(d13, -1), torch.full_like(d2, -1)
    p = L.problem(64, H, E, 1, 1, 1, 1, I, S, L.MOE_BF16, L.MOE_BF16)
    L.moe_pack_expert_weights_transposed(p, d13, d2, p13, p2)
    torch.cuda.synchronize()
    assert np.array_equal(p13.cpu().numpy().view(np.uint16).reshape(NG, H, 2 * I),
                          packT_np(w13).reshape(NG, H, 2 * I))
    assert np.array_equal(p2.cpu().numpy().view(np.uint16).reshape(NG, I, H),
                          packT_np(w2).reshape(NG, I, H))


def _bwd_compare(w, x, wr, b, w13, w2, dy, tag):
    """The backward input part over packed transposed weights against the natural-layout
    kernels on the same forward: [da|du] and dx_sorted bit-identical."""
    from mixture_experts_layer_added_amd.layer import MoELayer
    sh = shape_of(w)
    pk = MoELayer(sh, wr, b, w13, w2, gather=True, train=True, packed=True)
    nat = MoELayer(sh, wr, b, w13, w2, gather=True, train=True, packed=False)
    assert pk.w13tp is not None and nat.w13tp is None
    for layer in (pk, nat):
        layer.forward(x)
        layer.combine_backward(dy)
        layer.expert_ffn_backward_input()
    torch.cuda.synchronize()
    _same(pk.dau, nat.dau, tag + " [da|du]")
    _same(pk.dx_sorted, nat.dx_sorted, tag + " dx_sorted")
    counts = np_(pk.counts)
    return counts


@pytest.mark.parametrize("name", ["ragged-bf16", "rows150-bf16", "v3route-bf16", "noshared-bf16",
                                  "dense-bf16"])
def test_packed_backward_input_equals_natural_small(name):
    w = case(name)
    inp = make_cpu_inputs(w)
    dev = lambda t: t.contiguous().cuda()  # noqa: E731
    g = torch.Generator().manual_seed(11)
    dy = torch.randn((w.T, w.H), generator=g).to(torch.bfloat16)
    counts = _bwd_compare(w, dev(inp["x"]), dev(inp["w_router"]), dev(inp["bias"]),
                          dev(inp["w13"]), dev(inp["w2"]), dev(dy), name)
    log(f"    {name}: backward input part bit-identical; rows per expert "
        f"{counts.min()}..{counts.max()}")


def test_packed_backward_input_equals_natural_v3():
    w = workloads.get("v3-bf16")
    dev = torch.device("cuda")
    wr, b = workloads.make_router(w, dev)
    w13, w2 = workloads.make_experts(w, dev)
    x = workloads.make_x(w, device=dev)
    g = torch.Generator(device=dev).manual_seed(5)
    dy = torch.randn((w.T, w.H), generator=g, device=dev).to(torch.bfloat16)
    counts = _bwd_compare(w, x, wr, b, w13, w2, dy, "v3-bf16")
    log(f"[packed backward vs natural] v3-bf16 T={w.T}: [da|du] [{w.R}x{2 * w.I}] and "
        f"dx_sorted [{w.R}x{w.H}] bit-identical; rows per expert {counts.min()}..{counts.max()}")
    torch.cuda.empty_cache()
