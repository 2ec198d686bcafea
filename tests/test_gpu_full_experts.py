"""Element-by-element parity of whole experts at the full DeepSeek-V3 layer shape
(hidden 7168, 256 routed experts + 1 shared, top-8, SwiGLU width 2048), in the launch
configuration the benchmark times (gathered dispatch).

For the most loaded routed expert and one expert of 129..160 rows (the grouped GEMMs'
largest three-stage ring in bf16, the two-row-group path in FP8), every row and every
column of h (the gate/up output as stored between the GEMMs) and of Y is compared with
the oracle run on the same rows.  The shared expert's gate/up runs as its own dense
launch at this batch size; its rows are checked on every 16th token in bf16 (every
64th in FP8, whose oracle is slower), which puts sampled rows in every row tile of
that launch while every column of every tile is compared.  For bf16 the expert
backward's input part ([da|du] and dx_sorted) of the same experts is compared too,
from the GPU's own dY rows (pinned by the backward tests).

Bounds: bf16 2e-2 and FP8 1e-2 normwise on Y and dx/[da|du] (the benchmark spec's expert-output
tolerances); FP8 h is compared as codes: the scales within 1e-4 relative, and codes
that differ (the fp32 sums sit on the other side of a rounding boundary of the
oracle's fp64 sums) at most one E4M3 step plus 1/16 apart in units of the scale, and
at most 1% of them.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_cases import TOL, as_f64, log, rel_err, shape_of

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


def rows_of(t, rows):
    return np_(t[torch.from_numpy(np.asarray(rows, np.int64)).cuda()])


def _layer(w, train=False):
    from mixture_experts_layer_added_amd.layer import MoELayer, quantize_weights_fp8
    dev = torch.device("cuda")
    wr, b = workloads.make_router(w, dev)
    w13, w2 = workloads.make_experts(w, dev)
    if w.expert == "e4m3":
        q13, s13 = quantize_weights_fp8(w13)
        q2, s2 = quantize_weights_fp8(w2)
        return MoELayer(shape_of(w), wr, b, q13, q2, s13, s2, gather=True), (w13, w2)
    return MoELayer(shape_of(w), wr, b, w13, w2, gather=True, train=train), (w13, w2)


def _routing(w, layer, x):
    """Oracle routing and permutation of the whole batch; the GPU's must be identical."""
    xn = np_(x)
    idx, gate, counts, _ = oracle.route(xn, np_(layer.w_router), np_(layer.bias), w.G, w.M, w.K,
                                        w.J)
    assert np.array_equal(np_(layer.topk_idx), idx)
    assert np.array_equal(np_(layer.counts), counts)
    off, st, inv, xs, xsc = oracle.permute(xn, idx, counts, w.E, w.S,
                                           out_dtype=oracle.E4M3 if w.expert == "e4m3" else None)
    assert np.array_equal(np_(layer.offsets), off)
    assert np.array_equal(np_(layer.sorted_token), st)
    return counts, off, xs, xsc


def _pick(counts):
    """(most loaded expert, an expert with 129..160 rows -- the most loaded such)"""
    e_max = int(np.argmax(counts))
    mids = [e for e in range(len(counts)) if 129 <= counts[e] <= 160 and e != e_max]
    assert mids, "no expert with 129..160 rows in this batch"
    return e_max, max(mids, key=lambda e: counts[e])


def _fp8_h_check(hq_g, hs_g, hq_r, hs_r, tag):
    """FP8 h: scales (amax/448 of fp32 sums vs the oracle's rounded fp64 sums) within
    1e-4 relative; the decoded codes (h / scale) differ by at most one E4M3 step at the
    larger magnitude plus 1/16 (an absolute difference of 1.4e-4 of the tile's amax,
    which the fp32 sums can move the small values near zero by), and differ in at most
    1% of all codes."""
    assert np.all(np.abs(hs_g.astype(np.float64) - hs_r) <= np.abs(hs_r) * 1e-4), tag
    dg = torch.from_numpy(np.ascontiguousarray(hq_g)).view(torch.float8_e4m3fn).double().numpy()
    dr = torch.from_numpy(np.ascontiguousarray(hq_r)).view(torch.float8_e4m3fn).double().numpy()
    mag = np.maximum(np.abs(dg), np.abs(dr))
    step = np.where(mag >= 2.0 ** -6,
                    2.0 ** (np.floor(np.log2(np.maximum(mag, 2.0 ** -6))) - 3), 2.0 ** -9)
    bad = np.abs(dg - dr) > step + 2.0 ** -4
    if bad.any():
        r, c = np.nonzero(bad)
        worst = [(int(a), int(b), float(dg[a, b]), float(dr[a, b])) for a, b in zip(r[:5], c[:5])]
        raise AssertionError(f"{tag}: {int(bad.sum())} codes beyond the bound; (row, col, gpu, "
                             f"oracle): {worst}")
    frac = float((hq_g != hq_r).mean())
    assert frac <= 0.01, (tag, frac)
    return frac


@pytest.mark.parametrize("name", ["v3-bf16", "v3-fp8"])
def test_whole_experts_forward(name):
    w = workloads.get(name)
    fp8 = w.expert == "e4m3"
    log(f"[whole experts] {name}: T={w.T} H={w.H} E={w.E}+{w.S} K={w.K} I={w.I}, gathered")
    layer, (w13b, w2b) = _layer(w)
    x = workloads.make_x(w, device="cuda")
    layer.forward(x)
    torch.cuda.synchronize()
    counts, off, xs, xsc = _routing(w, layer, x)
    e_max, e_mid = _pick(counts)
    step = 64 if fp8 else 16
    shared_rows = w.T * w.K + np.arange(0, w.T, step)
    cases = [(f"expert {e_max} ({counts[e_max]} rows, most loaded)", e_max,
              np.arange(off[e_max], off[e_max + 1])),
             (f"expert {e_mid} ({counts[e_mid]} rows)", e_mid, np.arange(off[e_mid], off[e_mid + 1])),
             (f"shared expert, every {step}th of {w.T} rows", w.E, shared_rows)]
    out_dt = oracle.BF16
    for tag, g, rows in cases:
        if fp8:
            a, sa = oracle.quantize_weight_fp8(np_(w13b[g]))
            b, sb = oracle.quantize_weight_fp8(np_(w2b[g]))
            assert np.array_equal(np_(layer.w13[g]), a) and np.array_equal(np_(layer.w2[g]), b)
            y_r, h_r, hs_r = oracle.expert_ffn(xs[rows], a, b, out_dt, xsc[rows], sa, sb,
                                               want_h=True)
        else:
            y_r, h_r, hs_r = oracle.expert_ffn(xs[rows], np_(layer.w13[g]), np_(layer.w2[g]),
                                               out_dt, want_h=True)
        y_g = rows_of(layer.y_sorted, rows)
        ey = rel_err(as_f64(y_g, w.act), as_f64(y_r, w.act))
        if fp8:
            frac = _fp8_h_check(rows_of(layer.h, rows), rows_of(layer.h_scale, rows), h_r, hs_r,
                                tag)
            log(f"    {tag}: Y rel err {ey:.3e} over {len(rows)}x{w.H}; h codes differ at "
                f"{frac:.2e} of {len(rows)}x{w.I}")
        else:
            eh = rel_err(as_f64(rows_of(layer.h, rows), w.act), as_f64(h_r, w.act))
            log(f"    {tag}: h rel err {eh:.3e} over {len(rows)}x{w.I}, Y rel err {ey:.3e} "
                f"over {len(rows)}x{w.H}")
            assert eh <= TOL[w.expert], tag
        assert ey <= TOL[w.expert], tag
    del layer
    torch.cuda.empty_cache()


def test_whole_experts_backward_input():
    """The expert backward's input part ([da|du] and dx_sorted) of the same experts at
    the V3 bf16 shape, from the GPU's dY rows and the oracle's dispatched x rows."""
    w = workloads.get("v3-bf16")
    log(f"[whole experts, backward input part] T={w.T} H={w.H} E={w.E}+{w.S} I={w.I}")
    layer, _ = _layer(w, train=True)
    x = workloads.make_x(w, device="cuda")
    layer.forward(x)
    dy = workloads.make_dy(w, device="cuda")
    layer.backward(dy)
    torch.cuda.synchronize()
    counts, off, xs, _ = _routing(w, layer, x)
    e_max, e_mid = _pick(counts)
    shared_rows = w.T * w.K + np.arange(0, w.T, 64)
    cases = [(f"expert {e_max} ({counts[e_max]} rows)", e_max, np.arange(off[e_max], off[e_max + 1])),
             (f"expert {e_mid} ({counts[e_mid]} rows)", e_mid, np.arange(off[e_mid], off[e_mid + 1])),
             (f"shared expert, every 64th of {w.T} rows", w.E, shared_rows)]
    for tag, g, rows in cases:
        dys = rows_of(layer.dy_sorted, rows)
        _, dau_r, dx_r, _, _ = oracle.expert_backward(xs[rows], np_(layer.w13[g]),
                                                      np_(layer.w2[g]), dys, weights=False)
        e1 = rel_err(as_f64(rows_of(layer.dau, rows), w.act), as_f64(dau_r, w.act))
        e2 = rel_err(as_f64(rows_of(layer.dx_sorted, rows), w.act), as_f64(dx_r, w.act))
        log(f"    {tag}: [da|du] rel err {e1:.3e} over {len(rows)}x{2 * w.I}, dx_sorted rel err "
            f"{e2:.3e} over {len(rows)}x{w.H}")
        assert e1 <= TOL[w.expert] and e2 <= TOL[w.expert], tag
    del layer
    torch.cuda.empty_cache()


def test_shared_expert_fp8_tile_forms_agree():
    """The shared expert's FP8 gate/up has two dense forms: 256-row tiles when every CU
    gets one (T=4096 at the V3 shape), 128-row tiles below.  A shared row depends only
    on its own token (its per-token activation scales included), so the h codes and
    scales of tokens 0..2047 at T=4096 must equal those at T=2048 with the same first
    2048 tokens, bit for bit: the two forms promote the same per-block partial sums with
    the same scale products in the same order."""
    w4 = workloads.get("v3-fp8")
    w2k = workloads.get("v3-fp8", T=2048)
    tiles_wide = ((w4.T + 255) // 256) * (w4.I // 128)
    tiles_small = ((w2k.T + 255) // 256) * (w2k.I // 128)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    log(f"[shared fp8 forms] 256-row tiles at T={w4.T}: {tiles_wide}, at T={w2k.T}: "
        f"{tiles_small} (the wide form needs >= {cus})")
    if not tiles_small < cus <= tiles_wide:
        pytest.skip(f"{cus} CUs: the two batch sizes do not select the two tile forms")
    from mixture_experts_layer_added_amd.layer import MoELayer, quantize_weights_fp8
    dev = torch.device("cuda")
    wr, b = workloads.make_router(w4, dev)
    w13, w2 = workloads.make_experts(w4, dev)
    q13, s13 = quantize_weights_fp8(w13)
    q2, s2 = quantize_weights_fp8(w2)
    del w13, w2
    x = workloads.make_x(w4, device=dev)
    hs = []
    for w, xx in ((w4, x), (w2k, x[:w2k.T].contiguous())):
        layer = MoELayer(shape_of(w), wr, b, q13, q2, s13, s2, gather=True)
        layer.route(xx)
        layer.permute(xx)
        layer.expert_ffn_up()
        torch.cuda.synchronize()
        r0 = w.T * w.K
        hs.append((np_(layer.h[r0:r0 + w2k.T]), np_(layer.h_scale[r0:r0 + w2k.T])))
        del layer
        torch.cuda.empty_cache()
    assert np.array_equal(hs[0][0], hs[1][0])
    assert np.array_equal(hs[0][1].view(np.uint32), hs[1][1].view(np.uint32))
    log(f"    h codes [{w2k.T} x {w4.I}] and scales of the shared expert: bit-identical")
