#!/usr/bin/env python3
"""Benchmark of the MoE layer forward + aux-loss-free bias update on one MI355X.

One step = moe_route -> moe_permute -> moe_expert_ffn_up -> moe_expert_ffn_down ->
moe_combine -> moe_bias_update on one stream, over one resident batch of the
workload (default: the DeepSeek-V3-shaped bf16 layer, T=4096 tokens, hidden 7168,
256 routed experts + 1 shared, top-8 of 8 groups with at most 4 per token, SwiGLU
width 2048).  Inputs are seeded synthetic tensors already in HBM.

Prints ONE JSON line: throughput (tokens/s), the roofline of the dominant kernel
(the gate/up grouped GEMM, timed with HIP events on its launch stream) and the CPU
oracle timed on a bounded sample of the same workload.

  python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload v3-bf16]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s (7168d, 256e top-8, T=4096); MFMA % and HBM % of peak"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK = {"bf16": 2500.0, "e4m3": 5000.0, "f32": 157.3}  # dense TFLOP/s
VALU_FP32_PEAK = 78.6  # TFLOP/s: 256 CUs x 4 SIMD x 16 lanes x 2 flop x 2.4 GHz (no packed fp32)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_sha(expert):
    """sha256 over the sources that define the gate/up GEMM of this expert dtype."""
    csrc = os.path.join(ROOT, "mixture_experts_layer_added_amd", "csrc")
    files = ["gemm_fp8.hip" if expert == "e4m3" else "gemm.hip", "common.h"]
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload, expert, dispatch):
    """HBM bytes per gate/up launch from the committed FETCH_SIZE / WRITE_SIZE counter
    summary of this workload, or None when there is none or the kernel source has changed
    since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"ffn_up_{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return None, "no counter summary"
    with open(path) as fh:
        m = re.search(r"^traffic: (\{.*\})$", fh.read(), re.M)
    if not m:
        return None, "counter summary unreadable"
    rec = json.loads(m.group(1))
    if rec.get("source_sha256") != kernel_source_sha(expert):
        return None, "kernel changed since the counters were taken"
    if rec.get("dispatch") != dispatch:
        return None, f"counters were taken with dispatch '{rec.get('dispatch')}'"
    return int(rec["fetch_bytes"] + rec["write_bytes"]), path[len(ROOT) + 1:]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="v3-bf16")
    ap.add_argument("--tokens", type=int, default=0, help="override T of the workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--materialize", action="store_true",
                    help="permute writes x_sorted and the gate/up GEMM reads it (default: the "
                         "GEMM gathers its rows from x)")
    ap.add_argument("--cpu-ffn-rows", type=int, default=2048,
                    help="expert-FFN rows the oracle computes for its sample")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one device copy of this size (for counter calibration)")
    return ap.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import workloads
    from mixture_experts_layer_added_amd import _lib as L
    from mixture_experts_layer_added_amd.layer import MoELayer, Shape, quantize_weights_fp8

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs an MI355X GPU")
    L.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    w = workloads.get(args.workload)
    if args.tokens:
        w = workloads.get(args.workload, T=args.tokens)
    log(f"[bench] workload {w.name} T={w.T} H={w.H} E={w.E} K={w.K} I={w.I} expert={w.expert}")

    t0 = time.time()
    w_router, bias = workloads.make_router(w, dev)
    w13, w2 = workloads.make_experts(w, dev)
    x = workloads.make_x(w, device=dev)
    s13 = s2 = None
    if w.expert == "e4m3":
        q13, s13 = quantize_weights_fp8(w13)
        q2, s2 = quantize_weights_fp8(w2)
        w13_bf16, w2_bf16 = w13, w2
        w13, w2 = q13, q2
    torch.cuda.synchronize()
    log(f"[bench] inputs ready in {time.time() - t0:.1f}s")
    shape = Shape(T=w.T, H=w.H, E=w.E, G=w.G, M=w.M, K=w.K, J=w.J, I=w.I, S=w.S, act=w.act,
                  expert=w.expert)
    layer = MoELayer(shape, w_router, bias, w13, w2, s13, s2, device=dev,
                     gather=not args.materialize)
    stream = torch.cuda.current_stream()

    names = ["route", "permute", "ffn_up", "ffn_down", "combine", "bias_update"]

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        layer.route(x)
        if ev is not None:
            ev[1].record(stream)
        layer.permute(x)
        if ev is not None:
            ev[2].record(stream)
        layer.expert_ffn_up()
        if ev is not None:
            ev[3].record(stream)
        layer.expert_ffn_down()
        if ev is not None:
            ev[4].record(stream)
        layer.combine()
        if ev is not None:
            ev[5].record(stream)
        layer.bias_step(w.gamma)
        if ev is not None:
            ev[6].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly K steps, synchronised on both sides
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms_per_step = elapsed * 1e3 / args.steps
    tokens_per_s = w.T * args.steps / elapsed

    # per-kernel durations with HIP events on the launch stream (separate pass so the
    # event records do not perturb the timed region above)
    per = {n: [] for n in names}
    for _ in range(args.steps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(7)]
        step(ev)
        torch.cuda.synchronize()
        for i, n in enumerate(names):
            per[n].append(ev[i].elapsed_time(ev[i + 1]))
    avg_ms = {n: float(np.mean(v)) for n, v in per.items()}

    counts = workloads.to_numpy(layer.counts)
    touched = int((counts > 0).sum()) + w.S
    es = {"bf16": 2, "f32": 4, "e4m3": 1}[w.expert]
    act_es = 2 if w.act == "bf16" else 4
    R = w.R
    # algorithmic bytes and flops per launch (each touched expert's weights read once,
    # activations read and written once)
    up_w = touched * 2 * w.I * w.H * es
    up_scales = touched * (2 * w.I // 128) * (w.H // 128) * 4 if w.expert == "e4m3" else 0
    up_act = R * w.H * es + R * w.I * es + (R * (w.H // 128 + w.I // 128) * 4 if es == 1 else 0)
    up_bytes = up_w + up_scales + up_act
    up_flops = 2.0 * R * 2 * w.I * w.H
    down_w = touched * w.H * w.I * es
    down_bytes = down_w + R * w.I * es + R * w.H * act_es
    down_flops = 2.0 * R * w.I * w.H
    route_flops = 2.0 * w.T * w.E * w.H
    route_bytes = w.T * w.H * act_es + w.E * w.H * 4 + w.T * w.E * 4 * 2 + w.T * w.K * 8
    if args.materialize:
        perm_bytes = w.T * w.H * act_es + R * w.H * es + w.T * w.K * 4 * 3 + R * 4
    else:  # index maps (+ FP8: one quantisation of x per token)
        perm_bytes = w.T * w.K * 4 * 3 + R * 4
        if w.expert == "e4m3":
            perm_bytes += w.T * w.H * (act_es + 1) + w.T * (w.H // 128) * 4
    comb_bytes = R * w.H * act_es + w.T * w.H * act_es + w.T * w.K * 8

    def gbs(b, ms):
        return b / (ms * 1e-3) / 1e9

    def tfs(f, ms):
        return f / (ms * 1e-3) / 1e12

    kernels = {
        "route": {"ms": avg_ms["route"], "TFLOP/s": tfs(route_flops, avg_ms["route"]),
                  "valu_frac": tfs(route_flops, avg_ms["route"]) / VALU_FP32_PEAK},
        "permute": {"ms": avg_ms["permute"], "GB/s": gbs(perm_bytes, avg_ms["permute"]),
                    "hbm_frac": gbs(perm_bytes, avg_ms["permute"]) / HBM_PEAK_GBS},
        "ffn_up": {"ms": avg_ms["ffn_up"], "GB/s": gbs(up_bytes, avg_ms["ffn_up"]),
                   "hbm_frac": gbs(up_bytes, avg_ms["ffn_up"]) / HBM_PEAK_GBS,
                   "TFLOP/s": tfs(up_flops, avg_ms["ffn_up"]),
                   "mfma_frac": tfs(up_flops, avg_ms["ffn_up"]) / MFMA_PEAK[w.expert]},
        "ffn_down": {"ms": avg_ms["ffn_down"], "GB/s": gbs(down_bytes, avg_ms["ffn_down"]),
                     "hbm_frac": gbs(down_bytes, avg_ms["ffn_down"]) / HBM_PEAK_GBS,
                     "TFLOP/s": tfs(down_flops, avg_ms["ffn_down"]),
                     "mfma_frac": tfs(down_flops, avg_ms["ffn_down"]) / MFMA_PEAK[w.expert]},
        "combine": {"ms": avg_ms["combine"], "GB/s": gbs(comb_bytes, avg_ms["combine"]),
                    "hbm_frac": gbs(comb_bytes, avg_ms["combine"]) / HBM_PEAK_GBS},
        "bias_update": {"ms": avg_ms["bias_update"]},
    }
    up_gbs = gbs(up_bytes, avg_ms["ffn_up"])
    roofline = {"kernel": "k_gemm_bf16<true> (gate/up grouped GEMM + SwiGLU)"
                if w.expert == "bf16" else f"gate/up grouped GEMM ({w.expert})",
                "bound": "hbm", "achieved": round(up_gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(up_gbs / HBM_PEAK_GBS, 4),
                "bytes_per_launch": up_bytes, "ms_per_launch": round(avg_ms["ffn_up"], 4),
                "traffic": None}
    dispatch = "materialized x_sorted" if args.materialize else "gather from x"
    traffic, src = measured_traffic(w.name, w.expert, dispatch)
    roofline["traffic"] = traffic
    roofline["traffic_source"] = src
    roofline["kernel_source_sha256"] = kernel_source_sha(w.expert)
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20)
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        a.fill_(1)
        b.copy_(a)
        torch.cuda.synchronize()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, layer, x, w_router, bias,
                           w13 if w.expert != "e4m3" else (w13, s13, w2, s2), w2,
                           args.cpu_ffn_rows)

    out = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.expert, "data": "synthetic (seeded; weights N(0,0.006), x N(0,1))",
        "config": {"workload": w.name, "T": w.T, "H": w.H, "E": w.E, "G": w.G, "M": w.M,
                   "K": w.K, "J": w.J, "I": w.I, "S": w.S, "act": w.act, "expert": w.expert,
                   "dispatch": dispatch,
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "experts_touched": touched,
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(w, layer, x, w_router, bias, w13, w2, ffn_rows):
    """The CPU oracle on a bounded sample of the same workload: routing, permutation,
    combine and bias update of the whole batch, and the expert FFN on `ffn_rows`
    rows (half from the first routed expert, half from the shared expert), whose
    per-row time is scaled to the T*(K+1) rows of the batch."""
    import concurrent.futures as cf

    import numpy as np
    import torch

    import oracle
    import workloads

    threads = oracle.default_threads()
    xn = workloads.to_numpy(x)
    wr = workloads.to_numpy(w_router)
    bn = workloads.to_numpy(bias)
    fp8 = w.expert == "e4m3"
    log(f"[bench] cpu baseline: oracle on {threads} threads")
    t = time.perf_counter()
    idx, gate, counts, _ = oracle.route(xn, wr, bn, w.G, w.M, w.K, w.J, nthreads=threads)
    t_route = time.perf_counter() - t
    t = time.perf_counter()
    off, st, inv, xs, xsc = oracle.permute(xn, idx, counts, w.E, w.S,
                                           out_dtype=oracle.E4M3 if fp8 else None)
    t_perm = time.perf_counter() - t
    # FFN sample: ffn_rows/2 routed rows (whole experts, in index order) and ffn_rows/2
    # rows of the shared expert
    half = ffn_rows // 2
    sample = []
    taken = 0
    for g in range(w.E):
        if taken >= half:
            break
        n = min(int(off[g + 1] - off[g]), half - taken)
        if n > 0:
            sample.append((g, np.arange(off[g], off[g] + n)))
            taken += n
    if w.S:
        n_shared = min(half, w.T)
        sample.append((w.E, np.arange(off[w.E], off[w.E] + n_shared)))
    out_dt = oracle.BF16 if w.act == "bf16" else oracle.F32
    t_ffn_sample = 0.0
    n_rows = 0
    for g, rows in sample:
        if fp8:
            q13, s13, q2, s2 = w13
            a, sa, b, sb = (workloads.to_numpy(q13[g]), workloads.to_numpy(s13[g]),
                            workloads.to_numpy(q2[g]), workloads.to_numpy(s2[g]))
            t = time.perf_counter()
            oracle.expert_ffn(xs[rows], a, b, out_dt, xsc[rows], sa, sb, nthreads=threads)
        else:
            a, b = workloads.to_numpy(w13[g]), workloads.to_numpy(w2[g])
            t = time.perf_counter()
            oracle.expert_ffn(xs[rows], a, b, out_dt, nthreads=threads)
        t_ffn_sample += time.perf_counter() - t
        n_rows += len(rows)
    routed = [g for g, _ in sample if g < w.E]
    experts = f"experts {routed[0]}..{routed[-1]}" + (" and the shared expert" if w.S else "")
    t_ffn = t_ffn_sample * (w.R / n_rows)
    ys = workloads.to_numpy(workloads.make_y_sorted(w, seed=9, device=x.device))
    t = time.perf_counter()
    oracle.combine(ys, inv, gate, w.T, w.S, nthreads=threads)
    t_comb = time.perf_counter() - t
    t = time.perf_counter()
    oracle.bias_update(counts, w.T, w.K, w.gamma, bn)
    t_bias = time.perf_counter() - t
    total = t_route + t_perm + t_ffn + t_comb + t_bias
    measured = t_route + t_perm + t_ffn_sample + t_comb + t_bias
    log(f"[bench] cpu baseline: route {t_route:.2f}s permute {t_perm:.2f}s ffn sample "
        f"{t_ffn_sample:.2f}s ({n_rows} rows) combine {t_comb:.2f}s")
    return {"value": round(w.T / total, 3), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": (f"route+permute+combine+bias of all {w.T} tokens; expert FFN on "
                       f"{n_rows} rows ({experts}) scaled to the "
                       f"{w.R} rows of the batch; {measured:.1f}s measured"),
            "seconds_per_step_extrapolated": round(total, 2)}


if __name__ == "__main__":
    main()
