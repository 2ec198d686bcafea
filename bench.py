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

--train times a training step of the layer instead: the forward keeping the gate/up
pre-activations (moe_expert_ffn_up_save), the bias update, then the backward
(moe_combine_backward -> moe_router_backward -> moe_expert_ffn_backward_input ->
moe_expert_ffn_backward_weight -> moe_unpermute_sum) for a seeded output gradient.
Its roofline is that of the weight-gradient GEMMs (fp32 gradient writes).

  python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload v3-bf16] [--train]
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
METRIC_TRAIN = ("MoE-layer training-step tokens/s (forward + bias update + backward; 7168d, "
                "256e top-8, T=4096)")
HBM_PEAK_GBS = 8000.0
# peak of the expert GEMMs' arithmetic, TFLOP/s: dense MFMA for bf16 and fp8; the fp32
# expert GEMM is a SIMT kernel, so its roof is the (non-packed) VALU rate
MFMA_PEAK = {"bf16": 2500.0, "e4m3": 5000.0, "f32": 78.6}
GEMM_BOUND = {"bf16": "mfma", "e4m3": "mfma", "f32": "alu"}
VALU_FP32_PEAK = 78.6  # TFLOP/s: 256 CUs x 4 SIMD x 16 lanes x 2 flop x 2.4 GHz (no packed fp32)
MFMA_FP32_PEAK = 157.3  # TFLOP/s, dense fp32 MFMA
# the library computes the router logits on the matrix cores (k=1 fp32 MFMA chains) from
# this many tokens, on the VALU below it (router.hip's dispatch rule)
ROUTER_MFMA_MIN_TOKENS = 2048


def router_roof(T):
    """(logits kernel, bound, peak TFLOP/s) of moe_route at T tokens."""
    if T >= ROUTER_MFMA_MIN_TOKENS:
        return "k_router_logits_mfma", "mfma", MFMA_FP32_PEAK
    return "k_router_logits", "alu", VALU_FP32_PEAK


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_sha(expert, train=False, packed=False):
    """sha256 over the sources that define the measured kernel: the gate/up GEMM of this
    expert dtype (bf16: over packed or natural-layout weights), or (train) the
    weight-gradient GEMM."""
    csrc = os.path.join(ROOT, "mixture_experts_layer_added_amd", "csrc")
    if train:
        files = ["gemm_bwd.hip", "common.h"]
    elif expert == "e4m3" and packed:  # the shared expert's dense FP8 kernel is in gemm_fp8
        files = ["gemm_packed_fp8.hip", "gemm_fp8.hip", "common.h"]
    elif expert == "e4m3":
        files = ["gemm_fp8.hip", "gemm_dense.hip", "common.h"]
    elif packed:
        files = ["gemm_packed.hip", "gemm_dense.hip", "common.h"]
    else:
        files = ["gemm.hip", "gemm_dense.hip", "common.h"]
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload, expert, dispatch, train=False, packed=False):
    """HBM bytes per launch of the measured kernel (gate/up GEMM, or with train the
    weight-gradient GEMM) from the committed FETCH_SIZE / WRITE_SIZE counter summary of
    this workload, or None when there is none or the kernel source has changed since
    the counters were taken."""
    kind = "ffn_bwd_weight" if train else "ffn_up"
    path = os.path.join(ROOT, "profiles", f"{kind}_{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return None, "no counter summary"
    with open(path) as fh:
        m = re.search(r"^traffic: (\{.*\})$", fh.read(), re.M)
    if not m:
        return None, "counter summary unreadable"
    rec = json.loads(m.group(1))
    if rec.get("source_sha256") != kernel_source_sha(expert, train, packed):
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
    ap.add_argument("--route-only", action="store_true",
                    help="time moe_route alone (router logits + group-limited top-K); with "
                         "--tokens it runs at batch sizes whose expert FFN buffers would not fit")
    ap.add_argument("--natural", action="store_true",
                    help="bf16 / FP8: run the expert GEMMs over the natural weight layout (the "
                         "LDS-ring kernels); default: packed up to 160 rows per expert on average")
    ap.add_argument("--packed", action="store_true",
                    help="bf16 / FP8: run the expert GEMMs over packed weights at any batch size")
    ap.add_argument("--train", action="store_true",
                    help="time forward + bias update + backward (bf16 / fp32 experts)")
    ap.add_argument("--cpu-ffn-rows", type=int, default=0,
                    help="expert-FFN rows the oracle computes for its sample "
                         "(default 2048; 256 with --train)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one device copy of this size (for counter calibration)")
    ap.add_argument("--load-log", default="",
                    help="after the timed region, run the workload's balancing loop (its "
                         "step count, fresh seeded tokens each step; 50 for v3-skew-loop) and "
                         "write one JSON line of load statistics per step to this file "
                         "('-' for stderr)")
    return ap.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1",
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
    if args.route_only:
        return route_only(args, w, dev)
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
    if args.train and w.expert == "e4m3":
        raise SystemExit("--train: the backward is built for the bf16 and fp32 expert paths")
    layer = MoELayer(shape, w_router, bias, w13, w2, s13, s2, device=dev,
                     gather=not args.materialize, train=args.train,
                     packed=False if args.natural else (True if args.packed else None))
    dy = workloads.make_dy(w, device=dev) if args.train else None
    stream = torch.cuda.current_stream()

    calls = [("route", lambda: layer.route(x)), ("permute", lambda: layer.permute(x)),
             ("ffn_up", layer.expert_ffn_up), ("ffn_down", layer.expert_ffn_down),
             ("combine", layer.combine), ("bias_update", lambda: layer.bias_step(w.gamma))]
    if args.train:
        calls += [("combine_bwd", lambda: layer.combine_backward(dy)),
                  ("router_bwd", layer.router_backward),
                  ("ffn_bwd_input", layer.expert_ffn_backward_input),
                  ("ffn_bwd_weight", layer.expert_ffn_backward_weight),
                  ("unpermute_sum", layer.unpermute_sum)]
    names = [n for n, _ in calls]

    def step(ev=None):
        for i, (_, call) in enumerate(calls):
            if ev is not None:
                ev[i].record(stream)
            call()
        if ev is not None:
            ev[len(calls)].record(stream)

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
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
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
    # activations: the dispatched rows (materialised: R rows of x_sorted; gathered: each
    # token's row once, its other reads hit the L2) and h written once
    x_rows = w.T if not args.materialize else R
    up_act = (x_rows * w.H * es + R * w.I * es +
              ((x_rows * (w.H // 128) + R * (w.I // 128)) * 4 if es == 1 else 0))
    up_bytes = up_w + up_scales + up_act
    if args.train:  # the gate/up pre-activations kept for the backward
        up_bytes += R * 2 * w.I * act_es
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

    frac_key = "mfma_frac" if GEMM_BOUND[w.expert] == "mfma" else "valu_frac"
    kernels = {
        "route": {"ms": avg_ms["route"], "TFLOP/s": tfs(route_flops, avg_ms["route"]),
                  "kernel": router_roof(w.T)[0], "bound": router_roof(w.T)[1],
                  "frac": tfs(route_flops, avg_ms["route"]) / router_roof(w.T)[2]},
        "permute": {"ms": avg_ms["permute"], "GB/s": gbs(perm_bytes, avg_ms["permute"]),
                    "hbm_frac": gbs(perm_bytes, avg_ms["permute"]) / HBM_PEAK_GBS},
        "ffn_up": {"ms": avg_ms["ffn_up"], "GB/s": gbs(up_bytes, avg_ms["ffn_up"]),
                   "hbm_frac": gbs(up_bytes, avg_ms["ffn_up"]) / HBM_PEAK_GBS,
                   "TFLOP/s": tfs(up_flops, avg_ms["ffn_up"]),
                   frac_key: tfs(up_flops, avg_ms["ffn_up"]) / MFMA_PEAK[w.expert]},
        "ffn_down": {"ms": avg_ms["ffn_down"], "GB/s": gbs(down_bytes, avg_ms["ffn_down"]),
                     "hbm_frac": gbs(down_bytes, avg_ms["ffn_down"]) / HBM_PEAK_GBS,
                     "TFLOP/s": tfs(down_flops, avg_ms["ffn_down"]),
                     frac_key: tfs(down_flops, avg_ms["ffn_down"]) / MFMA_PEAK[w.expert]},
        "combine": {"ms": avg_ms["combine"], "GB/s": gbs(comb_bytes, avg_ms["combine"]),
                    "hbm_frac": gbs(comb_bytes, avg_ms["combine"]) / HBM_PEAK_GBS},
        "bias_update": {"ms": avg_ms["bias_update"]},
    }
    if args.train:
        a, T, H, I, K, E = act_es, w.T, w.H, w.I, w.K, w.E
        NG = E + w.S
        cb_bytes = T * H * a + T * K * H * a + R * H * a + T * K * 12
        rb_bytes = T * K * 12 + 2 * E * H * 4 + T * H * 4 + T * K * H * a
        # dh GEMM: dY, au in, dau out; dx GEMM: dau in, dx_sorted out
        bi_bytes = (R * H * a + touched * H * I * es + R * 2 * I * a * 3
                    + touched * 2 * I * H * es + R * H * a)
        bi_flops = 2.0 * R * H * I + 2.0 * R * 2 * I * H
        x_rows = R if args.materialize else T
        # per launch: dW2 (dY, h in; NG x H x I fp32 out), dW13 (dau, x in; NG x 2I x H out)
        bw_bytes = (R * H * a + R * I * a + NG * H * I * 4
                    + R * 2 * I * a + x_rows * H * a + NG * 2 * I * H * 4)
        bw_flops = 2.0 * R * H * I + 2.0 * R * 2 * I * H
        us_bytes = R * H * a + T * H * 4 + T * H * a + T * K * 4
        for n, b, f in (("combine_bwd", cb_bytes, 0), ("router_bwd", rb_bytes, 0),
                        ("ffn_bwd_input", bi_bytes, bi_flops),
                        ("ffn_bwd_weight", bw_bytes, bw_flops), ("unpermute_sum", us_bytes, 0)):
            k = {"ms": avg_ms[n], "GB/s": gbs(b, avg_ms[n]),
                 "hbm_frac": gbs(b, avg_ms[n]) / HBM_PEAK_GBS}
            if f:
                k["TFLOP/s"] = tfs(f, avg_ms[n])
                k[frac_key] = tfs(f, avg_ms[n]) / MFMA_PEAK[w.expert]
            kernels[n] = k
    if args.train:
        # the weight-gradient call: two launches of k_gemm_tn_bf16 (dW2, then dW13);
        # per-launch figures are the averages over the two
        per_launch_ms = avg_ms["ffn_bwd_weight"] / 2
        wg_gbs = gbs(bw_bytes / 2, per_launch_ms)
        roofline = {"kernel": "k_gemm_tn_bf16 (expert weight gradients, fp32 out; 2 launches)"
                    if w.expert == "bf16" else "k_tn_f32 (expert weight gradients)",
                    "bound": "hbm", "achieved": round(wg_gbs, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(wg_gbs / HBM_PEAK_GBS, 4),
                    "bytes_per_launch": bw_bytes // 2, "ms_per_launch": round(per_launch_ms, 4),
                    "traffic": None}
    else:
        # the bound is the roof the call's arithmetic intensity meets first: HBM below the
        # ridge (peak flop/s over peak bytes/s), the matrix cores above it (a large batch
        # puts enough rows on every expert)
        up_gbs = gbs(up_bytes, avg_ms["ffn_up"])
        up_tfs = tfs(up_flops, avg_ms["ffn_up"])
        intensity = up_flops / up_bytes
        ridge = MFMA_PEAK[w.expert] * 1e12 / (HBM_PEAK_GBS * 1e9)
        gk = "k_gemm_packed<0>" if layer.packed else "k_gemm_bf16<true>"
        if w.expert == "bf16":
            up_name = (f"gate/up GEMM + SwiGLU call: {gk} (routed experts, grouped) + "
                       "k_gemm_dense_swiglu_bf16 (the shared expert, when T >= 2048)")
        elif w.expert == "e4m3":
            up_name = ("gate/up GEMM + SwiGLU call (e4m3): "
                       f"{'k_gemm_packed_fp8<true>' if layer.packed else 'k_gemm_fp8<true>'} "
                       "(routed experts, grouped) + k_gemm_dense_swiglu_fp8_w (the shared "
                       "expert, when T >= 2048; k_gemm_dense_swiglu_fp8 where the wide tiles "
                       "would not fill the chip)")
        else:
            up_name = "gate/up GEMM + SwiGLU call (fp32): k_gemm_f32<true> (every group)"
        roofline = {"kernel": up_name,
                    "bound": "hbm", "achieved": round(up_gbs, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(up_gbs / HBM_PEAK_GBS, 4),
                    "bytes_per_launch": up_bytes, "ms_per_launch": round(avg_ms["ffn_up"], 4),
                    "traffic": None, "intensity_flop_per_byte": round(intensity, 1),
                    "ridge_flop_per_byte": round(ridge, 1)}
        if intensity >= ridge:
            roofline.update({"bound": GEMM_BOUND[w.expert], "achieved": round(up_tfs, 1),
                             "peak": MFMA_PEAK[w.expert], "unit": "TFLOP/s",
                             "frac": round(up_tfs / MFMA_PEAK[w.expert], 4),
                             "flops_per_launch": up_flops})
    dispatch = "materialized x_sorted" if args.materialize else "gather from x"
    traffic, src = measured_traffic(w.name, w.expert, dispatch, args.train, layer.packed)
    if args.tokens and args.tokens != workloads.get(w.name).T:
        traffic, src = None, f"counters were taken at T={workloads.get(w.name).T}"
    roofline["traffic"] = traffic
    roofline["traffic_source"] = src
    roofline["kernel_source_sha256"] = kernel_source_sha(w.expert, args.train, layer.packed)
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20)
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        a.fill_(1)
        b.copy_(a)
        torch.cuda.synchronize()

    if args.load_log:
        load_log(args, w, layer, dev)

    cpu = None
    if not args.no_cpu_baseline:
        ffn_rows = args.cpu_ffn_rows or (256 if args.train else 2048)
        cpu = cpu_baseline(w, layer, x, w_router, bias,
                           w13 if w.expert != "e4m3" else (w13, s13, w2, s2), w2,
                           ffn_rows, dy if args.train else None)

    out = {
        "metric": METRIC_TRAIN if args.train else METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.expert, "data": "synthetic (seeded; weights N(0,0.006), x N(0,1))",
        "config": {"workload": w.name, "T": w.T, "H": w.H, "E": w.E, "G": w.G, "M": w.M,
                   "K": w.K, "J": w.J, "I": w.I, "S": w.S, "act": w.act, "expert": w.expert,
                   "dispatch": dispatch,
                   "weights": "packed" if layer.packed else "natural layout",
                   "step": "forward + bias update + backward"
                   if args.train else "forward + bias update",
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "experts_touched": touched,
    }
    print(json.dumps(out), flush=True)


def load_log(args, w, layer, dev):
    """The balancing loop with per-step load statistics (untimed): step s routes fresh
    seeded tokens (seed x + s) with the bias left by step s-1, then updates the bias.
    The statistics come from moe_seq_load_stats over the batch as one sequence (max,
    min, experts without tokens, max/mean), the bias range from the bias itself."""
    import numpy as np
    import torch

    import workloads
    from mixture_experts_layer_added_amd import _lib as L

    out = sys.stderr if args.load_log == "-" else open(args.load_log, "w")
    off = torch.tensor([0, w.T], dtype=torch.int32, device=dev)
    c = torch.empty((1, w.E), dtype=torch.int32, device=dev)
    st = torch.empty((1, 3), dtype=torch.int32, device=dev)
    r = torch.empty((1,), dtype=torch.float32, device=dev)
    b0 = layer.bias.clone()
    layer.bias.copy_(workloads.make_router(w, dev)[1])  # the loop starts from the initial bias
    for step in range(max(w.steps, 1)):
        x = workloads.make_x(w, step=step, device=dev)
        layer.forward(x)
        L.moe_seq_load_stats(layer.p, layer.topk_idx, off, 1, c, st, r)
        layer.bias_step(w.gamma)
        s3 = st.cpu().numpy()[0]
        b = layer.bias.cpu().numpy()
        counts = np.sort(c.cpu().numpy()[0])[::-1]
        out.write(json.dumps({"step": step, "max_over_mean": round(float(r.item()), 4),
                              "max_load": int(s3[0]), "min_load": int(s3[1]),
                              "zero_load_experts": int(s3[2]),
                              "top16_share": round(float(counts[:16].sum() / counts.sum()), 4),
                              "bias_min": float(b.min()), "bias_max": float(b.max())}) + "\n")
    out.flush()
    if out is not sys.stderr:
        out.close()
    layer.bias.copy_(b0)


def route_only(args, w, dev):
    """moe_route alone: logits (fp32 sequential fma chains, on the matrix cores from 2048
    tokens) then the selection kernel."""
    import torch

    import workloads
    from mixture_experts_layer_added_amd import _lib as L

    w_router, bias = workloads.make_router(w, dev)
    x = workloads.make_x(w, device=dev)
    p = L.problem(w.T, w.H, w.E, w.G, w.M, w.K, w.J, w.I, w.S,
                  L.MOE_BF16 if w.act == "bf16" else L.MOE_F32,
                  L.MOE_BF16 if w.act == "bf16" else L.MOE_F32)
    idx = torch.empty((w.T, w.K), dtype=torch.int32, device=dev)
    gate = torch.empty((w.T, w.K), dtype=torch.float32, device=dev)
    counts = torch.empty((w.E,), dtype=torch.int32, device=dev)
    logits = torch.empty((w.T, w.E), dtype=torch.float32, device=dev)
    n = L.moe_workspace_bytes(p, L.MOE_CALL_ROUTE)
    ws = torch.empty((max(n, 256),), dtype=torch.uint8, device=dev)

    def step():
        L.moe_route(p, x, w_router, bias, idx, gate, counts, logits, ws, ws.numel())

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = elapsed * 1e3 / args.steps
    flops = 2.0 * w.T * w.E * w.H
    tfs = flops / (ms * 1e-3) / 1e12
    a = 2 if w.act == "bf16" else 4
    rk, rbound, rpeak = router_roof(w.T)
    out = {
        "metric": "MoE router tokens/s (route only: fp32 logits + group-limited top-K)",
        "value": round(w.T * args.steps / elapsed, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded; x N(0,1), router weight N(0,0.02))",
        "config": {"workload": w.name, "T": w.T, "H": w.H, "E": w.E, "G": w.G, "M": w.M,
                   "K": w.K, "J": w.J, "act": w.act, "step": "route only",
                   "parallelism": "single GPU"},
        # the whole call is timed; the logits kernel dominates it
        "roofline": {"kernel": f"moe_route ({rk} dominates)", "bound": rbound,
                     "achieved": round(tfs, 2), "peak": rpeak, "unit": "TFLOP/s",
                     "frac": round(tfs / rpeak, 4), "traffic": None},
        "cpu_baseline": None,
        # algorithmic bytes of the selection kernel (logits row + bias in, indices and
        # gates out); its duration comes from a kernel trace of this run
        "select_bytes": w.T * (w.E * 4 + w.K * 8) + 2 * w.E * 4,
        "logits_bytes": w.T * w.H * a + w.E * w.H * 4 + w.T * w.E * 4,
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(w, layer, x, w_router, bias, w13, w2, ffn_rows, dy=None):
    """The CPU oracle on a bounded sample of the same workload: routing, permutation,
    combine and bias update of the whole batch, and the expert FFN on `ffn_rows`
    rows (half from the first routed experts, half from the shared expert), whose
    per-row time is scaled to the T*(K+1) rows of the batch.  With dy (training step)
    also the combine, router and unpermute backward of the whole batch and the expert
    backward of the same sample rows, scaled the same way."""
    import numpy as np

    import oracle
    import workloads

    threads = oracle.default_threads()
    xn = workloads.to_numpy(x)
    wr = workloads.to_numpy(w_router)
    bn = workloads.to_numpy(bias)
    fp8 = w.expert == "e4m3"
    log(f"[bench] cpu baseline: oracle on {threads} threads")
    t = time.perf_counter()
    idx, gate, counts, z = oracle.route(xn, wr, bn, w.G, w.M, w.K, w.J, nthreads=threads,
                                        want_logits=dy is not None)
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
    what = (f"route+permute+combine+bias of all {w.T} tokens; expert FFN on {n_rows} rows "
            f"({experts})")
    if dy is not None:
        dyn = workloads.to_numpy(dy)
        t = time.perf_counter()
        dys, dg = oracle.combine_backward(dyn, ys, inv, gate, w.S, nthreads=threads)
        dz, dxr, _ = oracle.router_backward(xn, wr, z, idx, gate, dg, nthreads=threads)
        t_bwd_rest = time.perf_counter() - t
        t_eb_sample = 0.0
        for g, rows in sample:
            a, b = workloads.to_numpy(w13[g]), workloads.to_numpy(w2[g])
            t = time.perf_counter()
            oracle.expert_backward(xs[rows], a, b, dys[rows], nthreads=threads)
            t_eb_sample += time.perf_counter() - t
        t = time.perf_counter()
        oracle.unpermute_sum(ys, inv, dxr, w.T, w.S, nthreads=threads)
        t_bwd_rest += time.perf_counter() - t
        total += t_bwd_rest + t_eb_sample * (w.R / n_rows)
        measured += t_bwd_rest + t_eb_sample
        log(f"[bench] cpu baseline: backward (combine, router, unpermute) {t_bwd_rest:.2f}s, "
            f"expert backward sample {t_eb_sample:.2f}s")
        what = (f"forward, bias update and combine/router/unpermute backward of all {w.T} "
                f"tokens; expert FFN forward and backward on {n_rows} rows ({experts})")
    return {"value": round(w.T / total, 3), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": (f"{what} scaled to the {w.R} rows of the batch; {measured:.1f}s measured"),
            "seconds_per_step_extrapolated": round(total, 2)}


if __name__ == "__main__":
    main()
