"""Benchmark of the block-scaled FP8 MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode|prefill|longctx|r3|tiny|payload]
                    [--scales amax|pow2] [--weights fp8|fp4] [--backward]

A step is one full layer forward (gate logits, routing, activation quantisation, dispatch,
grouped GEMM1 + SwiGLU + h quantisation, grouped GEMM2, combine) over one batch of synthetic
tokens whose inputs and quantised weights are already resident in HBM.  The default workload is
the decode-shaped layer (256 tokens, hidden 4096, 64 experts, FFN 1408, top-6).  Consecutive steps
cycle through several copies of the layer (weights packed for the grouped GEMM, plus buffers), at
least 2 GiB of weights in all, as consecutive layers of a model would: a step never finds its
weights in the 256 MB Infinity Cache left behind by the step before.  The reported rate times
replays of a HIP graph holding the whole layer forward (--no-graph: eager launches); a second
pass of eager steps with HIP events between the stages gives the per-stage times.  Prints one JSON
line: layer tokens/s, per-stage times, the grouped GEMM's TFLOP/s, the roofline of the dominant
kernel, and the CPU oracle timed on a bounded sample.  With --backward a step is the layer's training
forward (GEMM1 also keeps its fp32 output) followed by its backward (output gradient -> dx, dWg,
db), and the line reports the backward's stages too.  --weights fp4 runs the same forward with FP4
expert weights (E2M1 in 1x32 blocks with E8M0 scales; activations stay FP8 with power-of-two scales).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_FP8_TFLOPS = 5000.0       # dense fp8 MFMA (published, no sparsity)
PEAK_FP32_TFLOPS = 157.3       # published fp32 vector peak (a non-packed fma loop reaches 110 on the box)
RIDGE_FP8 = PEAK_FP8_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)

STAGES = ["gate_logits", "route", "quant_x", "dispatch", "gemm1_swiglu", "gemm2", "combine"]
BWD_STAGES = ["bwd_combine", "bwd_gemm_dh", "bwd_gemm_g", "bwd_swiglu", "bwd_gemm_da", "bwd_combine_dx", "bwd_route",
              "bwd_gate"]
WGRAD_STAGES = ["bwd_wgrad_quant", "bwd_wgrad_gemm"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of HIP graph replays")
    ap.add_argument("--copies", type=int, default=0,
                    help="layer copies cycled through by consecutive steps (0: enough for 2 GiB of weights, >= 2)")
    ap.add_argument("--scales", choices=("amax", "pow2"), default="amax",
                    help="block-scale form: amax/448 fp32 scales (default) or power-of-two scales applied by "
                         "the matrix cores")
    ap.add_argument("--weights", choices=("fp8", "fp4"), default="fp8",
                    help="expert weight format: fp8 e4m3 in 128x128 blocks, or fp4 e2m1 in 1x32 blocks with E8M0 "
                         "scales (forward only; implies power-of-two activation scales)")
    ap.add_argument("--backward", action="store_true",
                    help="time forward + backward of the layer (gradients of x, the gate and its bias)")
    ap.add_argument("--weight-grads", action="store_true",
                    help="with --backward: also the expert-weight gradients dW1, dW2 (fp32)")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB (counter calibration)")
    return ap.parse_args()


def stage_model(cfg, counts, n_active1, fp4=False):
    """Algorithmic bytes and flops of each stage (inputs read once, outputs written once).  Expert
    weight bytes per element: 1 + 4/128^2 for e4m3 with 128x128 fp32 scales, 1/2 + 1/32 for FP4
    with one E8M0 byte per 1x32 block."""
    T, H, E, F, k = cfg.T, cfg.H, cfg.E, cfg.F, cfg.k
    ab = 4 if cfg.act == "f32" else 2
    sig = 4.0 / 128
    rows = int(sum(counts))
    G = cfg.groups
    act_groups = n_active1
    wb = (0.5 + 1.0 / 32) if fp4 else (1 + 4.0 / (128 * 128))
    w1 = act_groups * (2 * F * H) * wb
    w2 = act_groups * (H * F) * wb
    return {
        "gate_logits": dict(bytes=T * H * ab + E * H * 4 + T * E * 4, flops=2.0 * T * H * E, bound="alu"),
        "route": dict(bytes=T * E * 4 + T * k * 8, flops=0.0, bound="hbm"),
        "quant_x": dict(bytes=T * H * (ab + 1 + sig), flops=0.0, bound="hbm"),
        # ids in, dest_row and src_token out, the 1x128 scales permuted (GEMM1 gathers the codes)
        "dispatch": dict(bytes=T * k * 4 + T * k * 4 + rows * 4 + T * H * sig + rows * H * sig,
                         flops=0.0, bound="hbm"),
        "gemm1_swiglu": dict(bytes=rows * H * (1 + sig) + w1 + rows * F * (1 + sig), flops=4.0 * H * F * rows,
                             bound=None),
        "gemm2": dict(bytes=rows * F * (1 + sig) + w2 + rows * H * ab, flops=2.0 * H * F * rows, bound=None),
        "combine": dict(bytes=rows * H * ab + T * k * 8 + T * H * ab, flops=0.0, bound="hbm"),
        # backward (dY, dG quantised 1x128; dh, G, dA fp32; the router and gate in fp32)
        "bwd_combine": dict(bytes=T * H * ab + rows * H * ab + rows * H * (1 + sig) + T * k * 12, flops=0.0,
                            bound="hbm"),
        "bwd_gemm_dh": dict(bytes=rows * H * (1 + sig) + w2 + rows * F * 4, flops=2.0 * H * F * rows, bound=None),
        "bwd_gemm_g": dict(bytes=rows * H * (1 + sig) + w1 + rows * 2 * F * 4, flops=4.0 * H * F * rows, bound=None),
        "bwd_swiglu": dict(bytes=rows * F * 4 + rows * 2 * F * 4 + rows * 2 * F * (1 + sig), flops=0.0, bound="hbm"),
        "bwd_gemm_da": dict(bytes=rows * 2 * F * (1 + sig) + w1 + rows * H * 4, flops=4.0 * H * F * rows, bound=None),
        "bwd_combine_dx": dict(bytes=rows * H * 4 + T * k * 8 + T * H * 4, flops=0.0, bound="hbm"),
        "bwd_route": dict(bytes=T * E * 8 + T * k * 8, flops=0.0, bound="hbm"),
        "bwd_gate": dict(bytes=T * E * 4 + T * H * ab + E * H * 4 + T * H * 4 + T * H * ab + E * H * 4,
                         flops=4.0 * T * H * E, bound="alu"),
        # weight gradients: 128x1 operands (dY, x gathered; h, dG from G and dh), then fp32 dW1, dW2
        "bwd_wgrad_quant": dict(bytes=rows * (2 * H * ab + 2 * 8 * F + 4 * F) + rows * (2 * H + 3 * F) * (1 + sig),
                                flops=0.0, bound="hbm"),
        "bwd_wgrad_gemm": dict(bytes=rows * (2 * H + 3 * F) + act_groups * 3 * H * F * 4, flops=6.0 * H * F * rows,
                               bound=None),
        "_rows": rows, "_groups": G,
    }


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {a.gpus}): the layer's multi-GPU form (expert "
              "parallel dispatch/combine over xGMI) is not part of this build.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import block_scaled_fp8_top_amd as M
    import synth
    from dataclasses import replace

    from block_scaled_fp8_top_amd.layer import (MoELayer, MoELayerWeights, pack_expert_weights, quantize_expert_weights,
                                                quantize_expert_weights_fp4)

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    M.lib()  # fail loudly if the HIP library is missing
    dev = "cuda"
    if a.workload == "payload":
        payload_bench(a)
        return
    cfg = synth.CONFIGS[a.workload]
    sf = 0 if cfg.score_fn == "softmax" else 1
    rcfg = M.router_cfg(cfg.E, cfg.k, sf, cfg.renorm, cfg.n_group, cfg.topk_group, cfg.group_score_topk)
    wg, b = synth.make_gate(cfg, 0, dev)
    fp4 = a.weights == "fp4"
    if fp4 and a.backward:
        print("--weights fp4 is a forward-only format (no backward)", file=sys.stderr)
        sys.exit(2)
    pow2 = a.scales == "pow2" or fp4
    bwd_weights = None
    if fp4:
        w1p, w2p = quantize_expert_weights_fp4(cfg.groups, cfg.H, cfg.F, lambda g: synth.make_expert(cfg, g, 0, dev),
                                               device=dev)
        weights = MoELayerWeights(wg=wg, bias=b, w1q=None, w1s=None, w2q=None, w2s=None, cfg=rcfg, shared=cfg.shared,
                                  w1p=w1p, w2p=w2p, pow2=True)
        del w1p, w2p
    else:
        w1q, w1s, w2q, w2s = quantize_expert_weights(cfg.groups, cfg.H, cfg.F,
                                                     lambda g: synth.make_expert(cfg, g, 0, dev), device=dev, pow2=pow2)
        weights = pack_expert_weights(MoELayerWeights(wg=wg, bias=b, w1q=w1q, w1s=w1s, w2q=w2q, w2s=w2s, cfg=rcfg,
                                                      shared=cfg.shared, pow2=pow2), keep_rowmajor=a.backward)
        if a.backward:
            from block_scaled_fp8_top_amd.layer import prepare_backward_weights
            bwd_weights = prepare_backward_weights(weights)
            weights = replace(weights, w1q=None, w2q=None)
        del w1q, w2q
    wbytes = weights.w1p.data.numel() + weights.w2p.data.numel()
    copies = a.copies if a.copies > 0 else max(2, math.ceil((2 << 30) / wbytes))
    act = torch.bfloat16 if cfg.act == "bf16" else torch.float32
    layers = [MoELayer(weights, cfg.T, act, dev)]
    for _ in range(1, copies):
        if fp4:
            wc = replace(weights, w1p=replace(weights.w1p, data=weights.w1p.data.clone(),
                                              scales=weights.w1p.scales.clone()),
                         w2p=replace(weights.w2p, data=weights.w2p.data.clone(), scales=weights.w2p.scales.clone()))
        else:
            wc = replace(weights, w1p=replace(weights.w1p, data=weights.w1p.data.clone()),
                         w2p=replace(weights.w2p, data=weights.w2p.data.clone()), w1s=weights.w1s.clone(),
                         w2s=weights.w2s.clone())
        layers.append(MoELayer(wc, cfg.T, act, dev))
    layer = layers[0]
    x = synth.make_x(cfg, dev)
    torch.cuda.synchronize()
    if a.backward:
        backward_bench(a, cfg, layers, bwd_weights, x, copies, pow2)
        return

    for s in range(a.warmup):
        layers[s % copies].forward(x)
    torch.cuda.synchronize()
    K = a.steps

    # ---- timed region 1 (the reported rate): K steps, each one replay of a HIP graph holding the
    # whole layer forward (the launch sequence of a decode loop, without per-kernel launch gaps)
    graphs = None
    if not a.no_graph:
        graphs = []
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for c in range(copies):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=side):
                    layers[c].forward(x)
                graphs.append(g)
        torch.cuda.current_stream().wait_stream(side)
        for s in range(a.warmup):
            graphs[s % copies].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(K):
            graphs[s % copies].replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        graph_ms = (t1 - t0) * 1e3 / K

    # ---- timed region 2: K eager steps with HIP events between the stages on the launch stream
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(STAGES) + 1)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        layers[s % copies].forward(x, events=ev[s])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    eager_ms = (t1 - t0) * 1e3 / K
    ms_per_step = eager_ms if graphs is None else graph_ms
    stage_ms = {name: float(np.mean([ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(K)]))
                for i, name in enumerate(STAGES)}

    counts = layer.disp.counts.cpu().numpy()
    n_active = int((counts > 0).sum())
    model = stage_model(cfg, counts, n_active, fp4)
    stages = {}
    for name in STAGES:
        m = model[name]
        t = stage_ms[name] * 1e-3
        d = {"ms": round(stage_ms[name], 4), "GB_s": round(m["bytes"] / t / 1e9, 1)}
        if m["flops"]:
            d["TFLOP_s"] = round(m["flops"] / t / 1e12, 2)
        if name.startswith("gemm"):
            intensity = m["flops"] / m["bytes"]
            d["bound"] = "mfma" if intensity >= RIDGE_FP8 else "hbm"
            d["frac"] = round((m["flops"] / t / 1e12 / PEAK_FP8_TFLOPS) if d["bound"] == "mfma"
                              else (m["bytes"] / t / 1e9 / PEAK_HBM_GBS), 4)
        elif m["bound"] == "alu":
            d["bound"] = "alu"
            d["frac"] = round(m["flops"] / t / 1e12 / PEAK_FP32_TFLOPS, 4)
        else:
            d["bound"] = "hbm"
            d["frac"] = round(m["bytes"] / t / 1e9 / PEAK_HBM_GBS, 4)
        stages[name] = d

    gemm_ms = stage_ms["gemm1_swiglu"] + stage_ms["gemm2"]
    gemm_flops = model["gemm1_swiglu"]["flops"] + model["gemm2"]["flops"]
    gemm_tflops = gemm_flops / (gemm_ms * 1e-3) / 1e12
    dom = max(STAGES, key=lambda n: stage_ms[n])
    dm = model[dom]
    dt = stage_ms[dom] * 1e-3
    bound = stages[dom]["bound"]
    if bound == "mfma":
        roof = {"bound": "mfma", "achieved": round(dm["flops"] / dt / 1e12, 2), "peak": PEAK_FP8_TFLOPS,
                "unit": "TFLOP/s"}
    elif bound == "alu":
        roof = {"bound": "alu", "achieved": round(dm["flops"] / dt / 1e12, 2), "peak": PEAK_FP32_TFLOPS,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(dm["bytes"] / dt / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    kname = stage_kernel(dom, layer)
    roof["traffic"] = measured_traffic(kname, cfg.name)
    roof["kernel"] = kname
    roof["stage"] = dom

    if a.copy_probe_mb:
        n = a.copy_probe_mb * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()

    cpu = None
    if not a.no_cpu_baseline:
        cpu = cpu_baseline(cfg, x, dev, pow2, fp4)

    tokens_per_s = cfg.T / (ms_per_step * 1e-3)
    line = {
        "metric": "MoE layer tokens/s + grouped FP8 GEMM TFLOP/s (% of fp8 MFMA peak), 1 GPU",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "launch": "eager" if graphs is None else "hip-graph replay",
        "eager_ms_per_step": round(eager_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp4-e2m1 weights x fp8-e4m3" if fp4 else "fp8-e4m3 x fp8-e4m3") + " -> fp32 (GEMM); fp32 router; "
                 + ("bf16" if cfg.act == "bf16" else "fp32") + " activations",
        "data": "synthetic (seeded N(0,1) activations, N(0,1/sqrt(fan_in)) weights, random-init)",
        "config": {"workload": cfg.name, "tokens": cfg.T, "hidden": cfg.H, "experts": cfg.E,
                   "shared_experts": int(cfg.shared), "ffn": cfg.F, "top_k": cfg.k, "score": cfg.score_fn,
                   "rows": model["_rows"], "active_experts": n_active, "layer_copies": copies,
                   "weight_layout": "packed", "block_scales": "power of two" if pow2 else "amax/448 fp32",
                   "expert_weights": "fp4 e2m1, 1x32 e8m0 scales" if fp4 else "fp8 e4m3, 128x128 scales",
                   "parallelism": "none (1 GPU)"},
        "gemm_tflops": round(gemm_tflops, 2),
        "gemm_frac_fp8_peak": round(gemm_tflops / PEAK_FP8_TFLOPS, 4),
        "stages": stages,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


GEMM_SRC = os.path.join(ROOT, "block_scaled_fp8_top_amd", "csrc", "grouped_gemm.hip")


def stage_entry(name, model, ms):
    """Achieved rates of one stage and its roofline fraction."""
    m = model[name]
    t = ms * 1e-3
    d = {"ms": round(ms, 4), "GB_s": round(m["bytes"] / t / 1e9, 1)}
    if m["flops"]:
        d["TFLOP_s"] = round(m["flops"] / t / 1e12, 2)
    if m["bound"] is None:
        d["bound"] = "mfma" if m["flops"] / m["bytes"] >= RIDGE_FP8 else "hbm"
    else:
        d["bound"] = m["bound"]
    if d["bound"] == "mfma":
        d["frac"] = round(m["flops"] / t / 1e12 / PEAK_FP8_TFLOPS, 4)
    elif d["bound"] == "alu":
        d["frac"] = round(m["flops"] / t / 1e12 / PEAK_FP32_TFLOPS, 4)
    else:
        d["frac"] = round(m["bytes"] / t / 1e9 / PEAK_HBM_GBS, 4)
    return d


def backward_bench(a, cfg, layers, bw, x, copies, pow2):
    """Forward + backward steps: HIP-graph replays of both for the rate, then eager steps with
    events between every stage of each pass."""
    import numpy as np
    import torch

    import synth

    dev = "cuda"
    dout = synth.make_dout(cfg, dev)
    for s in range(a.warmup):
        layers[s % copies].forward(x, training=True)
        layers[s % copies].backward(x, dout, bw, weight_grads=a.weight_grads)
    torch.cuda.synchronize()
    K = a.steps
    graphs = None
    if not a.no_graph:
        graphs = []
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for c in range(copies):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=side):
                    layers[c].forward(x, training=True)
                    layers[c].backward(x, dout, bw, weight_grads=a.weight_grads)
                graphs.append(g)
        torch.cuda.current_stream().wait_stream(side)
        for s in range(a.warmup):
            graphs[s % copies].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(K):
            graphs[s % copies].replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t0) * 1e3 / K
    evf = [[torch.cuda.Event(enable_timing=True) for _ in range(len(STAGES) + 1)] for _ in range(K)]
    bst = BWD_STAGES + (WGRAD_STAGES if a.weight_grads else [])
    evb = [[torch.cuda.Event(enable_timing=True) for _ in range(len(bst) + 1)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        layers[s % copies].forward(x, events=evf[s], training=True)
        layers[s % copies].backward(x, dout, bw, events=evb[s], weight_grads=a.weight_grads)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / K
    ms_per_step = eager_ms if graphs is None else graph_ms
    stage_ms = {name: float(np.mean([evf[s][i].elapsed_time(evf[s][i + 1]) for s in range(K)]))
                for i, name in enumerate(STAGES)}
    stage_ms.update({name: float(np.mean([evb[s][i].elapsed_time(evb[s][i + 1]) for s in range(K)]))
                     for i, name in enumerate(bst)})
    layer = layers[0]
    counts = layer.disp.counts.cpu().numpy()
    n_active = int((counts > 0).sum())
    model = stage_model(cfg, counts, n_active)
    # the training forward's GEMM1 also writes G (fp32); the backward then has no recompute
    g1 = model["gemm1_swiglu"]
    model["gemm1_swiglu"] = dict(g1, bytes=g1["bytes"] + model["_rows"] * 2 * cfg.F * 4)
    timed = [n for n in STAGES + bst if n != "bwd_gemm_g"]   # no recompute after a training forward
    stages = {name: stage_entry(name, model, stage_ms[name]) for name in timed}
    fwd_ms = sum(stage_ms[n] for n in STAGES)
    bwd_ms = sum(stage_ms[n] for n in bst)
    gemm_names = [n for n in ("bwd_gemm_dh", "bwd_gemm_g", "bwd_gemm_da") if n in stages]
    bgemm_ms = sum(stage_ms[n] for n in gemm_names)
    bgemm_tflops = sum(model[n]["flops"] for n in gemm_names) / (bgemm_ms * 1e-3) / 1e12
    dom = max((n for n in bst if n in stages), key=lambda n: stage_ms[n])
    e = stages[dom]
    if e["bound"] == "hbm":
        roof = {"bound": "hbm", "achieved": e["GB_s"], "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": e["bound"], "achieved": e["TFLOP_s"],
                "peak": PEAK_FP8_TFLOPS if e["bound"] == "mfma" else PEAK_FP32_TFLOPS, "unit": "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = None
    p2 = ", pow2" if pow2 else ""
    if dom == "bwd_wgrad_gemm":
        roof["kernel"] = f"wgrad_gemm_kernel<{'pow2' if pow2 else 'amax'}>"
    else:
        roof["kernel"] = f"grouped_gemm_kernel<{layer.plan.tile_rows}, store_f32, packed{p2}>" if "gemm" in dom else dom
    roof["stage"] = dom
    cpu = None if a.no_cpu_baseline else cpu_baseline_backward(cfg, x, dout, dev, pow2)
    line = {
        "metric": "MoE layer forward+backward tokens/s + backward grouped FP8 GEMM TFLOP/s, 1 GPU",
        "value": round(cfg.T / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": a.warmup, "ms_per_step": round(ms_per_step, 4),
        "launch": "eager" if graphs is None else "hip-graph replay", "eager_ms_per_step": round(eager_ms, 4),
        "forward_ms": round(fwd_ms, 4), "backward_ms": round(bwd_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8-e4m3 x fp8-e4m3 -> fp32 (GEMMs, forward and backward); fp32 router and gate; "
                 + ("bf16" if cfg.act == "bf16" else "fp32") + " activations and gradients",
        "data": "synthetic (seeded N(0,1) activations and output gradient, N(0,1/sqrt(fan_in)) weights)",
        "config": {"workload": cfg.name, "pass": "forward+backward" + (" (with expert-weight gradients)"
                                                                       if a.weight_grads else ""),
                   "tokens": cfg.T, "hidden": cfg.H,
                   "experts": cfg.E, "shared_experts": int(cfg.shared), "ffn": cfg.F, "top_k": cfg.k,
                   "score": cfg.score_fn, "rows": model["_rows"], "active_experts": n_active,
                   "layer_copies": copies, "weight_layout": "packed",
                   "block_scales": "power of two" if pow2 else "amax/448 fp32", "parallelism": "none (1 GPU)"},
        "backward_gemm_tflops": round(bgemm_tflops, 2),
        "backward_gemm_frac_fp8_peak": round(bgemm_tflops / PEAK_FP8_TFLOPS, 4),
        "stages": stages, "roofline": roof, "cpu_baseline": cpu,
    }
    print(json.dumps(line))


def cpu_baseline_backward(cfg, x, dout, dev, pow2=False):
    """The backward oracle, per token with no dispatch, on a seeded sample of tokens."""
    import oracle as O
    import oracle.backward as B
    import oracle.layer as L
    import synth

    wg, b = synth.make_gate(cfg, 0, dev)
    rc = O.router_cfg(cfg.E, cfg.k, 0 if cfg.score_fn == "softmax" else 1, cfg.renorm, cfg.n_group,
                      cfg.topk_group, cfg.group_score_topk)

    def expert(e):
        w1, w2 = synth.make_expert(cfg, e, 0, dev)
        return L.quantize_expert(w1.cpu().numpy(), w2.cpu().numpy(), pow2)

    ol = L.OracleLayer(wg=wg.cpu().numpy(), bias=None if b is None else b.cpu().numpy(), cfg=rc, shared=cfg.shared,
                       act=cfg.act, F=cfg.F, expert=expert, pow2=pow2)
    toks = synth.sample_tokens(cfg.T, 4, cfg.seed + 98)
    xh, dh = x.float().cpu().numpy()[toks], dout.float().cpu().numpy()[toks]
    r0 = O.moe_route(O.moe_gate_logits(xh, ol.wg, ol.bias), rc)[0]
    for e in set(r0.reshape(-1).tolist()) | ({cfg.E} if cfg.shared else set()):
        ol.get(e)                              # weight quantisation is offline on the GPU side too
    t0 = time.perf_counter()
    B.backward_token(ol, xh, dh)
    dt = time.perf_counter() - t0
    return {"value": round(len(toks) / dt, 3), "unit": "tokens/s", "cores": O.num_threads(), "kind": "oracle",
            "sample": f"{len(toks)} seeded tokens of {cfg.T}, per-token backward (with its forward), "
                      "expert weights pre-quantised", "seconds": round(dt, 2)}


def stage_kernel(stage, layer):
    """The kernel a stage launches (the GEMM stages are one kernel each; the tile plan is part of
    the dispatch stage)."""
    import torch
    p2 = ", fp4" if layer.w.fp4 else ", pow2" if layer.w.pow2 else ""
    if stage == "gemm1_swiglu":
        return f"grouped_gemm_kernel<{layer.plan.tile_rows}, swiglu_quant, packed{p2}>"
    if stage == "gemm2":
        out = "bf16" if layer.act == torch.bfloat16 else "f32"
        return f"grouped_gemm_kernel<{layer.plan.tile_rows}, store_{out}, packed{p2}>"
    return stage


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed rocprofv3 counter runs
    (FETCH_SIZE and WRITE_SIZE, scaled by a plain copy's readings), or None when they were taken
    on a different kernel source than the one built here."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    with open(GEMM_SRC, "rb") as f:
        src = hashlib.sha256(f.read()).hexdigest()
    for r in rec.get("kernels", []):
        if r["kernel"] == kernel and r["workload"] == workload and r["source_sha256"] == src:
            return r["bytes_per_launch"]
    return None


PAYLOAD_SHAPE = (60, 8, 131072)   # [num_layers, top_k, seq_len]: a long-context rollout of a 60-layer model
PAYLOAD_EXPERTS = 256


def payload_bench(a):
    """Router-replay payload codec: pack (int32 -> ceil(log2 E) bits) and unpack on the device, and
    the pack + copy to pinned host / copy from host + unpack transport, on a synthetic uniform
    payload resident in HBM.  One JSON line; `value` is the pack kernel's algorithmic GB/s."""
    import numpy as np
    import torch

    import block_scaled_fp8_top_amd as M

    L, k, T = PAYLOAD_SHAPE
    E = PAYLOAD_EXPERTS
    n = L * k * T
    g = torch.Generator(device="cuda").manual_seed(11)
    idx = torch.randint(0, E, (L, k, T), dtype=torch.int32, device="cuda", generator=g)
    nb = M.payload_bytes(n, E)
    packed = torch.empty(nb, dtype=torch.uint8, device="cuda")
    staging = torch.empty(nb, dtype=torch.uint8, device="cuda")
    back = torch.empty_like(idx)
    hostbuf = torch.empty(nb, dtype=torch.uint8, pin_memory=True)
    st = torch.cuda.current_stream()

    def timed(fn, steps):
        for _ in range(max(a.warmup, 1)):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(steps):
            fn()
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    steps = a.steps
    t_pack = timed(lambda: M.moe_payload_pack(idx, E, out=packed), steps)
    t_unpack = timed(lambda: M.moe_payload_unpack(packed, (L, k, T), E, out=back), steps)
    t_d2h = timed(lambda: M.moe_payload_to_host(idx, E, staging, hostbuf), max(steps // 5, 2))
    t_h2d = timed(lambda: M.moe_payload_from_host(hostbuf, (L, k, T), E, staging, out=back), max(steps // 5, 2))
    torch.cuda.synchronize()
    ok = bool(torch.equal(back, idx))
    # the raw int32 payload copied to pinned host, for comparison with the packed transport
    rawhost = torch.empty(n, dtype=torch.int32, pin_memory=True)
    t_raw = timed(lambda: rawhost.copy_(idx.view(-1), non_blocking=True), max(steps // 5, 2))
    algo = n * 4 + nb
    gbs = algo / (t_pack * 1e-3) / 1e9

    # CPU baseline: the oracle's pack on one layer of the payload
    import oracle.payload as OP
    sample = idx[0].cpu().numpy()
    t0 = time.perf_counter()
    OP.payload_pack(sample, E)
    dt = time.perf_counter() - t0
    line = {
        "metric": "R3 router-replay payload pack, 1 GPU",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": a.warmup,
        "ms_per_step": round(t_pack, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int32 -> packed bits", "data": "synthetic (seeded uniform expert indices)",
        "config": {"workload": "payload", "shape": list(PAYLOAD_SHAPE), "experts": E,
                   "bits": nb * 8 // (((n + 31) // 32) * 32), "int32_bytes": n * 4, "packed_bytes": nb},
        "round_trip_exact": ok,
        "stages": {
            "pack": {"ms": round(t_pack, 4), "GB_s": round(gbs, 1), "bound": "hbm", "frac": round(gbs / 8000, 4)},
            "unpack": {"ms": round(t_unpack, 4), "GB_s": round(algo / (t_unpack * 1e-3) / 1e9, 1), "bound": "hbm",
                       "frac": round(algo / (t_unpack * 1e-3) / 1e9 / 8000, 4)},
            "pack_to_pinned_host": {"ms": round(t_d2h, 4), "payload_GB_s": round(n * 4 / (t_d2h * 1e-3) / 1e9, 1),
                                    "wire_GB_s": round(nb / (t_d2h * 1e-3) / 1e9, 1)},
            "pinned_host_to_unpack": {"ms": round(t_h2d, 4), "payload_GB_s": round(n * 4 / (t_h2d * 1e-3) / 1e9, 1)},
            "raw_int32_to_pinned_host": {"ms": round(t_raw, 4), "payload_GB_s": round(n * 4 / (t_raw * 1e-3) / 1e9, 1)},
        },
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": 8000.0, "unit": "GB/s",
                     "frac": round(gbs / 8000, 4), "traffic": None, "kernel": "payload_pack_kernel<8>",
                     "stage": "pack"},
        "cpu_baseline": {"value": round(sample.size * 4 / dt / 1e9, 3), "unit": "GB/s", "cores": 1,
                         "kind": "oracle", "sample": f"one layer ({k} x {T} indices) of the payload",
                         "seconds": round(dt, 3)},
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(cfg, x, dev, pow2=False, fp4=False):
    """The CPU oracle on a bounded sample of the same workload, timed on this host: the whole
    batch for small layers, else a seeded token sample evaluated per token."""
    import numpy as np

    import oracle as O
    import oracle.layer as L
    import synth

    wg, b = synth.make_gate(cfg, 0, dev)
    rc = O.router_cfg(cfg.E, cfg.k, 0 if cfg.score_fn == "softmax" else 1, cfg.renorm, cfg.n_group,
                      cfg.topk_group, cfg.group_score_topk)

    def expert(e):
        w1, w2 = synth.make_expert(cfg, e, 0, dev)
        if fp4:
            return L.quantize_expert_fp4(w1.cpu().numpy(), w2.cpu().numpy())
        return L.quantize_expert(w1.cpu().numpy(), w2.cpu().numpy(), pow2)

    ol = L.OracleLayer(wg=wg.cpu().numpy(), bias=None if b is None else b.cpu().numpy(), cfg=rc, shared=cfg.shared,
                       act=cfg.act, F=cfg.F, expert=expert, pow2=pow2)
    xh = x.float().cpu().numpy()
    if cfg.T <= 256:
        toks = np.arange(cfg.T)
        for g in range(cfg.groups):          # weight quantisation is offline on the GPU side too
            ol.get(g)
        # whole-batch passes until about 10 s of CPU work (at least one, at most six)
        passes = 0
        t0 = time.perf_counter()
        while passes < 6 and (passes == 0 or time.perf_counter() - t0 < 10.0):
            L.forward_dispatch(ol, xh)
            passes += 1
        dt = time.perf_counter() - t0
        toks = np.arange(cfg.T * passes)
        sample = (f"whole batch ({cfg.T} tokens) x {passes} passes, dispatch path, expert weights "
                  "pre-quantised")
    else:
        n = 12
        toks = synth.sample_tokens(cfg.T, n, cfg.seed + 99)
        pre = L.forward_sampled(ol, xh[toks[:1]])   # warm the expert cache for token 0 only
        del pre
        r0 = O.moe_route(O.moe_gate_logits(xh[toks], ol.wg, ol.bias), rc)[0]
        for e in set(r0.reshape(-1).tolist()) | ({cfg.E} if cfg.shared else set()):
            ol.get(e)
        t0 = time.perf_counter()
        L.forward_sampled(ol, xh[toks])
        dt = time.perf_counter() - t0
        sample = f"{len(toks)} seeded tokens of {cfg.T}, per-token path, expert weights pre-quantised"
    return {"value": round(len(toks) / dt, 3), "unit": "tokens/s", "cores": O.num_threads(), "kind": "oracle",
            "sample": sample, "seconds": round(dt, 2)}


if __name__ == "__main__":
    main()
