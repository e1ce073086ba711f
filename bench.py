"""Benchmark of the block-scaled FP8 MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload longctx|prefill|decode|r3|tiny|payload]
                    [--scales amax|pow2] [--weights fp8|fp4] [--backward] [--no-extras]

A step is one pass of the layer forward (gate logits, routing with the 1x128 quantisation of x,
dispatch, grouped GEMM1 + SwiGLU + h quantisation, grouped GEMM2, combine) over one batch of
synthetic tokens whose inputs and quantised weights are already resident in HBM.  The default
workload is the long-context layer: 131072 tokens streamed through one layer (hidden 6144, 256
experts, FFN 2048, top-8 sigmoid routing in 8 groups keeping 4, with a Zipf(1.2) expert-popularity
bias) as 16 chunks of 8192 tokens, each chunk's output written to its rows of the [131072, 6144]
output; a step is the whole stream.  Consecutive steps cycle through several copies of the layer
(weights packed for the grouped GEMM, plus buffers), at least 2 GiB of weights in all, so a step
never finds its weights in the 256 MB Infinity Cache left behind by the step before.  The reported
rate times replays of a HIP graph holding the whole step (--no-graph: eager launches); a second
pass of eager steps with HIP events between the stages gives the per-stage times (on the launch
stream).  Prints one JSON line: tokens/s, per-stage times and roofline fractions, the grouped
GEMM's TFLOP/s, the roofline of the dominant kernel, the CPU oracle timed on a bounded sample and,
unless --no-extras, the prefill layer (16384 tokens, 256 routed + 1 shared expert), the four-layer
router-replay stack (32768 tokens: pass A routes and records, pass B replays on perturbed weights,
pass C recomputes the routing on them) and the 128x128 quantisation of one layer's expert weights
(the per-step cost of block-scaled FP8 training) as extra keys.
With --backward a step is the layer's training forward (GEMM1 also keeps its fp32 output)
followed by its backward (output gradient -> dx, dWg, db), and the line reports the backward's
stages too.  --weights fp4 runs the same forward with FP4 expert weights (E2M1 in 1x32 blocks with
E8M0 scales; activations stay FP8 with power-of-two scales).
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
# fp32 vector peak the library's kernels can issue: the published 157.3 TFLOP/s needs packed fp32 FMAs,
# which the library's compile flags turn off, so one fma per lane per clock:
# 256 CUs x 4 SIMDs x 16 lanes x 2 flop x 2.4 GHz
PEAK_FP32_TFLOPS = 78.6
RIDGE_FP8 = PEAK_FP8_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
PEAKS = {"hbm": "8.0 TB/s HBM3E (published)", "mfma": "5.0 PFLOP/s dense fp8 (published)",
         "alu": "78.6 TFLOP/s fp32 vector without packed FMA (published 157.3 needs packed fp32 FMA, "
                "which the library's compile flags turn off)"}
# achievable peaks measured on MI355X with in-bounds microbenchmarks built here (a register-only fp8
# MFMA loop, 16 independent accumulators, 2 waves per SIMD; streaming reads of contiguous 32 KB
# blocks by 256-1024 workgroups); reported beside the published ones
MEASURED_FP8_TFLOPS = 4680.0
MEASURED_HBM_READ_GBS = 6300.0

def log(msg):
    """Progress line on stderr (the JSON result is the only line on stdout)."""
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


STAGES = ["gate_logits", "route_quant", "dispatch", "gemm1_swiglu", "gemm2", "combine"]
BWD_STAGES = ["bwd_combine", "bwd_gemm_dh", "bwd_gemm_g", "bwd_swiglu", "bwd_gemm_da", "bwd_combine_dx", "bwd_route",
              "bwd_gate"]
WGRAD_STAGES = ["bwd_wgrad_quant", "bwd_wgrad_gemm"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="longctx")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the prefill layer, the replay stack and the weight quantisation after the headline")
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
    ap.add_argument("--tile-rows", type=int, default=0,
                    help="row-tile height of the expert GEMMs (0: chosen from the group sizes)")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB (counter calibration)")
    return ap.parse_args()


def stage_model(cfg, counts, n_active1, fp4=False, record=False):
    """Algorithmic bytes and flops of each stage (inputs read once, outputs written once).  Expert
    weight bytes per element: 1 + 4/128^2 for e4m3 with 128x128 fp32 scales, 1/2 + 1/32 for FP4
    with one E8M0 byte per 1x32 block.  route_quant is one launch: the router (logits in, indices
    and weights out, the payload record) and x's 1x128 quantisation."""
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
        "route_quant": dict(bytes=T * E * 4 + T * k * 8 + (T * k * 4 if record else 0) + T * H * (ab + 1 + sig),
                            flops=0.0, bound="hbm"),
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


def rates(m, ms):
    """Achieved rates of work m (bytes, flops, bound) done in ms, and its roofline fraction.  A
    GEMM's bound is the larger of its MFMA time (flops / fp8 peak) and its HBM time (algorithmic
    bytes / HBM peak); both fractions are reported."""
    t = ms * 1e-3
    d = {"ms": round(ms, 4), "GB_s": round(m["bytes"] / t / 1e9, 1)}
    if m["flops"]:
        d["TFLOP_s"] = round(m["flops"] / t / 1e12, 2)
    if m["bound"] is None:
        t_mfma = m["flops"] / (PEAK_FP8_TFLOPS * 1e12)
        t_hbm = m["bytes"] / (PEAK_HBM_GBS * 1e9)
        d["bound"] = "mfma" if t_mfma >= t_hbm else "hbm"
        d["frac"] = round(max(t_mfma, t_hbm) / t, 4)
        d["frac_mfma"] = round(t_mfma / t, 4)
        d["frac_hbm"] = round(t_hbm / t, 4)
    else:
        d["bound"] = m["bound"]
        if d["bound"] == "alu":
            d["frac"] = round(m["flops"] / t / 1e12 / PEAK_FP32_TFLOPS, 4)
        else:
            d["frac"] = round(m["bytes"] / t / 1e9 / PEAK_HBM_GBS, 4)
    return d


def sum_models(models, names):
    """Stage models of several launches (chunks) added up."""
    out = {}
    for n in names:
        out[n] = dict(bytes=sum(m[n]["bytes"] for m in models), flops=sum(m[n]["flops"] for m in models),
                      bound=models[0][n]["bound"])
    return out


def build_weights(cfg, dev, pow2=False, fp4=False, layer=0, perturbed=False, keep_rowmajor=False):
    """One layer's router gate and expert weights (quantised and packed on the GPU from the seeded
    fp32 masters, one expert at a time)."""
    import synth
    import block_scaled_fp8_top_amd as M
    from block_scaled_fp8_top_amd.layer import (MoELayerWeights, pack_expert_weights, quantize_expert_weights,
                                                quantize_expert_weights_fp4)
    sf = 0 if cfg.score_fn == "softmax" else 1
    rcfg = M.router_cfg(cfg.E, cfg.k, sf, cfg.renorm, cfg.n_group, cfg.topk_group, cfg.group_score_topk)
    wg, b = synth.make_gate(cfg, layer, dev, perturbed=perturbed)
    master = lambda g: synth.make_expert(cfg, g, layer, dev, perturbed=perturbed)  # noqa: E731
    if fp4:
        w1p, w2p = quantize_expert_weights_fp4(cfg.groups, cfg.H, cfg.F, master, device=dev)
        return MoELayerWeights(wg=wg, bias=b, w1q=None, w1s=None, w2q=None, w2s=None, cfg=rcfg, shared=cfg.shared,
                               w1p=w1p, w2p=w2p, pow2=True)
    w1q, w1s, w2q, w2s = quantize_expert_weights(cfg.groups, cfg.H, cfg.F, master, device=dev, pow2=pow2)
    return pack_expert_weights(MoELayerWeights(wg=wg, bias=b, w1q=w1q, w1s=w1s, w2q=w2q, w2s=w2s, cfg=rcfg,
                                               shared=cfg.shared, pow2=pow2), keep_rowmajor=keep_rowmajor)


def clone_weights(weights):
    """A second copy of a layer's packed expert weights (same values, other memory)."""
    from dataclasses import replace
    if weights.fp4:
        return replace(weights, w1p=replace(weights.w1p, data=weights.w1p.data.clone(),
                                            scales=weights.w1p.scales.clone()),
                       w2p=replace(weights.w2p, data=weights.w2p.data.clone(), scales=weights.w2p.scales.clone()))
    return replace(weights, w1p=replace(weights.w1p, data=weights.w1p.data.clone()),
                   w2p=replace(weights.w2p, data=weights.w2p.data.clone()), w1s=weights.w1s.clone(),
                   w2s=weights.w2s.clone())


def free_gpu():
    import gc
    import torch
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def gemm_launch_heights(plan):
    """Row-tile heights of the launches of one planned grouped GEMM call: a plan of 256-row tiles
    runs as two launches (then the groups' short remainders of up to 128 rows as 128-row tiles)
    when its workspace holds the third tile list, which it does whenever the average group has
    85 rows or more (the library's rule: 2 * (ceil(rows/256) + G) + G <= ceil(rows/32) + G)."""
    bm, rows, g = plan.tile_rows, plan.max_rows, plan.groups
    mt = -(-rows // 256) + g
    cap = -(-rows // 32) + g
    return [256, 128] if bm == 256 and 2 * mt + g <= cap else [bm]


def stage_kernel(stage, layer):
    """The kernel(s) a stage launches, joined by " + " (a grouped GEMM call is one or two launches;
    the tile plan is part of the dispatch stage)."""
    import torch
    p2 = ", fp4" if layer.w.fp4 else ", pow2" if layer.w.pow2 else ""
    if stage == "gemm1_swiglu":
        return " + ".join(f"grouped_gemm_kernel<{h}, swiglu_quant, packed{p2}>" for h in gemm_launch_heights(layer.plan))
    if stage == "gemm2":
        out = "bf16" if layer.act == torch.bfloat16 else "f32"
        return " + ".join(f"grouped_gemm_kernel<{h}, store_{out}, packed{p2}>" for h in gemm_launch_heights(layer.plan))
    if stage == "route_quant":
        return "route_quant_kernel"
    if stage == "gate_logits":
        return "gate_logits_kernel"
    if stage == "combine":
        return "combine_kernel"
    return stage


def run_forward_workload(a, cfg, dev, steps, warmup, pow2=False, fp4=False, cpu=True):
    """Time the layer forward on workload cfg; a step covers all of cfg's chunks.  Returns the
    result dict (the JSON line's body for the headline, an extra key otherwise)."""
    import numpy as np
    import torch

    import synth
    from block_scaled_fp8_top_amd.layer import MoELayer

    log(f"{cfg.name}: building weights")
    weights = build_weights(cfg, dev, pow2, fp4)
    wbytes = weights.w1p.data.numel() + weights.w2p.data.numel()
    copies = a.copies if a.copies > 0 else max(2, math.ceil((2 << 30) / wbytes))
    act = torch.bfloat16 if cfg.act == "bf16" else torch.float32
    layers = [MoELayer(weights, cfg.T, act, dev, tile_rows=a.tile_rows)]
    for _ in range(1, copies):
        layers.append(MoELayer(clone_weights(weights), cfg.T, act, dev, tile_rows=a.tile_rows))
    C, T = cfg.chunks, cfg.T
    if C > 1:
        x_all = torch.empty((C * T, cfg.H), dtype=act, device=dev)
        for c in range(C):
            x_all[c * T:(c + 1) * T] = synth.make_x(cfg, dev, chunk=c)
    else:
        x_all = synth.make_x(cfg, dev)
    out_all = torch.empty_like(x_all)
    xs = [x_all[c * T:(c + 1) * T] for c in range(C)]
    outs = [out_all[c * T:(c + 1) * T] for c in range(C)]

    def step(copy, evs=None):
        lay = layers[copy]
        if evs is None and C > 1:
            # the stream: chunk c + 1's gate projection beside chunk c's combine (forward_chunks)
            lay.forward_chunks(xs, outs)
            return
        for c in range(C):
            lay.forward(xs[c], out=outs[c], events=None if evs is None else evs[c])

    # census of the realised routing of every chunk (untimed): each chunk's group sizes
    counts = []
    for c in range(C):
        layers[0].forward(xs[c], out=outs[c])
        counts.append(layers[0].disp.counts.cpu().numpy())
    for s in range(warmup):
        step(s % copies)
    torch.cuda.synchronize()
    log(f"{cfg.name}: {copies} layer copies, {C} chunk(s) per step; timing {steps} steps")

    graphs = None
    if not a.no_graph:
        graphs = []
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for c in range(copies):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=side):
                    step(c)
                graphs.append(g)
        torch.cuda.current_stream().wait_stream(side)
        for s in range(warmup):
            graphs[s % copies].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(steps):
            graphs[s % copies].replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t0) * 1e3 / steps

    ns = len(STAGES)
    ev = [[[torch.cuda.Event(enable_timing=True) for _ in range(ns + 1)] for _ in range(C)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        step(s % copies, ev[s])
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / steps
    ms_per_step = eager_ms if graphs is None else graph_ms
    # stage time of chunk c, averaged over the steps (events on the launch stream)
    chunk_ms = [{name: float(np.mean([ev[s][c][i].elapsed_time(ev[s][c][i + 1]) for s in range(steps)]))
                 for i, name in enumerate(STAGES)} for c in range(C)]
    models = [stage_model(cfg, counts[c], int((counts[c] > 0).sum()), fp4) for c in range(C)]
    total = sum_models(models, STAGES)
    stage_ms = {n: sum(chunk_ms[c][n] for c in range(C)) for n in STAGES}
    stages = {n: rates(total[n], stage_ms[n]) for n in STAGES}
    gemm_ms = stage_ms["gemm1_swiglu"] + stage_ms["gemm2"]
    gemm_flops = total["gemm1_swiglu"]["flops"] + total["gemm2"]["flops"]
    gemm_tflops = gemm_flops / (gemm_ms * 1e-3) / 1e12

    # dominant kernel: the slowest stage; per launch = per chunk (same rows in every chunk, the
    # active experts vary), so achieved = mean algorithmic work per launch / mean launch time
    dom = max(STAGES, key=lambda n: stage_ms[n])
    e = stages[dom]
    launch_ms = stage_ms[dom] / C
    if e["bound"] == "mfma":
        roof = {"bound": "mfma", "achieved": round(total[dom]["flops"] / C / (launch_ms * 1e-3) / 1e12, 2),
                "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s"}
    elif e["bound"] == "alu":
        roof = {"bound": "alu", "achieved": round(total[dom]["flops"] / C / (launch_ms * 1e-3) / 1e12, 2),
                "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(total[dom]["bytes"] / C / (launch_ms * 1e-3) / 1e9, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    if roof["bound"] == "mfma":
        roof["frac_of_measured_mfma_loop"] = round(roof["achieved"] / MEASURED_FP8_TFLOPS, 4)
    elif roof["bound"] == "hbm":
        roof["frac_of_measured_stream_read"] = round(roof["achieved"] / MEASURED_HBM_READ_GBS, 4)
    kname = stage_kernel(dom, layers[0])
    roof["traffic"] = measured_traffic(kname, cfg.name)
    roof["kernel"] = kname
    roof["stage"] = dom
    roof["launch_ms"] = round(launch_ms, 4)
    roof["launches_per_step"] = C

    res = {
        "value": round(C * T / (ms_per_step * 1e-3), 1),
        "ms_per_step": round(ms_per_step, 4),
        "launch": "eager" if graphs is None else "hip-graph replay",
        "eager_ms_per_step": round(eager_ms, 4),
        "config": {"workload": cfg.name, "tokens": C * T, "chunk_tokens": T, "chunks": C, "hidden": cfg.H,
                   "experts": cfg.E, "shared_experts": int(cfg.shared), "ffn": cfg.F, "top_k": cfg.k,
                   "score": cfg.score_fn, "group_limit": f"{cfg.n_group} groups keep {cfg.topk_group}"
                   if cfg.n_group > 1 else None, "expert_bias": cfg.bias,
                   "rows_per_chunk": models[0]["_rows"],
                   "active_experts_per_chunk": [int((cc > 0).sum()) for cc in counts],
                   "layer_copies": copies, "weight_layout": "packed",
                   "block_scales": "power of two" if pow2 else "amax/448 fp32",
                   "expert_weights": "fp4 e2m1, 1x32 e8m0 scales" if fp4 else "fp8 e4m3, 128x128 scales",
                   "parallelism": "none (1 GPU)"},
        "gemm_tflops": round(gemm_tflops, 2),
        "gemm_frac_fp8_peak": round(gemm_tflops / PEAK_FP8_TFLOPS, 4),
        "stages": stages,
        "roofline": roof,
    }
    if C > 1:
        # per chunk: GEMM1's bound and fraction from that chunk's realised group sizes
        res["per_chunk"] = [{"active_experts": int((counts[c] > 0).sum()),
                             "max_group_rows": int(counts[c].max()),
                             "gemm1_swiglu": {k2: v for k2, v in rates(models[c]["gemm1_swiglu"],
                                                                       chunk_ms[c]["gemm1_swiglu"]).items()
                                              if k2 in ("ms", "bound", "frac", "frac_mfma", "frac_hbm")},
                             "gemm2_frac": rates(models[c]["gemm2"], chunk_ms[c]["gemm2"])["frac"]}
                            for c in range(C)]
    if a.copy_probe_mb:
        n = a.copy_probe_mb * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    x0 = xs[0].clone()
    del layers, graphs, weights, x_all, out_all, xs, outs
    free_gpu()
    log(f"{cfg.name}: {res['value']:.0f} tokens/s, {res['ms_per_step']:.3f} ms per step")
    if cpu:
        log(f"{cfg.name}: CPU oracle baseline")
        res["cpu_baseline"] = cpu_baseline(cfg, x0, dev, pow2, fp4)
    return res


def run_r3_stack(a, cfg, dev, steps, warmup):
    """The four-layer replay stack (residual x_{l+1} = act(x_l + out_l)): pass A routes on W and
    records the [layers, top_k, seq_len] payload, pass B replays it on W' = W + N(0, 1e-3), pass C
    recomputes the routing on W'.  Each pass is one HIP graph replayed `steps` times; an untimed
    eager run checks replay exactness and measures the drift that replay removes."""
    import torch

    import synth
    from block_scaled_fp8_top_amd.layer import MoELayer

    Lyr, T, k = cfg.layers, cfg.T, cfg.k
    act = torch.bfloat16 if cfg.act == "bf16" else torch.float32
    W, Wp = [], []
    for l in range(Lyr):
        log(f"r3: building weights of layer {l} (W and W')")
        W.append(build_weights(cfg, dev, layer=l))
        Wp.append(build_weights(cfg, dev, layer=l, perturbed=True))
    lay = MoELayer(W[0], T, act, dev, tile_rows=a.tile_rows)
    payload = torch.full((Lyr, k, T), -1, dtype=torch.int32, device=dev)
    x0 = synth.make_x(cfg, dev)
    xbuf = {p: torch.empty_like(x0) for p in "ABC"}

    def run_pass(p, keep=None):
        x = xbuf[p]
        x.copy_(x0)
        for l in range(Lyr):
            lay.w = W[l] if p == "A" else Wp[l]
            if p == "A":
                lay.forward(x, record=payload[l], residual_out=x)
            elif p == "B":
                lay.forward(x, replay=payload[l], residual_out=x)
            else:
                lay.forward(x, residual_out=x)
            if keep is not None:
                keep[(p, l)] = (lay.idx.clone(), lay.disp.counts.clone(), lay.disp.dest_row.clone(),
                                int(lay.bad.item()))
        return x

    lay.bad.zero_()
    keep = {}
    for p in "ABC":
        run_pass(p, keep)
    torch.cuda.synchronize()
    mismatch = sum(int((keep[("B", l)][0] != payload[l].t()).sum().item()) for l in range(Lyr))
    perm_equal = all(torch.equal(keep[("B", l)][1], keep[("A", l)][1]) and
                     torch.equal(keep[("B", l)][2], keep[("A", l)][2]) for l in range(Lyr))
    drift = []
    for l in range(Lyr):
        ia, ic = keep[("A", l)][0], keep[("C", l)][0]
        slot = (ic != ia).float().mean().item()
        setd = 1.0 - (ic[:, :, None] == ia[:, None, :]).any(-1).float().mean().item()
        drift.append({"layer": l, "slot_drift": round(slot, 4), "expert_set_drift": round(setd, 4)})

    def rel(u, v):
        u, v = u.float(), v.float()
        return float((u - v).abs().max() / v.abs().max())

    dB, dC = rel(xbuf["B"], xbuf["A"]), rel(xbuf["C"], xbuf["A"])
    log(f"r3: checked passes (replay mismatch {mismatch}); timing")
    passes = {}
    for p in "ABC":
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                run_pass(p)
        torch.cuda.current_stream().wait_stream(side)
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            g.replay()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        passes[p] = {"ms_per_pass": round(ms, 3), "tokens_per_s": round(T / (ms * 1e-3), 1),
                     "layer_tokens_per_s": round(Lyr * T / (ms * 1e-3), 1)}
        del g
    passes["A"]["what"] = "route on W, record the payload"
    passes["B"]["what"] = "replay the payload on W' (gate projection fused with the replay: k logits per token)"
    passes["C"]["what"] = "route again on W'"
    res = {"workload": "r3", "layers": Lyr, "tokens": T, "passes": passes, "replay_index_mismatch": mismatch,
           "replay_bad_ids": int(lay.bad.item()), "replay_permutation_equal": perm_equal,
           "recompute_drift_per_layer": drift, "out_rel_diff_B_vs_A": round(dB, 4),
           "out_rel_diff_C_vs_A": round(dC, 4), "steps": steps}
    del W, Wp, lay, payload, xbuf, keep
    free_gpu()
    return res


def run_weight_quant(cfg, dev, steps, pow2=False):
    """128x128 block quantisation of one layer's expert weights (fp32 masters -> e4m3 codes + fp32
    scales; all routed and shared experts, W1 and W2, one batched call each): the per-step weight
    cast of block-scaled FP8 training, which inference does once offline."""
    import torch

    import block_scaled_fp8_top_amd as M
    import synth

    G, H, F = cfg.groups, cfg.H, cfg.F
    log(f"weight quantisation: drawing {G} experts' fp32 masters")
    w1 = torch.empty((G, 2 * F, H), dtype=torch.float32, device=dev)
    w2 = torch.empty((G, H, F), dtype=torch.float32, device=dev)
    for g in range(G):
        a1, a2 = synth.make_expert(cfg, g, 0, dev)
        w1[g].copy_(a1)
        w2[g].copy_(a2)
        del a1, a2
    q1 = torch.empty(w1.shape, dtype=torch.uint8, device=dev)
    q2 = torch.empty(w2.shape, dtype=torch.uint8, device=dev)
    s1 = torch.empty((G, 2 * F // 128, H // 128), dtype=torch.float32, device=dev)
    s2 = torch.empty((G, H // 128, F // 128), dtype=torch.float32, device=dev)

    def once():
        M.moe_quant_fp8_block(w1, 128, q=q1, scales=s1, pow2=pow2)
        M.moe_quant_fp8_block(w2, 128, q=q2, scales=s2, pow2=pow2)

    once()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        once()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    n = w1.numel() + w2.numel()
    nbytes = n * (4 + 1) + (s1.numel() + s2.numel()) * 4
    del w1, w2, q1, q2, s1, s2
    free_gpu()
    d = rates(dict(bytes=nbytes, flops=0.0, bound="hbm"), ms)
    d.update({"kernel": "quant_128x128_kernel", "experts": G, "elements": n,
              "what": "one layer's expert weights, fp32 masters -> e4m3 + 128x128 fp32 scales"})
    return d


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {a.gpus}): the layer's multi-GPU form (expert "
              "parallel dispatch/combine over xGMI) is not implemented in this library.", file=sys.stderr)
        sys.exit(2)

    import torch

    import block_scaled_fp8_top_amd as M
    import synth

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    M.lib()  # fail loudly if the HIP library is missing
    dev = "cuda"
    if a.workload == "payload":
        payload_bench(a)
        return
    cfg = synth.CONFIGS[a.workload]
    fp4 = a.weights == "fp4"
    if fp4 and a.backward:
        print("--weights fp4 is a forward-only format (no backward)", file=sys.stderr)
        sys.exit(2)
    pow2 = a.scales == "pow2" or fp4
    if a.backward:
        backward_main(a, cfg, dev, pow2)
        return
    if a.workload == "r3":
        r = run_r3_stack(a, cfg, dev, a.steps, a.warmup)
        pa = r["passes"]["A"]
        line = {"metric": "MoE layer tokens/s + grouped FP8 GEMM TFLOP/s (% of fp8 MFMA peak), 1 GPU",
                "value": pa["layer_tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": a.steps,
                "warmup": a.warmup, "ms_per_step": pa["ms_per_pass"], "higher_is_better": True,
                "scaling": "weak", "vs_baseline": None, "dtype": "fp8-e4m3 x fp8-e4m3 -> fp32 (GEMM); fp32 router",
                "data": "synthetic", "config": {"workload": "r3", "layers": cfg.layers, "tokens": cfg.T},
                "r3": r}
        print(json.dumps(line), flush=True)
        return
    steps, warm = a.steps, a.warmup
    head = run_forward_workload(a, cfg, dev, steps, warm, pow2, fp4, cpu=not a.no_cpu_baseline)
    line = {
        "metric": "MoE layer tokens/s + grouped FP8 GEMM TFLOP/s (% of fp8 MFMA peak), 1 GPU",
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": head["ms_per_step"],
        "launch": head["launch"],
        "eager_ms_per_step": head["eager_ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp4-e2m1 weights x fp8-e4m3" if fp4 else "fp8-e4m3 x fp8-e4m3") + " -> fp32 (GEMM); fp32 router; "
                 + ("bf16" if cfg.act == "bf16" else "fp32") + " activations",
        "data": "synthetic (seeded N(0,1) activations, N(0,1/sqrt(fan_in)) weights, random-init)",
        "config": head["config"],
        "gemm_tflops": head["gemm_tflops"],
        "gemm_frac_fp8_peak": head["gemm_frac_fp8_peak"],
        "stages": head["stages"],
        "roofline": head["roofline"],
        "cpu_baseline": head.get("cpu_baseline"),
        "peaks": PEAKS,
    }
    if "per_chunk" in head:
        line["per_chunk"] = head["per_chunk"]
    if not a.no_extras and a.workload == "longctx" and not fp4:
        xs = min(steps, 10)
        pre = run_forward_workload(a, synth.CONFIGS["prefill"], dev, xs, 2, pow2, False, cpu=False)
        line["prefill"] = {k2: pre[k2] for k2 in ("value", "ms_per_step", "gemm_tflops", "gemm_frac_fp8_peak",
                                                 "stages", "roofline")}
        line["prefill"]["unit"] = "tokens/s"
        line["prefill"]["config"] = {k2: pre["config"][k2] for k2 in ("workload", "tokens", "experts",
                                                                      "shared_experts", "block_scales")}
        line["r3"] = run_r3_stack(a, synth.CONFIGS["r3"], dev, min(steps, 5), 1)
        line["weight_quant"] = run_weight_quant(synth.CONFIGS["prefill"], dev, 3, pow2)
    print(json.dumps(line), flush=True)


GEMM_SRC = os.path.join(ROOT, "block_scaled_fp8_top_amd", "csrc", "grouped_gemm.hip")


def backward_main(a, cfg, dev, pow2):
    """Layer copies with the backward's weight copies, then the forward + backward bench."""
    import torch

    import synth
    from block_scaled_fp8_top_amd.layer import MoELayer, prepare_backward_weights
    from dataclasses import replace

    weights = build_weights(cfg, dev, pow2, keep_rowmajor=True)
    bwd_weights = prepare_backward_weights(weights)
    weights = replace(weights, w1q=None, w2q=None)
    wbytes = weights.w1p.data.numel() + weights.w2p.data.numel()
    copies = a.copies if a.copies > 0 else max(2, math.ceil((2 << 30) / wbytes))
    act = torch.bfloat16 if cfg.act == "bf16" else torch.float32
    layers = [MoELayer(weights, cfg.T, act, dev)]
    for _ in range(1, copies):
        layers.append(MoELayer(clone_weights(weights), cfg.T, act, dev))
    x = synth.make_x(cfg, dev)
    torch.cuda.synchronize()
    backward_bench(a, cfg, layers, bwd_weights, x, copies, pow2)


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
    stages = {name: rates(model[name], stage_ms[name]) for name in timed}
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


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed rocprofv3 counter runs
    (FETCH_SIZE and WRITE_SIZE, scaled by a plain copy's readings), or None when they were taken
    on a different kernel source than the one built here.  Kernels joined by " + " (one GEMM call
    of two launches) add up, and give None if any of them has no entry."""
    if " + " in kernel:
        parts = [measured_traffic(k, workload) for k in kernel.split(" + ")]
        return None if any(p is None for p in parts) else sum(parts)
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
        n = 48                                # about 10-15 s of the oracle on 16 host threads
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
