"""Helpers shared by the GPU parity tests: build the same layer for the HIP path and for the oracle.

Every input comes from ``synth`` drawn on the GPU; the oracle receives host copies of those same
draws (never anything computed by the HIP path) and quantises the expert masters itself.
"""
from __future__ import annotations

import numpy as np
import torch

import block_scaled_fp8_top_amd as M
import oracle as O
import oracle.layer as L
import synth
from block_scaled_fp8_top_amd.layer import (MoELayer, MoELayerWeights, pack_expert_weights, quantize_expert_weights,
                                            quantize_expert_weights_fp4)

DEV = "cuda"
TOL = 2e-2          # max |gpu - ref| / max |ref| for GEMM and combine outputs


def cfgs_for(cfg: synth.LayerConfig):
    """(GPU router cfg, oracle router cfg) of a workload."""
    sf = 0 if cfg.score_fn == "softmax" else 1
    args = (cfg.E, cfg.k, sf, cfg.renorm, cfg.n_group, cfg.topk_group, cfg.group_score_topk)
    return M.router_cfg(*args), O.router_cfg(*args)


def gpu_weights(cfg: synth.LayerConfig, layer: int = 0, perturbed: bool = False, pow2: bool = False,
                fp4: bool = False) -> MoELayerWeights:
    """fp4: FP4 experts (packed only), with power-of-two activation scales."""
    wg, b = synth.make_gate(cfg, layer, DEV, perturbed=perturbed)
    if fp4:
        w1p, w2p = quantize_expert_weights_fp4(
            cfg.groups, cfg.H, cfg.F, lambda g: synth.make_expert(cfg, g, layer, DEV, perturbed=perturbed), device=DEV)
        return MoELayerWeights(wg=wg, bias=b, w1q=None, w1s=None, w2q=None, w2s=None, cfg=cfgs_for(cfg)[0],
                               shared=cfg.shared, w1p=w1p, w2p=w2p, pow2=True)
    w1q, w1s, w2q, w2s = quantize_expert_weights(
        cfg.groups, cfg.H, cfg.F, lambda g: synth.make_expert(cfg, g, layer, DEV, perturbed=perturbed), device=DEV,
        pow2=pow2)
    # the layer streams the packed copies; the row-major codes stay for the weight checks
    return pack_expert_weights(MoELayerWeights(wg=wg, bias=b, w1q=w1q, w1s=w1s, w2q=w2q, w2s=w2s,
                                               cfg=cfgs_for(cfg)[0], shared=cfg.shared, pow2=pow2))


def oracle_layer(cfg: synth.LayerConfig, layer: int = 0, perturbed: bool = False, pow2: bool = False,
                 fp4: bool = False) -> L.OracleLayer:
    """Oracle view of the same layer: gate and masters re-drawn from the same GPU streams and
    copied to the host; the oracle quantises each expert it needs (fp4: FP4 experts, pow2 scales)."""
    wg, b = synth.make_gate(cfg, layer, DEV, perturbed=perturbed)

    def expert(e):
        w1, w2 = synth.make_expert(cfg, e, layer, DEV, perturbed=perturbed)
        if fp4:
            return L.quantize_expert_fp4(w1.cpu().numpy(), w2.cpu().numpy())
        return L.quantize_expert(w1.cpu().numpy(), w2.cpu().numpy(), pow2)

    return L.OracleLayer(wg=wg.cpu().numpy(), bias=None if b is None else b.cpu().numpy(), cfg=cfgs_for(cfg)[1],
                         shared=cfg.shared, act=cfg.act, F=cfg.F, expert=expert, pow2=pow2 or fp4)


def host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy (bf16 widened to fp32 exactly)."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy()


def rows_host(t: torch.Tensor, rows) -> np.ndarray:
    """Selected rows of a device tensor, gathered on the device, as numpy."""
    return host(t[torch.as_tensor(np.asarray(rows), dtype=torch.long, device=t.device)])


def rel_err(got, ref) -> float:
    return L.rel_err(got, ref)


def assert_equal(name, got, ref):
    got, ref = np.asarray(got), np.asarray(ref)
    assert got.shape == ref.shape, f"{name}: shape {got.shape} vs {ref.shape}"
    if got.dtype.kind == "f":
        same = np.array_equal(got.view(np.uint32 if got.dtype == np.float32 else np.uint64),
                              ref.astype(got.dtype).view(np.uint32 if got.dtype == np.float32 else np.uint64))
    else:
        same = np.array_equal(got, ref)
    if not same:
        bad = np.argwhere(got != ref) if got.dtype.kind != "f" else np.argwhere(
            got.view(np.uint32) != ref.astype(np.float32).view(np.uint32))
        first = tuple(bad[0]) if len(bad) else None
        raise AssertionError(f"{name}: {len(bad)} mismatches, first at {first}: "
                             f"gpu {got[first] if first else None} ref {ref[first] if first else None}")
