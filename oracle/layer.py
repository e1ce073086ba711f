"""Whole-layer oracle: the MoE layer forward composed from the step functions of ``oracle``.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Two independent compositions are provided:

* ``forward_dispatch`` follows the method's data path: route (or replay) -> 1x128 activation
  quantisation -> dispatch into expert-contiguous groups -> grouped GEMM1 -> SwiGLU -> 1x128
  quantisation of h -> grouped GEMM2 -> output rows stored in the activation dtype -> weighted
  combine back to token order ("RL at 1T Scale: prime-rl Performance Deep Dive", sections
  "Wide EP" (dispatch / combine), "Router replay", "FP8 training").
* ``forward_token`` evaluates one token at a time with no dispatch at all: the token's own
  selected experts applied directly (and, with ``dense=True``, every expert applied with a gate
  vector that is zero off the selection).  A MoE layer's output for a token depends only on
  that token, so both compositions must agree; the second also serves large layers on sampled
  tokens, fetching only the experts those tokens use.

Readings (the pages are silent on these): a shared expert, when present, has the routed
experts' FFN width, weight 1 and is added after the routed slots; expert output rows are
stored in the activation dtype (fp32 or bf16) before the combine.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, Optional

import numpy as np

import oracle as O


@dataclass
class ExpertWeights:
    """One expert's quantised FFN: W1 [2F,H] (rows [0,F) gate, [F,2F) up), W2 [H,F].  FP8: e4m3
    codes with 128x128 fp32 block scales; fp4: FP4 E2M1 codes two per byte ([rows, cols/2]) with
    1x32 E8M0 scale codes ([rows, cols/32]) in the scale fields."""
    w1q: np.ndarray
    w1s: np.ndarray
    w2q: np.ndarray
    w2s: np.ndarray
    fp4: bool = False

    def w1(self) -> np.ndarray:
        """fp64 value of the quantised W1."""
        return O.dequant_mxfp4(self.w1q, self.w1s) if self.fp4 else O.dequant_weight(self.w1q, self.w1s)

    def w2(self) -> np.ndarray:
        return O.dequant_mxfp4(self.w2q, self.w2s) if self.fp4 else O.dequant_weight(self.w2q, self.w2s)


def quantize_expert(w1: np.ndarray, w2: np.ndarray, pow2: bool = False) -> ExpertWeights:
    """128x128 block quantisation of one expert's fp32 masters (power-of-two scales with pow2)."""
    w1q, w1s = O.moe_quant_fp8_block(w1, 128, pow2)
    w2q, w2s = O.moe_quant_fp8_block(w2, 128, pow2)
    return ExpertWeights(w1q, w1s, w2q, w2s)


def quantize_expert_fp4(w1: np.ndarray, w2: np.ndarray) -> ExpertWeights:
    """FP4 (E2M1 in 1x32 blocks along the input dimension, E8M0 scales) quantisation of one
    expert's fp32 masters: the 4-bit variant of the expert weights, with the activations kept in
    FP8 (power-of-two 1x128 scales)."""
    w1q, w1e = O.quant_mxfp4(np.asarray(w1, np.float32))
    w2q, w2e = O.quant_mxfp4(np.asarray(w2, np.float32))
    return ExpertWeights(w1q, w1e, w2q, w2e, fp4=True)


@dataclass
class OracleLayer:
    """Router parameters plus a way to obtain each expert's quantised weights.

    ``expert(e)`` returns ExpertWeights for routed expert e in [0,E) and, when ``shared`` is
    set, for the shared expert at index E."""
    wg: np.ndarray                       # [E,H] fp32
    bias: Optional[np.ndarray]           # [E] fp32 or None
    cfg: O.RouterCfg
    shared: bool
    act: str                             # "f32" or "bf16"
    F: int
    expert: Callable[[int], ExpertWeights]
    pow2: bool = False                   # power-of-two block scales for activations and h (the
                                         # expert weights come from ``expert`` as they are)
    _cache: dict = field(default_factory=dict)

    def get(self, e: int) -> ExpertWeights:
        if e not in self._cache:
            self._cache[e] = self.expert(e)
        return self._cache[e]

    @property
    def E(self) -> int:
        return int(self.cfg.num_experts)

    @property
    def groups(self) -> int:
        return self.E + (1 if self.shared else 0)


def to_act(y: np.ndarray, act: str) -> np.ndarray:
    """Store rows in the activation dtype (fp64 -> fp32, then -> bf16 when act is bf16)."""
    y32 = np.asarray(y, np.float32)
    return O.round_to_bf16(y32) if act == "bf16" else y32


def residual_add(x: np.ndarray, out: np.ndarray, act: str) -> np.ndarray:
    """A MoE layer on a residual branch, stacked: the next layer's input is the fp32 sum of the
    layer input and the layer output as stored in the activation dtype, rounded once more to the
    activation dtype (reading R23 of the replay stack: "the config-3 layer stacked 4 deep" says
    nothing of what lies between the layers; a residual connection with no attention or norm is the
    plainest reading)."""
    s32 = np.asarray(x, np.float32) + to_act(out, act).astype(np.float32)   # one IEEE fp32 add
    return to_act(s32, act)


def route_or_replay(layer: OracleLayer, z: np.ndarray, replay: Optional[np.ndarray] = None,
                    record: Optional[np.ndarray] = None):
    if replay is not None:
        idx, w, bad = O.moe_replay_route(z, layer.cfg, replay)
        return idx, w, bad
    idx, w = O.moe_route(z, layer.cfg, record=record)
    return idx, w, 0


def forward_dispatch(layer: OracleLayer, x: np.ndarray, replay=None, record=None) -> dict:
    """Full layer over all T tokens of x ([T,H] fp32, bf16 values already widened)."""
    E, F = layer.E, layer.F
    z = O.moe_gate_logits(x, layer.wg, layer.bias)
    idx, w, bad = route_or_replay(layer, z, replay, record)
    xq, xs = O.moe_quant_fp8_block(x, 1, layer.pow2)
    counts, offsets, dest, src = O.moe_dispatch(idx, E, layer.shared)
    aq, as_ = O.permute_rows(xq, src), O.permute_rows(xs, src)
    G = layer.groups
    w1q = np.stack([layer.get(g).w1q for g in range(G)])
    w1s = np.stack([layer.get(g).w1s for g in range(G)])
    w2q = np.stack([layer.get(g).w2q for g in range(G)])
    w2s = np.stack([layer.get(g).w2s for g in range(G)])
    gemm = O.moe_grouped_gemm_fp4w if layer.get(0).fp4 else O.moe_grouped_gemm_fp8
    g1 = gemm(aq, as_, offsets, w1q, w1s)
    h = O.swiglu(g1, F)
    hq, hs = O.moe_quant_fp8_block(h, 1, layer.pow2)
    y = gemm(hq, hs, offsets, w2q, w2s)
    y_act = to_act(y, layer.act)
    T = x.shape[0]
    y_sh = y_act[offsets[E]:offsets[E] + T] if layer.shared else None
    out = O.moe_combine(y_act, dest, w, y_sh)
    return dict(z=z, idx=idx, w=w, bad=bad, xq=xq, xs=xs, counts=counts, offsets=offsets, dest=dest,
                src=src, aq=aq, as_=as_, g1=g1, h=h, hq=hq, hs=hs, y=y, y_act=y_act, out=out)


def expert_ffn(ew: ExpertWeights, xq: np.ndarray, xs: np.ndarray, F: int, act: str, pow2: bool = False):
    """FFN_e on already-quantised activation rows: returns (g1, h, hq, hs, y, y_act)."""
    g1 = O.dequant_act(xq, xs) @ ew.w1().T
    h = O.swiglu(g1, F)
    hq, hs = O.moe_quant_fp8_block(h, 1, pow2)
    y = O.dequant_act(hq, hs) @ ew.w2().T
    return g1, h, hq, hs, y, to_act(y, act)


def forward_token(layer: OracleLayer, x_rows: np.ndarray, replay_rows: Optional[np.ndarray] = None,
                  dense: bool = False) -> dict:
    """Per-token evaluation with no dispatch.  x_rows: [n,H] fp32 (the sampled tokens);
    replay_rows: [k,n] int32 recorded indices for those tokens, or None to route."""
    E, F = layer.E, layer.F
    z = O.moe_gate_logits(x_rows, layer.wg, layer.bias)
    idx, w, bad = route_or_replay(layer, z, replay_rows)
    xq, xs = O.moe_quant_fp8_block(x_rows, 1, layer.pow2)
    n, H = x_rows.shape
    out = np.zeros((n, H), np.float64)
    for t in range(n):
        if dense:
            gate = np.zeros(E, np.float64)
            for j in range(idx.shape[1]):
                if idx[t, j] >= 0:
                    gate[idx[t, j]] = w[t, j]
            for e in range(E):
                y_act = expert_ffn(layer.get(e), xq[t:t + 1], xs[t:t + 1], F, layer.act, layer.pow2)[5]
                out[t] += gate[e] * y_act[0].astype(np.float64)
        else:
            for j in range(idx.shape[1]):
                e = int(idx[t, j])
                if e < 0:
                    continue
                y_act = expert_ffn(layer.get(e), xq[t:t + 1], xs[t:t + 1], F, layer.act, layer.pow2)[5]
                out[t] += float(w[t, j]) * y_act[0].astype(np.float64)
        if layer.shared:
            y_act = expert_ffn(layer.get(E), xq[t:t + 1], xs[t:t + 1], F, layer.act, layer.pow2)[5]
            out[t] += y_act[0].astype(np.float64)
    return dict(z=z, idx=idx, w=w, bad=bad, xq=xq, xs=xs, out=out)


def forward_unquantized(layer: OracleLayer, x_rows: np.ndarray, masters: Callable[[int], tuple]) -> np.ndarray:
    """Context only (not a parity reference): the same routing with fp64 unquantised experts,
    to report how far FP8 block quantisation moves the layer output."""
    E, F = layer.E, layer.F
    z = O.moe_gate_logits(x_rows, layer.wg, layer.bias)
    idx, w, _ = route_or_replay(layer, z)
    xd = np.asarray(x_rows, np.float64)
    out = np.zeros_like(xd)
    for t in range(xd.shape[0]):
        experts = [(int(idx[t, j]), float(w[t, j])) for j in range(idx.shape[1])]
        if layer.shared:
            experts.append((E, 1.0))
        for e, we in experts:
            w1, w2 = masters(e)
            g = xd[t] @ np.asarray(w1, np.float64).T
            h = g[:F] / (1.0 + np.exp(-g[:F])) * g[F:]
            out[t] += we * (h @ np.asarray(w2, np.float64).T)
    return out


def rel_err(got, ref) -> float:
    """max |got - ref| / max |ref| (the tolerance metric for GEMM and combine outputs)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    if den == 0.0:
        return float(np.max(np.abs(got))) if got.size else 0.0
    return float(np.max(np.abs(got - ref))) / den


def forward_sampled(layer: OracleLayer, x_rows: np.ndarray, replay_rows: Optional[np.ndarray] = None,
                    workers: int = 1) -> dict:
    """Per-token evaluation of sampled tokens, in matrix form: route each token, then apply each
    used expert once to all sampled rows that selected it (no dispatch permutation, no shared
    state between tokens beyond the expert weights).  Same values as ``forward_token``.
    ``workers`` > 1 evaluates the experts on that many threads (each expert's arithmetic is
    unchanged; only the wall time differs)."""
    E, F = layer.E, layer.F
    z = O.moe_gate_logits(x_rows, layer.wg, layer.bias)
    idx, w, bad = route_or_replay(layer, z, replay_rows)
    xq, xs = O.moe_quant_fp8_block(x_rows, 1, layer.pow2)
    n, H = x_rows.shape
    ys = {}
    users = {}
    for t in range(n):
        for j in range(idx.shape[1]):
            if idx[t, j] >= 0:
                users.setdefault(int(idx[t, j]), []).append((t, j))
    def one_expert(item):
        e, lst = item
        rows = np.array([t for t, _ in lst])
        return expert_ffn(layer.get(e), xq[rows], xs[rows], F, layer.act, layer.pow2)[5]

    items = list(users.items())
    if workers > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(workers) as ex:
            results = list(ex.map(one_expert, items))
    else:
        results = [one_expert(it) for it in items]
    for (e, lst), y_act in zip(items, results):
        for (t, j), yr in zip(lst, y_act):
            ys[(t, j)] = yr
    out = np.zeros((n, H), np.float64)
    for t in range(n):
        for j in range(idx.shape[1]):
            if idx[t, j] >= 0:
                out[t] += float(w[t, j]) * ys[(t, j)].astype(np.float64)
    if layer.shared:
        y_act = expert_ffn(layer.get(E), xq, xs, F, layer.act, layer.pow2)[5]
        out += y_act.astype(np.float64)
    return dict(z=z, idx=idx, w=w, bad=bad, xq=xq, xs=xs, out=out, experts=sorted(users))
