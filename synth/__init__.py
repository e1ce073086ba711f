"""Seeded synthetic inputs for the block-scaled FP8 MoE layer.

This module is the only code that both the HIP path's callers and the CPU oracle's callers
use.  It holds the workload records and the seeded random draws, and none of the layer's
arithmetic: no routing, quantisation, dispatch, GEMM or combine happens here.

Every tensor is drawn from its own stream: a 64-bit seed derived with numpy's SeedSequence from
(workload seed, tensor id, layer, expert, part) feeds a ``torch.Generator`` on the requested
device.  A given (workload, tensor, device) therefore always yields the same values, and any
single expert can be regenerated on its own.  The CPU and GPU generators produce different
streams, so a test draws each input once, on one device, and hands the *same* values to both
sides (uploading or downloading as needed).

Value distributions follow the workload descriptions: activations N(0,1) (bf16 by
round-to-nearest-even from fp32 where the workload is bf16), expert weights N(0, 1/sqrt(fan_in)),
router gate N(0, 1/sqrt(H)) unless a workload names another scale, an optional per-expert
logit bias (normal, or Zipf-shaped), and an optional weight perturbation N(0, 1e-3).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import Optional

import numpy as np
import torch

# tensor ids of the per-tensor streams
X, WG, BIAS, W1, W2, SW1, SW2, PERTURB, ZIPF, STAGE, DOUT = range(11)


@dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int                     # tokens per layer call (chunk size for chunked workloads)
    H: int                     # hidden size
    E: int                     # routed experts
    F: int                     # expert FFN width
    k: int                     # experts per token
    shared: bool               # one always-on shared expert
    score_fn: str              # "softmax" | "sigmoid"
    renorm: bool
    n_group: int = 1
    topk_group: int = 1
    group_score_topk: int = 2
    act: str = "bf16"          # activation dtype: "f32" | "bf16"
    wg_std: Optional[float] = None      # None -> 1/sqrt(H)
    bias: str = "none"         # "none" | "normal" | "zipf"
    bias_std: float = 0.0
    zipf_s: float = 0.0
    total_tokens: int = 0      # >T for chunked workloads (T is then the chunk size)
    layers: int = 1
    perturb_std: float = 0.0
    seed: int = 0

    @property
    def gate_std(self) -> float:
        return self.wg_std if self.wg_std is not None else 1.0 / math.sqrt(self.H)

    @property
    def groups(self) -> int:
        return self.E + (1 if self.shared else 0)

    @property
    def rows(self) -> int:
        return self.T * self.k + (self.T if self.shared else 0)

    @property
    def chunks(self) -> int:
        return max(1, (self.total_tokens or self.T) // self.T)


CONFIGS = {
    # Tiny MoE layer: 64 tokens, hidden 256, 8 experts, FFN 512, top-2 softmax renormalised, fp32 acts.
    "tiny": LayerConfig("tiny", T=64, H=256, E=8, F=512, k=2, shared=False, score_fn="softmax", renorm=True,
                        act="f32", seed=0),
    # Decode-shaped: 256 tokens, hidden 4096, 64 experts, FFN 1408, top-6 softmax (not renormalised),
    # gate N(0, 0.02) plus per-expert bias N(0, 0.5) for load skew.
    "decode": LayerConfig("decode", T=256, H=4096, E=64, F=1408, k=6, shared=False, score_fn="softmax",
                          renorm=False, act="bf16", wg_std=0.02, bias="normal", bias_std=0.5, seed=1),
    # Prefill-shaped: 16384 tokens, hidden 6144, 256 routed + 1 shared expert, FFN 2048, top-8 sigmoid,
    # 8 groups / best 4, renormalised.
    "prefill": LayerConfig("prefill", T=16384, H=6144, E=256, F=2048, k=8, shared=True, score_fn="sigmoid",
                           renorm=True, n_group=8, topk_group=4, group_score_topk=2, act="bf16", seed=2),
    # Long context: 131072 tokens in 8192-token chunks, prefill dims, no shared expert, Zipf(1.2) bias.
    "longctx": LayerConfig("longctx", T=8192, H=6144, E=256, F=2048, k=8, shared=False, score_fn="sigmoid",
                           renorm=True, n_group=8, topk_group=4, group_score_topk=2, act="bf16", bias="zipf",
                           zipf_s=1.2, total_tokens=131072, seed=3),
    # Router-replay stack: the prefill layer 4 deep at 32768 tokens; record with W, replay on W + N(0,1e-3).
    "r3": LayerConfig("r3", T=32768, H=6144, E=256, F=2048, k=8, shared=True, score_fn="sigmoid", renorm=True,
                      n_group=8, topk_group=4, group_score_topk=2, act="bf16", layers=4, perturb_std=1e-3, seed=4),
}


def stream_seed(seed: int, tensor_id: int, layer: int = 0, expert: int = 0, part: int = 0) -> int:
    ss = np.random.SeedSequence(entropy=int(seed), spawn_key=(int(tensor_id), int(layer), int(expert), int(part)))
    s = ss.generate_state(2, dtype=np.uint32)
    return int((int(s[0]) << 31) ^ int(s[1])) & ((1 << 63) - 1)


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def randn(shape, seed: int, tensor_id: int, layer: int = 0, expert: int = 0, part: int = 0,
          device="cpu", std: float = 1.0) -> torch.Tensor:
    """fp32 N(0, std^2) draw from the stream (seed, tensor_id, layer, expert, part)."""
    g = _gen(device, stream_seed(seed, tensor_id, layer, expert, part))
    t = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t


def to_act(x32: torch.Tensor, act: str) -> torch.Tensor:
    """fp32 draw -> activation dtype (bf16 by round-to-nearest-even)."""
    return x32.to(torch.bfloat16) if act == "bf16" else x32


def make_x(cfg: LayerConfig, device="cpu", chunk: int = 0, tokens: Optional[int] = None) -> torch.Tensor:
    """Activations [T,H] in the activation dtype (chunk c of a chunked workload)."""
    T = cfg.T if tokens is None else tokens
    return to_act(randn((T, cfg.H), cfg.seed, X, 0, chunk, device=device), cfg.act)


def make_dout(cfg: LayerConfig, device="cpu", chunk: int = 0) -> torch.Tensor:
    """Output gradient [T,H] for the backward, N(0,1) in the activation dtype."""
    return to_act(randn((cfg.T, cfg.H), cfg.seed, DOUT, 0, chunk, device=device), cfg.act)


def zipf_bias(cfg: LayerConfig) -> np.ndarray:
    """Per-expert logit bias ln p_r(e), p_r proportional to r^-s, with rank r(e) = 1 + pi(e) for a
    seeded permutation pi (fp64 on the host, returned as fp32)."""
    rng = np.random.Generator(np.random.PCG64(stream_seed(cfg.seed, ZIPF)))
    perm = rng.permutation(cfg.E)
    r = np.arange(1, cfg.E + 1, dtype=np.float64)
    p = r ** (-cfg.zipf_s)
    p /= p.sum()
    return np.log(p[perm]).astype(np.float32)


def make_gate(cfg: LayerConfig, layer: int = 0, device="cpu", perturbed: bool = False):
    """Router gate Wg [E,H] fp32 and bias [E] fp32 (or None)."""
    wg = randn((cfg.E, cfg.H), cfg.seed, WG, layer, device=device, std=cfg.gate_std)
    if perturbed:
        wg = wg + randn((cfg.E, cfg.H), cfg.seed, PERTURB, layer, 0, 0, device=device, std=cfg.perturb_std)
    if cfg.bias == "normal":
        b = randn((cfg.E,), cfg.seed, BIAS, layer, device=device, std=cfg.bias_std)
    elif cfg.bias == "zipf":
        b = torch.from_numpy(zipf_bias(cfg)).to(device)
    else:
        b = None
    return wg, b


def make_expert(cfg: LayerConfig, e: int, layer: int = 0, device="cpu", perturbed: bool = False):
    """fp32 masters of expert e: W1 [2F,H] (gate rows then up rows) and W2 [H,F].  e == E is the
    shared expert (own streams)."""
    t1, t2 = (SW1, SW2) if e == cfg.E else (W1, W2)
    w1 = randn((2 * cfg.F, cfg.H), cfg.seed, t1, layer, e, device=device, std=1.0 / math.sqrt(cfg.H))
    w2 = randn((cfg.H, cfg.F), cfg.seed, t2, layer, e, device=device, std=1.0 / math.sqrt(cfg.F))
    if perturbed:
        w1 = w1 + randn(w1.shape, cfg.seed, PERTURB, layer, e + 1, 1, device=device, std=cfg.perturb_std)
        w2 = w2 + randn(w2.shape, cfg.seed, PERTURB, layer, e + 1, 2, device=device, std=cfg.perturb_std)
    return w1, w2


def make_logits(cfg: LayerConfig, T: Optional[int] = None, device="cpu", part: int = 0) -> torch.Tensor:
    """Stage input for the router alone: logits [T,E] fp32 with the spread x.Wg would have
    (std gate_std*sqrt(H)) plus the workload's bias."""
    T = cfg.T if T is None else T
    z = randn((T, cfg.E), cfg.seed, STAGE, 0, 0, part, device=device, std=cfg.gate_std * math.sqrt(cfg.H))
    _, b = make_gate(cfg, 0, device="cpu") if cfg.bias != "none" else (None, None)
    if b is not None:
        z = z + b.to(device)[None, :]
    return z


def tie_logits(T: int, E: int, levels: int, seed: int, device="cpu") -> torch.Tensor:
    """Logits drawn from a coarse grid of `levels` values, so that many keys tie exactly."""
    g = _gen(device, stream_seed(seed, STAGE, 0, 0, 99))
    return (torch.randint(0, levels, (T, E), generator=g, device=device).to(torch.float32) - levels / 2) * 0.25


def random_codes(shape, seed: int, part: int, device="cpu") -> torch.Tensor:
    """Uniformly random finite e4m3 bytes (every code except the two NaNs 0x7F / 0xFF)."""
    g = _gen(device, stream_seed(seed, STAGE, 1, 0, part))
    c = torch.randint(0, 254, tuple(shape), generator=g, device=device, dtype=torch.uint8)
    c += (c >= 0x7F).to(torch.uint8)              # skip 0x7F; 0xFE is the largest code drawn
    return c


def random_scales(shape, seed: int, part: int, device="cpu", lo: float = 2.0 ** -12, hi: float = 2.0 ** -4):
    """Positive fp32 block scales, log-uniform in [lo, hi]."""
    g = _gen(device, stream_seed(seed, STAGE, 2, 0, part))
    u = torch.rand(tuple(shape), generator=g, device=device, dtype=torch.float32)
    return torch.exp2(math.log2(lo) + u * (math.log2(hi) - math.log2(lo)))


# e4m3 byte codes of the integers -8..8, from the format definition (bias 7, 3 mantissa bits):
# v = 2^e (1 + m/8) -> code (e + 7) << 3 | m, negative values set bit 7.
E4M3_INT_CODES = {0: 0x00, 1: 0x38, 2: 0x40, 3: 0x44, 4: 0x48, 5: 0x4A, 6: 0x4C, 7: 0x4E, 8: 0x50}


def integer_codes(shape, seed: int, part: int, lo: int = -8, hi: int = 8, device="cpu"):
    """e4m3 codes of random integers in [lo, hi] and the integers themselves (int64)."""
    g = _gen("cpu", stream_seed(seed, STAGE, 3, 0, part))
    v = torch.randint(lo, hi + 1, tuple(shape), generator=g, dtype=torch.int64)
    table = torch.tensor([E4M3_INT_CODES[abs(i)] | (0x80 if i < 0 else 0) for i in range(-8, 9)], dtype=torch.uint8)
    return table[v + 8].to(device), v


def routing_indices(cfg: LayerConfig, T: int, seed_part: int = 0, device="cpu") -> torch.Tensor:
    """Stage input for dispatch alone: per-token distinct expert ids [T,k] int32 drawn with
    probabilities that follow the workload's bias (uniform when it has none)."""
    g = _gen("cpu", stream_seed(cfg.seed, STAGE, 4, 0, seed_part))
    if cfg.bias == "zipf":
        logp = torch.from_numpy(zipf_bias(cfg)).double()
    elif cfg.bias == "normal":
        _, b = make_gate(cfg, 0, "cpu")
        logp = b.double()
    else:
        logp = torch.zeros(cfg.E, dtype=torch.float64)
    p = torch.softmax(logp, 0).expand(T, cfg.E)
    idx = torch.multinomial(p, cfg.k, replacement=False, generator=g).to(torch.int32)
    return idx.to(device)


def sample_tokens(T: int, n: int, seed: int) -> np.ndarray:
    """Sorted distinct token indices to sample (always includes the first and last token)."""
    rng = np.random.Generator(np.random.PCG64(stream_seed(seed, STAGE, 5)))
    n = min(n, T)
    pick = set(rng.choice(T, size=max(0, n - 2), replace=False).tolist()) | {0, T - 1}
    return np.array(sorted(pick), dtype=np.int64)


def with_tokens(cfg: LayerConfig, T: int) -> LayerConfig:
    return replace(cfg, T=T)
