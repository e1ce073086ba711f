"""Pins of the backward oracle (CPU only).

* Chain rule: with every quantisation switched off, the oracle's backward equals torch.autograd
  (fp64) applied to an independent torch composition of the same layer (router score function,
  normalisation, SwiGLU experts, weighted combine, shared expert) with the selection held fixed,
  for all four router forms (sigmoid / softmax, renormalised or not), with and without bias.
* Quantisation placement: the FP8 backward stays within FP8 rounding of the unquantised chain
  rule on the same forward quantities, and its gradient codes are the pinned 1x128 quantisation
  of the fp32 row gradients (dY bit for bit: a single fp32 product feeds it).
* Dispatch-free evaluation: per-token backward equals the grouped backward.
* Invariants of the router backward: the renormalised and softmax forms are unchanged by a common
  shift of the logits, so their dz sums to zero per token.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle as O
import oracle.backward as B
import oracle.layer as L
import synth

CASES = {
    # softmax top-2 renormalised, no bias, fp32 activations
    "tiny": synth.CONFIGS["tiny"],
    # softmax top-6 not renormalised, with bias
    "decode_small": replace(synth.CONFIGS["decode"], name="decode_small", T=24, H=256, E=16, F=128, k=6),
    # sigmoid, 8 groups keep 4, top-8 renormalised, shared expert
    "prefill_small": replace(synth.CONFIGS["prefill"], name="prefill_small", T=20, H=256, E=32, F=128, k=8),
    # sigmoid top-4 not renormalised, shared expert, bias
    "sigmoid_plain": replace(synth.CONFIGS["prefill"], name="sigmoid_plain", T=20, H=256, E=16, F=128, k=4,
                             renorm=False, n_group=1, topk_group=1),
}


def rcfg(cfg):
    return O.router_cfg(cfg.E, cfg.k, O.SOFTMAX if cfg.score_fn == "softmax" else O.SIGMOID, cfg.renorm,
                        cfg.n_group, cfg.topk_group, cfg.group_score_topk)


def masters(cfg):
    G = cfg.E + (1 if cfg.shared else 0)
    w = [synth.make_expert(cfg, g, 0, "cpu") for g in range(G)]
    return [a.double().numpy() for a, _ in w], [b.double().numpy() for _, b in w]


def gate(cfg, with_bias=True):
    wg, b = synth.make_gate(cfg, 0, "cpu")
    if not with_bias:
        b = None
    elif b is None:
        b = torch.from_numpy(np.random.default_rng(5).normal(0, 0.5, cfg.E).astype(np.float32))
    return wg.double().numpy(), (None if b is None else b.double().numpy())


def dout_for(cfg, seed=11):
    return np.random.default_rng(seed).standard_normal((cfg.T, cfg.H)).astype(np.float32)


def torch_reference(cfg, x, wg, b, W1, W2, idx, dout):
    """torch.autograd through the real-valued layer with the selection idx held fixed."""
    F = cfg.F
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    wgt = torch.tensor(wg, dtype=torch.float64, requires_grad=True)
    W1t = [torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in W1]
    W2t = [torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in W2]
    bt = torch.tensor(b, dtype=torch.float64, requires_grad=True) if b is not None else None
    z = xt @ wgt.T + (bt if bt is not None else 0.0)
    z.retain_grad()
    sc = torch.sigmoid(z) if cfg.score_fn == "sigmoid" else torch.softmax(z, dim=1)
    it = torch.tensor(idx, dtype=torch.int64)
    sel = sc.gather(1, it)
    w = sel / sel.sum(dim=1, keepdim=True) if cfg.renorm else sel
    w.retain_grad()

    def ffn(rows, g):
        a = rows @ W1t[g].T
        h = torch.nn.functional.silu(a[:, :F]) * a[:, F:]
        return h @ W2t[g].T

    out = torch.zeros_like(xt)
    for e in range(cfg.E):
        for j in range(cfg.k):
            m = (it[:, j] == e)
            if m.any():
                out = out.index_add(0, m.nonzero()[:, 0], w[m, j][:, None] * ffn(xt[m], e))
    if cfg.shared:
        out = out + ffn(xt, cfg.E)
    (out * torch.tensor(dout, dtype=torch.float64)).sum().backward()
    zero = lambda t, a: t.grad.numpy() if t.grad is not None else np.zeros_like(a)
    return dict(dx=xt.grad.numpy(), dwg=wgt.grad.numpy(), db=None if bt is None else bt.grad.numpy(),
                dw=w.grad.numpy(), dz=z.grad.numpy(), w=w.detach().numpy(), out=out.detach().numpy(),
                dW1=np.stack([zero(t, a) for t, a in zip(W1t, W1)]), dW2=np.stack([zero(t, a) for t, a in zip(W2t, W2)]))


def real_forward_rows(cfg, x, idx, W1, W2):
    """Forward quantities the backward consumes, real-valued: dispatch, GEMM1 output, expert rows."""
    counts, offsets, dest, src = O.moe_dispatch(idx, cfg.E, cfg.shared)
    rows = int(offsets[-1])
    g1 = np.zeros((rows, 2 * cfg.F))
    y = np.zeros((rows, cfg.H))
    for g in range(len(W1)):
        r0, r1 = int(offsets[g]), int(offsets[g + 1])
        if r1 > r0:
            a = x[src[r0:r1]].astype(np.float64) @ W1[g].T
            g1[r0:r1] = a
            h = a[:, :cfg.F] / (1 + np.exp(-a[:, :cfg.F])) * a[:, cfg.F:]
            y[r0:r1] = h @ W2[g].T
    return offsets, dest, g1, y, src


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("with_bias", [False, True])
def test_unquantised_backward_equals_autograd(name, with_bias):
    cfg = CASES[name]
    x = synth.make_x(cfg, "cpu").float().numpy()
    wg, b = gate(cfg, with_bias)
    W1, W2 = masters(cfg)
    z = x.astype(np.float64) @ wg.T + (b if b is not None else 0.0)
    idx, _ = O.moe_route(z.astype(np.float32), rcfg(cfg))
    dout = dout_for(cfg)
    ref = torch_reference(cfg, x, wg, b, W1, W2, idx, dout)
    offsets, dest, g1, y, src = real_forward_rows(cfg, x, idx, W1, W2)
    got = B.backward_core(dout, x, z, idx, ref["w"], dest, offsets, y, g1, rcfg(cfg), wg, W1, W2, cfg.F,
                          cfg.shared, quant=False, src=src)
    # the oracle's own roundings: dY = fp32(w) * fp32(dout), and h, dG rounded to fp32 (the
    # weight gradients' operands), i.e. ~2^-24 relative
    for key in ("dw", "dz", "dx", "dwg", "dW1", "dW2"):
        assert L.rel_err(got[key], ref[key]) < 1e-6, (key, L.rel_err(got[key], ref[key]))
    if b is not None:
        assert L.rel_err(got["db"], ref["db"]) < 1e-6
    # the expert-path part alone is nonzero and so is the router part (both terms are exercised)
    assert np.abs(got["dx_experts"]).max() > 0 and np.abs(got["dx_router"]).max() > 0


def quantised_case(name, pow2=False):
    cfg = CASES[name]
    rc = rcfg(cfg)
    wg, b = synth.make_gate(cfg, 0, "cpu")

    def expert(e):
        w1, w2 = synth.make_expert(cfg, e, 0, "cpu")
        return L.quantize_expert(w1.numpy(), w2.numpy(), pow2)

    lay = L.OracleLayer(wg=wg.numpy(), bias=None if b is None else b.numpy(), cfg=rc, shared=cfg.shared,
                        act=cfg.act, F=cfg.F, expert=expert, pow2=pow2)
    x = synth.make_x(cfg, "cpu").float().numpy()
    return cfg, lay, x


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("pow2", [False, True])
def test_quantised_backward_codes_and_error(name, pow2):
    cfg, lay, x = quantised_case(name, pow2)
    fwd = L.forward_dispatch(lay, x)
    dout = dout_for(cfg)
    got = B.backward_dispatch(lay, fwd, x, dout)
    # dY is one fp32 product per element, quantised by the pinned 1x128 rule: recompute both
    T, k = fwd["dest"].shape
    rows = int(fwd["offsets"][-1])
    dY = np.zeros((rows, cfg.H), np.float32)
    for t in range(T):
        for j in range(k):
            if fwd["dest"][t, j] >= 0:
                dY[fwd["dest"][t, j]] = np.float32(fwd["w"][t, j]) * dout[t]
        if cfg.shared:
            dY[fwd["offsets"][cfg.E] + t] = dout[t]
    assert np.array_equal(got["dY"], dY)
    q, s = O.moe_quant_fp8_block(dY, 1, pow2)
    assert np.array_equal(got["dYq"], q) and np.array_equal(got["dYs"], s)
    # the FP8 backward against the real-valued chain rule on the same forward quantities
    G = lay.groups
    w1 = [O.dequant_weight(lay.get(g).w1q, lay.get(g).w1s) for g in range(G)]
    w2 = [O.dequant_weight(lay.get(g).w2q, lay.get(g).w2s) for g in range(G)]
    real = B.backward_core(dout, x, fwd["z"], fwd["idx"], fwd["w"], fwd["dest"], fwd["offsets"], fwd["y_act"],
                           fwd["g1"], lay.cfg, lay.wg, w1, w2, cfg.F, cfg.shared, quant=False, src=fwd["src"])
    for key in ("dh", "dA", "dx", "dW1", "dW2"):
        e = L.rel_err(got[key], real[key])
        # one FP8 rounding per operand (2^-4 relative, coarser in the subnormal range); the weight
        # gradients sum few rows per expert here, so their max error is less averaged
        assert e < (1e-1 if key.startswith("dW") else 6e-2), (key, e)
    # quantisation changed something (the two paths are not the same computation)
    assert L.rel_err(got["dA"], real["dA"]) > 1e-4 and L.rel_err(got["dW1"], real["dW1"]) > 1e-4
    # the 128x1 operand codes of dW2 are the pinned 1x128 rule applied to the transposed,
    # zero-padded segments of the fp32 dY (bitwise reproducible: one product per element)
    seg = B.colwise_segments(dY, fwd["offsets"], True, pow2)
    g0 = next(g for g in range(len(fwd["offsets"]) - 1) if fwd["offsets"][g + 1] > fwd["offsets"][g])
    r0, r1 = int(fwd["offsets"][g0]), int(fwd["offsets"][g0 + 1])
    pad = np.zeros((-(-(r1 - r0) // 128) * 128, cfg.H), np.float32)
    pad[:r1 - r0] = dY[r0:r1]
    q0, s0 = O.moe_quant_fp8_block(np.ascontiguousarray(pad.T), 1, pow2)
    assert np.array_equal(seg[g0][0], q0) and np.array_equal(seg[g0][1], s0)
    assert np.array_equal(got["dw"], real["dw"]) and np.array_equal(got["dz"], real["dz"])


@pytest.mark.parametrize("name", ["tiny", "prefill_small"])
def test_per_token_backward_equals_grouped(name):
    cfg, lay, x = quantised_case(name)
    fwd = L.forward_dispatch(lay, x)
    dout = dout_for(cfg)
    full = B.backward_dispatch(lay, fwd, x, dout)
    pick = np.array([0, 3, cfg.T - 1])
    tok = B.backward_token(lay, x[pick], dout[pick])
    for key in ("dw", "dz", "dx_experts", "dx_router", "dx"):
        assert L.rel_err(tok[key], full[key][pick]) < 1e-9, key


@pytest.mark.parametrize("name", list(CASES))
def test_router_backward_shift_invariance(name):
    cfg = CASES[name]
    rng = np.random.default_rng(3)
    z = rng.standard_normal((cfg.T, cfg.E))
    idx, _ = O.moe_route(z.astype(np.float32), rcfg(cfg))
    dw = rng.standard_normal((cfg.T, cfg.k))
    dz = B.route_backward(z, idx, dw, rcfg(cfg))
    if cfg.score_fn == "softmax":
        # softmax weights (renormalised or not) are unchanged by z -> z + c: dz sums to zero
        assert np.abs(dz.sum(axis=1)).max() < 1e-12
    elif cfg.renorm:
        # s_j / sum s is unchanged by scaling every selected score: sum_j s_j ds_j = 0 with
        # ds_j = dz_j / (s_j (1 - s_j)), i.e. sum_j dz_j / (1 - s_j) = 0
        s = 1 / (1 + np.exp(-np.take_along_axis(z, idx.astype(np.int64), axis=1)))
        dzs = np.take_along_axis(dz, idx.astype(np.int64), axis=1)
        assert np.abs((dzs / (1 - s)).sum(axis=1)).max() < 1e-12
    # only the selected experts (or, for plain softmax, every expert) carry gradient
    if not (cfg.score_fn == "softmax" and not cfg.renorm):
        mask = np.zeros_like(dz, bool)
        np.put_along_axis(mask, idx.astype(np.int64), True, axis=1)
        assert np.all(dz[~mask] == 0)


@pytest.mark.parametrize("name", ["tiny", "decode_small", "prefill_small"])
@pytest.mark.parametrize("pow2", [False, True])
def test_wgrad_expert_equals_grouped_weight_gradients(name, pow2):
    """The one-expert weight gradient (the reference of the full-size GPU weight-gradient tests)
    equals the grouped backward's dW1[e], dW2[e] for every expert, the shared one included; an
    expert that no token selected has zero gradients."""
    cfg, lay, x = quantised_case(name, pow2)
    fwd = L.forward_dispatch(lay, x)
    dout = dout_for(cfg)
    full = B.backward_dispatch(lay, fwd, x, dout)
    for e in range(lay.groups):
        if fwd["counts"][e] == 0:
            assert not full["dW1"][e].any() and not full["dW2"][e].any()
            continue
        dW1, dW2 = B.wgrad_expert(lay, x, dout, e)
        assert L.rel_err(dW1, full["dW1"][e]) < 1e-12, ("dW1", e)
        assert L.rel_err(dW2, full["dW2"][e]) < 1e-12, ("dW2", e)


def test_wgrad_expert_follows_replayed_routing():
    cfg, lay, x = quantised_case("prefill_small")
    payload = np.zeros((cfg.k, cfg.T), np.int32)
    L.forward_dispatch(lay, x, record=payload)
    # replay a rotated routing (every token's experts shifted by one), so the rows differ from routing
    rot = np.ascontiguousarray((payload + 1) % cfg.E)
    fwd = L.forward_dispatch(lay, x, replay=rot)
    dout = dout_for(cfg)
    full = B.backward_dispatch(lay, fwd, x, dout)
    for e in sorted(set(int(v) for v in rot[:, :3].reshape(-1)))[:4]:
        dW1, dW2 = B.wgrad_expert(lay, x, dout, e, replay=rot)
        assert L.rel_err(dW1, full["dW1"][e]) < 1e-12 and L.rel_err(dW2, full["dW2"][e]) < 1e-12
        d_routed = B.wgrad_expert(lay, x, dout, e)
        assert L.rel_err(d_routed[1], full["dW2"][e]) > 1e-6
