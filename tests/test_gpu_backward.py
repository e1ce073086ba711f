"""Parity of the layer backward (HIP path, through the C ABI) against the backward oracle.

Stage by stage on shared seeded inputs: the weight-block transpose (bit-exact), the combine
backward (dY codes and scales bit-exact: one fp32 product feeds them; dw within fp32 summation),
the SwiGLU backward codes (the oracle's fp64 chain rounded to fp32, quantised by the pinned rule:
codes equal up to rare one-step boundary cases), the router backward and the gate backward (fp32
against fp64).  Whole layers: small layers on every token and every intermediate, and the decode-
and prefill-shaped layers at full size on sampled tokens, which the oracle evaluates per token
with no dispatch; the full-size dWg / db against the oracle's fp64 product of the same dz.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

import block_scaled_fp8_top_amd as M
import oracle as O
import oracle.backward as B
import oracle.layer as L
import synth
from block_scaled_fp8_top_amd.layer import MoELayer, prepare_backward_weights
from gpu_helpers import DEV, TOL, assert_equal, cfgs_for, gpu_weights, host, oracle_layer, rel_err, rows_host

pytestmark = pytest.mark.gpu

SMALL = {
    "tiny": synth.CONFIGS["tiny"],
    "decode_small": replace(synth.CONFIGS["decode"], name="decode_small", T=96, H=512, E=16, F=256, k=6),
    "prefill_small": replace(synth.CONFIGS["prefill"], name="prefill_small", T=80, H=256, E=32, F=256, k=8),
}


def _act(cfg):
    return torch.bfloat16 if cfg.act == "bf16" else torch.float32


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_transpose_blocks_exact():
    G, N, K = 3, 384, 256
    q = synth.random_codes((G, N, K), 5, 1, device=DEV)
    s = synth.random_scales((G, N // 128, K // 128), 5, 2, device=DEV)
    qt, st = M.moe_transpose_fp8_blocks(q, s)
    assert_equal("qt", host(qt), np.ascontiguousarray(np.transpose(host(q), (0, 2, 1))))
    assert_equal("st", host(st), np.ascontiguousarray(np.transpose(host(s), (0, 2, 1))))


def _routing(cfg, T, part=0, invalid=()):
    """Distinct per-token expert ids [T,k] (host int32); tokens in `invalid` routed nowhere (-1)."""
    idx = synth.routing_indices(cfg, T, seed_part=part).numpy().astype(np.int32)
    for t in invalid:
        idx[t] = -1
    return idx


@pytest.mark.parametrize("name,H,pow2", [("tiny", 256, False), ("decode", 4096, False), ("prefill", 2176, False),
                                         ("prefill", 6144, True), ("decode", 128, True)])
def test_combine_backward(name, H, pow2):
    cfg = replace(synth.CONFIGS[name], H=H)
    T = 300
    idx = _routing(cfg, T, invalid=(7, 299))
    counts, offsets, dest, src = O.moe_dispatch(idx, cfg.E, cfg.shared)
    rows = int(offsets[-1])
    act = _act(cfg)
    y = synth.to_act(synth.randn((rows, H), 9, synth.STAGE, 0, 0, 31, device=DEV), cfg.act)
    dout = synth.to_act(synth.randn((T, H), 9, synth.STAGE, 0, 0, 32, device=DEV), cfg.act)
    w = synth.random_scales((T, cfg.k), 9, 33, device=DEV, lo=0.01, hi=1.0)
    dest_d = torch.from_numpy(dest).to(DEV)
    off_d = torch.from_numpy(offsets).to(DEV)
    shared = off_d[cfg.E:cfg.E + 1] if cfg.shared else None
    dyq, dys, dw = M.moe_combine_backward(dout, y, dest_d, w, shared, pow2=pow2)
    dY, dw_ref = B.combine_backward(host(dout), host(y), dest, host(w), rows, int(offsets[cfg.E]) if cfg.shared else None)
    q, s = O.moe_quant_fp8_block(dY, 1, pow2)
    assert_equal("dyq", host(dyq), q)
    assert_equal("dys", host(dys), s)
    assert np.all(host(dw)[[7, 299]] == 0)
    assert rel_err(host(dw), dw_ref) < 1e-5
    assert act in (torch.float32, torch.bfloat16)


@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("rows,F", [(1, 128), (1000, 384), (4099, 2048)])
def test_swiglu_backward(rows, F, pow2):
    dh = synth.randn((rows, F), 11, synth.STAGE, 0, 0, 41, device=DEV, std=0.5)
    g = synth.randn((rows, 2 * F), 11, synth.STAGE, 0, 0, 42, device=DEV, std=2.0)
    dgq, dgs = M.moe_swiglu_backward_quant(dh, g, pow2=pow2)
    dG = B.swiglu_backward(host(dh), host(g), F)
    q, s = O.moe_quant_fp8_block(dG, 1, pow2)
    gs, gq = host(dgs), host(dgq)
    # scales: amax of fp32 values a few ulp apart (equal for power-of-two scales but at a boundary)
    assert np.max(np.abs(gs - s) / s) < 1e-5
    # codes: equal except where a value sits on a rounding boundary; then one step apart
    diff = gq != q
    assert diff.mean() < 1e-3, diff.mean()
    if diff.any():
        tab = O.e4m3_table()
        step = np.abs(tab[gq[diff]] - tab[q[diff]])
        assert np.all(step <= np.maximum(np.abs(tab[q[diff]]) / 8, 2.0 ** -9))


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "sigmoid_plain"])
def test_route_backward(name):
    base = synth.CONFIGS["prefill"] if name == "sigmoid_plain" else synth.CONFIGS[name]
    cfg = replace(base, renorm=False, n_group=1, topk_group=1) if name == "sigmoid_plain" else base
    T = 513
    gcfg, ocfg = cfgs_for(cfg)
    z = synth.make_logits(cfg, T, DEV)
    idx, _ = M.moe_route(z, gcfg)
    idx[[3, 500]] = -1   # tokens a replay rejected: no gradient
    dw = synth.randn((T, cfg.k), 13, synth.STAGE, 0, 0, 51, device=DEV)
    dz = M.moe_route_backward(z, idx, dw, gcfg)
    ref = B.route_backward(host(z), host(idx), host(dw), ocfg)
    assert np.all(host(dz)[[3, 500]] == 0)
    assert rel_err(host(dz), ref) < 1e-5


@pytest.mark.parametrize("T,H,E,act", [(100, 256, 8, "f32"), (1000, 264, 64, "bf16"), (16384, 6144, 256, "bf16")])
def test_gate_backward(T, H, E, act):
    dz = synth.randn((T, E), 17, synth.STAGE, 0, 0, 61, device=DEV, std=0.1)
    x = synth.to_act(synth.randn((T, H), 17, synth.STAGE, 0, 0, 62, device=DEV), act)
    wg = synth.randn((E, H), 17, synth.STAGE, 0, 0, 63, device=DEV, std=0.05)
    dx_in = synth.randn((T, H), 17, synth.STAGE, 0, 0, 64, device=DEV)
    dx, dwg, db = M.moe_gate_backward(dz, x, wg, dx_in=dx_in, dx_dtype=torch.float32)
    dx_r, dwg_r, db_r = B.gate_backward(host(dz), host(x), host(wg))
    assert rel_err(host(dx), host(dx_in) + dx_r) < 1e-5
    assert rel_err(host(dwg), dwg_r) < 1e-4
    assert rel_err(host(db), db_r) < 1e-4
    # bf16 output: one rounding of the fp32 sum
    dxb, _, _ = M.moe_gate_backward(dz, x, wg, dx_in=dx_in, dx_dtype=torch.bfloat16, want_db=False)
    assert torch.equal(dxb, dx.to(torch.bfloat16))


def _layer_pair(cfg, pow2=False):
    gw = gpu_weights(cfg, pow2=pow2)
    bw = prepare_backward_weights(gw)
    return gw, bw, oracle_layer(cfg, pow2=pow2)


@pytest.mark.parametrize("name,pow2", [("tiny", False), ("decode_small", False), ("prefill_small", False),
                                       ("prefill_small", True)])
def test_layer_backward_every_intermediate(name, pow2):
    cfg = SMALL[name]
    gw, bw, ol = _layer_pair(cfg, pow2)
    lay = MoELayer(gw, cfg.T, _act(cfg))
    x = synth.make_x(cfg, DEV)
    dout = synth.make_dout(cfg, DEV)
    lay.forward(x)
    g = lay.backward(x, dout, bw)
    torch.cuda.synchronize()
    r = L.forward_dispatch(ol, host(x))
    rb = B.backward_dispatch(ol, r, host(x), host(dout))
    n = int(r["offsets"][-1])
    b = lay.bwd
    # dY = w * dout with w bit-exact (routing is pinned): codes and scales bit-exact
    assert_equal("dyq", host(b["dyq"])[:n], rb["dYq"])
    assert_equal("dys", host(b["dys"])[:n], rb["dYs"])
    # fp32 GEMMs on identical codes against fp64
    assert rel_err(host(b["dh"])[:n], rb["dh"]) < 1e-4
    assert rel_err(host(b["g"])[:n], r["g1"]) < 1e-4
    assert rel_err(O.dequant_act(host(b["dgq"])[:n], host(b["dgs"])[:n]),
                   O.dequant_act(rb["dGq"], rb["dGs"])) < TOL
    assert rel_err(host(b["dA"])[:n], rb["dA"]) < TOL
    for key in ("dw", "dz", "dx", "dwg"):
        e = rel_err(host(g[key]), rb[key])
        print(f"{name} pow2={pow2} {key} err {e:.2e}")
        assert e < TOL, key
    if ol.bias is not None:
        assert rel_err(host(g["db"]), rb["db"]) < TOL
    else:
        assert g["db"] is None


def test_layer_backward_after_fused_replay():
    """Sigmoid replay runs fused (no logits written); the backward recomputes the logits."""
    cfg = SMALL["prefill_small"]
    gw, bw, ol = _layer_pair(cfg)
    lay = MoELayer(gw, cfg.T, _act(cfg))
    x = synth.make_x(cfg, DEV)
    dout = synth.make_dout(cfg, DEV)
    payload = torch.empty((cfg.k, cfg.T), dtype=torch.int32, device=DEV)
    lay.forward(x, record=payload)
    g_rec = {k: (v.clone() if v is not None else None) for k, v in lay.backward(x, dout, bw).items()}
    lay.forward(x, replay=payload)
    assert not lay.logits_valid
    g_rep = lay.backward(x, dout, bw)
    torch.cuda.synchronize()
    for key in ("dx", "dwg", "dw", "dz"):
        assert torch.equal(g_rep[key], g_rec[key]), key


@pytest.mark.parametrize("name,n", [("decode", 24), ("prefill", 4)])
def test_layer_backward_full_size_sampled(name, n):
    cfg = synth.CONFIGS[name]
    gw, bw, ol = _layer_pair(cfg)
    lay = MoELayer(gw, cfg.T, _act(cfg))
    x = synth.make_x(cfg, DEV)
    dout = synth.make_dout(cfg, DEV)
    lay.forward(x)
    g = lay.backward(x, dout, bw)
    torch.cuda.synchronize()
    toks = synth.sample_tokens(cfg.T, n, cfg.seed + 7)
    rt = B.backward_token(ol, rows_host(x, toks), rows_host(dout, toks))
    for key in ("dw", "dz", "dx"):
        e = rel_err(rows_host(g[key], toks), rt[key])
        print(f"{name} sampled {key} err {e:.2e}")
        assert e < TOL, key
    # the token-summed gradients at full size: the oracle's fp64 products of the same dz
    dz = host(g["dz"])
    _, dwg_r, db_r = B.gate_backward(dz, host(x), ol.wg)
    assert rel_err(host(g["dwg"]), dwg_r) < 1e-4
    if g["db"] is not None:
        assert rel_err(host(g["db"]), db_r) < 1e-4
    del lay, gw, bw
    _free()


@pytest.mark.parametrize("name,pow2", [("tiny", False), ("prefill_small", False), ("prefill_small", True)])
def test_training_forward_keeps_g(name, pow2):
    """GEMM1 of a training forward also stores its fp32 output: h codes and scales unchanged, G
    bitwise the store-epilogue recompute, and the backward's gradients bitwise unchanged."""
    cfg = SMALL[name]
    gw, bw, _ = _layer_pair(cfg, pow2)
    lay = MoELayer(gw, cfg.T, _act(cfg))
    x = synth.make_x(cfg, DEV)
    dout = synth.make_dout(cfg, DEV)
    lay.forward(x)
    hq, hs, out = lay.hq.clone(), lay.hs.clone(), lay.out.clone()
    ref = {k: (v.clone() if v is not None else None) for k, v in lay.backward(x, dout, bw).items()}
    g_re = lay.bwd["g"].clone()
    lay.bwd["g"].fill_(float("nan"))
    lay.forward(x, training=True)
    n = int(host(lay.disp.offsets)[-1])
    assert torch.equal(lay.hq[:n], hq[:n]) and torch.equal(lay.hs[:n], hs[:n]) and torch.equal(lay.out, out)
    assert torch.equal(lay.bwd["g"][:n], g_re[:n])
    got = lay.backward(x, dout, bw)
    torch.cuda.synchronize()
    for key in ("dx", "dwg", "dw", "dz"):
        assert torch.equal(got[key], ref[key]), key



def _segments(G, sizes_seed):
    """Group offsets with an empty group, a multiple of 128 and ragged sizes."""
    rng = np.random.default_rng(sizes_seed)
    counts = rng.integers(1, 300, G).astype(np.int32)
    counts[1] = 0
    counts[2] = 256
    counts[-1] = 129
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


@pytest.mark.parametrize("xdt,pow2", [("bf16", False), ("f32", False), ("bf16", True)])
def test_colwise_quant_rows(xdt, pow2):
    G, C, T = 7, 384, 900
    offsets = _segments(G, 3)
    rows = int(offsets[-1])
    x = synth.to_act(synth.randn((T, C), 21, synth.STAGE, 0, 0, 71, device=DEV), xdt)
    src = torch.from_numpy(np.random.default_rng(4).integers(0, T, rows).astype(np.int32)).to(DEV)
    scale = synth.random_scales((rows,), 21, 72, device=DEV, lo=0.01, hi=1.0)
    off_d = torch.from_numpy(offsets).to(DEV)
    tf = M.moe_wgrad_tiles(off_d)
    mt = M.wgrad_max_tiles(rows, G)
    qt, st = M.moe_colwise_quant_rows(x, off_d, tf, mt, src_row=src, row_scale=scale, pow2=pow2)
    vals = (host(scale)[:, None] * host(x)[host(src)]).astype(np.float32)
    segs = B.colwise_segments(vals, offsets, True, pow2)
    tfh = host(tf)
    assert tfh[-1] == sum(-(-int(c) // 128) for c in np.diff(offsets))
    for g in range(G):
        qg, sg = M.colwise_block(qt, st, tfh, g)
        assert_equal(f"codes g{g}", host(qg), segs[g][0])
        assert_equal(f"scales g{g}", host(sg), segs[g][1])
    # without a row map / factor: the rows themselves
    qi, si = M.moe_colwise_quant_rows(x[:rows] if rows <= T else x, off_d[:1 + 3], M.moe_wgrad_tiles(off_d[:4]),
                                      M.wgrad_max_tiles(int(offsets[3]), 3), pow2=pow2)
    seg0 = B.colwise_segments(host(x)[:int(offsets[3])], offsets[:4], True, pow2)
    assert_equal("identity rows", host(M.colwise_block(qi, si, [0, seg0[0][0].shape[1] // 128], 0)[0]), seg0[0][0])


@pytest.mark.parametrize("dg,pow2", [(False, False), (True, False), (True, True)])
def test_colwise_quant_swiglu(dg, pow2):
    G, F = 5, 256
    offsets = _segments(G, 5)
    rows = int(offsets[-1])
    g = synth.randn((rows, 2 * F), 23, synth.STAGE, 0, 0, 73, device=DEV, std=2.0)
    dh = synth.randn((rows, F), 23, synth.STAGE, 0, 0, 74, device=DEV, std=0.5) if dg else None
    off_d = torch.from_numpy(offsets).to(DEV)
    tf = M.moe_wgrad_tiles(off_d)
    mt = M.wgrad_max_tiles(rows, G)
    qt, st = M.moe_colwise_quant_swiglu(g, off_d, tf, mt, dh=dh, pow2=pow2)
    gh = host(g)
    vals = B.swiglu_backward(host(dh), gh, F) if dg else O.swiglu(gh, F)
    segs = B.colwise_segments(vals, offsets, True, pow2)
    tfh = host(tf)
    tab = O.e4m3_table()
    for gi in range(G):
        if tfh[gi + 1] == tfh[gi]:
            continue                          # the empty group: no tiles
        gq, gs = (host(t) for t in M.colwise_block(qt, st, tfh, gi))
        rq, rs = segs[gi]
        assert np.max(np.abs(gs - rs) / rs) < 1e-5
        diff = gq != rq
        assert diff.mean() < 1e-3
        if diff.any():
            assert np.all(np.abs(tab[gq[diff]] - tab[rq[diff]]) <= np.maximum(np.abs(tab[rq[diff]]) / 8, 2.0 ** -9))


@pytest.mark.parametrize("pow2", [False, True])
def test_wgrad_gemm(pow2):
    G, M_, N_ = 6, 256, 384
    offsets = _segments(G, 7)
    rows = int(offsets[-1])
    off_d = torch.from_numpy(offsets).to(DEV)
    tf = M.moe_wgrad_tiles(off_d)
    mt = M.wgrad_max_tiles(rows, G)
    a32 = synth.randn((rows, M_), 25, synth.STAGE, 0, 0, 75, device=DEV)
    b32 = synth.randn((rows, N_), 25, synth.STAGE, 0, 0, 76, device=DEV)
    aq, as_ = M.moe_colwise_quant_rows(a32, off_d, tf, mt, pow2=pow2)
    bq, bs = M.moe_colwise_quant_rows(b32, off_d, tf, mt, pow2=pow2)
    c = M.moe_grouped_gemm_wgrad(aq, as_, bq, bs, tf, mt, pow2=pow2)
    tfh = host(tf)
    ref = np.zeros((G, M_, N_))
    for g in range(G):
        if tfh[g + 1] > tfh[g]:
            A = O.dequant_act(*(host(t) for t in M.colwise_block(aq, as_, tfh, g)))
            Bm = O.dequant_act(*(host(t) for t in M.colwise_block(bq, bs, tfh, g)))
            ref[g] = A @ Bm.T
    assert np.all(host(c)[1] == 0)            # the empty group
    # fp32 accumulation over up to 3 steps of 128 products: error <= ~K u sum|a b|, and with random
    # signs sum|a b| / max|C| is ~sqrt(K), so ~1e-4 of max|C| at K = 384 (1.9e-5 observed)
    assert rel_err(host(c), ref) < 1e-4


# weight gradients sum an expert's rows, so a one-step FP8 code difference (where the two sides'
# fp32 and fp64 values straddle a rounding boundary) moves them by ~1/(16 sqrt(rows)) of their
# largest entry: these layers give every expert a few hundred rows
WG_CASES = {
    "tiny": replace(synth.CONFIGS["tiny"], name="tiny_wg", T=512),
    "prefill_wg": replace(synth.CONFIGS["prefill"], name="prefill_wg", T=512, H=256, E=16, F=256, k=8),
}


@pytest.mark.parametrize("name,pow2", [("tiny", False), ("prefill_wg", False), ("prefill_wg", True)])
def test_layer_weight_gradients(name, pow2):
    cfg = WG_CASES[name]
    gw, bw, ol = _layer_pair(cfg, pow2)
    lay = MoELayer(gw, cfg.T, _act(cfg))
    x = synth.make_x(cfg, DEV)
    dout = synth.make_dout(cfg, DEV)
    lay.forward(x, training=True)
    g = lay.backward(x, dout, bw, weight_grads=True)
    torch.cuda.synchronize()
    r = L.forward_dispatch(ol, host(x))
    rb = B.backward_dispatch(ol, r, host(x), host(dout))
    for key in ("dW1", "dW2"):
        e = rel_err(host(g[key]), rb[key])
        print(f"{name} pow2={pow2} {key} err {e:.2e}")
        assert e < TOL, key


@pytest.mark.parametrize("name", ["decode", "prefill"])
def test_layer_weight_gradients_full_size_sampled(name):
    """Full-size layers: the busiest routed expert of the oracle's own routing, and the shared
    expert (all tokens) where there is one."""
    cfg = synth.CONFIGS[name]
    gw, bw, ol = _layer_pair(cfg)
    lay = MoELayer(gw, cfg.T, _act(cfg))
    x = synth.make_x(cfg, DEV)
    dout = synth.make_dout(cfg, DEV)
    lay.forward(x, training=True)
    g = lay.backward(x, dout, bw, weight_grads=True)
    torch.cuda.synchronize()
    xh, dh = host(x), host(dout)
    idx, _ = O.moe_route(O.moe_gate_logits(xh, ol.wg, ol.bias), ol.cfg)
    busiest = int(np.argmax(np.bincount(idx[idx >= 0].ravel(), minlength=cfg.E)))
    experts = (busiest, cfg.E) if cfg.shared else (busiest,)
    for e in experts:
        dW1, dW2 = B.wgrad_expert(ol, xh, dh, e)
        e1, e2 = rel_err(host(g["dW1"][e]), dW1), rel_err(host(g["dW2"][e]), dW2)
        print(f"{name} expert {e} dW1 err {e1:.2e} dW2 err {e2:.2e}")
        assert e1 < TOL and e2 < TOL
    del lay, gw, bw, g
    _free()
