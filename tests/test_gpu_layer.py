"""End-to-end parity of the MoE layer forward (HIP path) against the oracle.

The tiny layer is compared on every token and every intermediate; the larger layers run at full
size on the GPU and are compared on sampled tokens, which the oracle evaluates without any
dispatch (per-token independence of MoE outputs).  Routing (logits, indices, weights), activation
and weight FP8 codes and scales are compared bit for bit; layer outputs within 2e-2.
"""
import numpy as np
import pytest
import torch

import block_scaled_fp8_top_amd as M
import oracle as O
import oracle.layer as L
import synth
from block_scaled_fp8_top_amd.layer import MoELayer
from gpu_helpers import DEV, TOL, assert_equal, cfgs_for, gpu_weights, host, oracle_layer, rel_err, rows_host

pytestmark = pytest.mark.gpu


def _act(cfg):
    return torch.bfloat16 if cfg.act == "bf16" else torch.float32


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_layer_tiny_every_intermediate():
    cfg = synth.CONFIGS["tiny"]
    gw = gpu_weights(cfg)
    lay = MoELayer(gw, cfg.T, _act(cfg))
    x = synth.make_x(cfg, DEV)
    out = lay.forward(x)
    ol = oracle_layer(cfg)
    r = L.forward_dispatch(ol, host(x))
    for g in range(cfg.groups):
        ew = ol.get(g)
        assert_equal(f"w1q[{g}]", host(gw.w1q[g]), ew.w1q)
        assert_equal(f"w1s[{g}]", host(gw.w1s[g]), ew.w1s)
        assert_equal(f"w2q[{g}]", host(gw.w2q[g]), ew.w2q)
        assert_equal(f"w2s[{g}]", host(gw.w2s[g]), ew.w2s)
    assert_equal("logits", host(lay.logits), r["z"])
    assert_equal("idx", host(lay.idx), r["idx"])
    assert_equal("w", host(lay.wts), r["w"])
    assert_equal("xq", host(lay.xq), r["xq"])
    assert_equal("xs", host(lay.xs), r["xs"])
    assert_equal("counts", host(lay.disp.counts), r["counts"])
    assert_equal("offsets", host(lay.disp.offsets), r["offsets"])
    assert_equal("dest", host(lay.disp.dest_row), r["dest"])
    n = int(r["offsets"][-1])
    assert_equal("src", host(lay.disp.src_token)[:n], r["src"])
    # the rows GEMM1 reads: xq gathered through src_token (the layer keeps no permuted copy)
    assert_equal("gathered rows", host(lay.xq)[host(lay.disp.src_token)[:n]], r["aq"])
    assert_equal("as", host(lay.disp.as_)[:n], r["as_"])
    assert rel_err(host(lay.y)[:n], r["y_act"]) < TOL
    err = rel_err(host(out), r["out"])
    print(f"tiny layer output err {err:.3e}")
    assert err < TOL
    # per-token dense evaluation (all experts, zero-masked gate) agrees with the dispatch path
    dense = L.forward_token(ol, host(x)[:6], dense=True)
    assert rel_err(host(out)[:6], dense["out"]) < TOL


SAMPLES = {"decode": 48, "prefill": 4, "longctx": 4, "r3": 3}


@pytest.mark.parametrize("name,chunk", [("decode", 0), ("prefill", 0), ("longctx", 0), ("longctx", 15), ("r3", 0)])
def test_layer_full_size_sampled(name, chunk):
    cfg = synth.CONFIGS[name]
    gw = gpu_weights(cfg)
    lay = MoELayer(gw, cfg.T, _act(cfg))
    x = synth.make_x(cfg, DEV, chunk=chunk)
    out = lay.forward(x)
    torch.cuda.synchronize()
    toks = synth.sample_tokens(cfg.T, SAMPLES[name], cfg.seed + chunk)
    ol = oracle_layer(cfg)
    xr = rows_host(x, toks)
    r = L.forward_sampled(ol, xr)
    assert_equal("logits", rows_host(lay.logits, toks), r["z"])
    assert_equal("idx", rows_host(lay.idx, toks), r["idx"])
    assert_equal("w", rows_host(lay.wts, toks), r["w"])
    assert_equal("xq", rows_host(lay.xq, toks), r["xq"])
    assert_equal("xs", rows_host(lay.xs, toks), r["xs"])
    for e in r["experts"][:3]:
        ew = ol.get(e)
        assert_equal(f"w1q[{e}]", host(gw.w1q[e]), ew.w1q)
        assert_equal(f"w2s[{e}]", host(gw.w2s[e]), ew.w2s)
    err = rel_err(rows_host(out, toks), r["out"])
    counts = host(lay.disp.counts)
    print(f"{name} chunk {chunk}: output err {err:.3e}; group rows min {counts.min()} max {counts.max()} "
          f"empty {(counts == 0).sum()}")
    assert err < TOL
    assert int(host(lay.disp.offsets)[-1]) == cfg.rows
    del lay, gw, x, out
    _free()


def test_layer_deterministic_and_chunk_concatenation():
    """Two runs give identical bits; a 2-chunk call equals two 1-chunk calls (no split-K,
    every kernel is row-local), on the decode layer."""
    cfg = synth.CONFIGS["decode"]
    gw = gpu_weights(cfg)
    x = torch.cat([synth.make_x(cfg, DEV, chunk=0), synth.make_x(cfg, DEV, chunk=1)])
    l1 = MoELayer(gw, cfg.T, _act(cfg))
    a0 = l1.forward(x[:cfg.T]).clone()
    a1 = l1.forward(x[cfg.T:]).clone()
    a0b = l1.forward(x[:cfg.T]).clone()
    l2 = MoELayer(gw, 2 * cfg.T, _act(cfg))
    both = l2.forward(x)
    assert torch.equal(a0.view(torch.int16), a0b.view(torch.int16))
    assert torch.equal(torch.cat([a0, a1]).view(torch.int16), both.view(torch.int16))


def test_layer_longctx_chunk_concatenation():
    """The long-context layer: one 16384-token call is bitwise two 8192-token calls (every kernel
    is row-local and the expert GEMMs' accumulation order does not depend on the group sizes)."""
    cfg = synth.CONFIGS["longctx"]
    gw = gpu_weights(cfg)
    x = torch.cat([synth.make_x(cfg, DEV, chunk=0), synth.make_x(cfg, DEV, chunk=1)])
    l1 = MoELayer(gw, cfg.T, _act(cfg))
    a0 = l1.forward(x[:cfg.T]).clone()
    a1 = l1.forward(x[cfg.T:]).clone()
    del l1
    l2 = MoELayer(gw, 2 * cfg.T, _act(cfg))
    both = l2.forward(x)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([a0, a1]).view(torch.int16), both.view(torch.int16))
    del l2, gw, x, both
    _free()


@pytest.mark.parametrize("name,chunks", [("decode", 5), ("longctx", 3)])
def test_forward_chunks_equals_forward(name, chunks):
    """forward_chunks (each chunk's gate projection after the first on a second stream, beside the
    previous chunk's combine) gives every chunk the bits of forward(chunk): eagerly, and in a HIP
    graph captured from it, on every replay with eager work and synchronisations in between."""
    cfg = synth.CONFIGS[name]
    gw = gpu_weights(cfg)
    lay = MoELayer(gw, cfg.T, _act(cfg))
    xs = [synth.make_x(cfg, DEV, chunk=c) for c in range(chunks)]
    ref = [lay.forward(x).clone() for x in xs]
    outs = [torch.full_like(r, 3.0) for r in ref]
    lay.forward_chunks(xs, outs)
    torch.cuda.synchronize()
    bits = lambda t: t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)
    for c in range(chunks):
        assert torch.equal(bits(outs[c]), bits(ref[c])), f"eager chunk {c}"
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            lay.forward_chunks(xs, outs)
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(3):
        for o in outs:
            o.fill_(5.0)
        g.replay()
        torch.cuda.synchronize()
        for c in range(chunks):
            assert torch.equal(bits(outs[c]), bits(ref[c])), f"replay {rep} chunk {c}"
        lay.forward(xs[0])   # eager work on the same layer between replays
        torch.cuda.synchronize()
    del g, lay, gw, xs, ref, outs
    _free()


def _edge_payload(cfg, seed):
    """A routing payload [k, T] for router replay: slot 0 is expert 0 for every token but 7, 8
    and 9 (so group 0 has T - 3 rows and a ragged last tile), token 5 alone takes expert 1 (a
    1-row group), nobody takes expert 2 (an empty group); the other slots are distinct random
    experts from 3..E-1.  Returns (payload int32 [k, T], the 32 sampled tokens), the sampled
    tokens' other slots drawn from experts 3..14 so that the oracle evaluates few experts."""
    T, E, k = cfg.T, cfg.E, cfg.k
    rng = np.random.default_rng(seed)
    idx = np.empty((T, k), np.int32)
    idx[:, 0] = 0
    keys = rng.random((T, E - 3))
    idx[:, 1:] = np.argsort(keys, axis=1)[:, :k - 1] + 3
    fixed = [0, 1, 2, 3, 5, 7, 8, 9, T // 2, T // 2 + 1, T - 300, T - 3, T - 2, T - 1]
    others = rng.choice(np.setdiff1d(np.arange(T), fixed), 32 - len(fixed), replace=False)
    toks = np.array(sorted(set(fixed) | set(int(t) for t in others)))
    pool = np.arange(3, 15)
    for t in toks:
        idx[t, 1:] = rng.choice(pool, k - 1, replace=False)
    idx[5, 1] = 1
    for t in (7, 8, 9):
        idx[t, 0] = [e for e in pool if e not in idx[t, 1:]][0]
    return np.ascontiguousarray(idx.T), toks


@pytest.mark.parametrize("name", ["prefill", "longctx"])
def test_layer_replayed_edge_groups_32_tokens(name):
    """The full-size layer on a crafted replay payload (largest possible group with a ragged last
    tile, a 1-row group, an empty group): 32 sampled tokens, among them the 1-row group's token and
    rows in the first, a middle and the ragged last tile of the largest group, match the oracle:
    indices, weights and activation codes bit for bit, outputs within the tolerance."""
    cfg = synth.CONFIGS[name]
    T, k = cfg.T, cfg.k
    pay, toks = _edge_payload(cfg, cfg.seed + 99)
    gw = gpu_weights(cfg)
    lay = MoELayer(gw, T, _act(cfg))
    x = synth.make_x(cfg, DEV, chunk=7)
    out = lay.forward(x, replay=torch.from_numpy(pay).to(DEV))
    torch.cuda.synchronize()
    assert int(lay.bad.item()) == 0
    counts = host(lay.disp.counts)
    assert counts[0] == T - 3 and counts[1] == 1 and counts[2] == 0
    tile = lay.plan.tile_rows
    assert (T - 3) % tile != 0
    dest = host(lay.disp.dest_row).reshape(T, k)
    off0 = int(host(lay.disp.offsets)[0])
    last_tile0 = ((T - 3) // tile) * tile
    assert sum(1 for t in toks if t not in (7, 8, 9) and dest[t, 0] - off0 >= last_tile0) >= 3
    ol = oracle_layer(cfg)
    r = L.forward_sampled(ol, rows_host(x, toks), replay_rows=np.ascontiguousarray(pay[:, toks]), workers=8)
    assert_equal("idx", rows_host(lay.idx, toks), r["idx"])
    assert_equal("w", rows_host(lay.wts, toks), r["w"])
    assert_equal("xq", rows_host(lay.xq, toks), r["xq"])
    assert_equal("xs", rows_host(lay.xs, toks), r["xs"])
    err = rel_err(rows_host(out, toks), r["out"])
    print(f"{name}: 32 tokens over edge groups (tile {tile}): output err {err:.3e}")
    assert err < TOL
    del lay, gw, x, out
    _free()


@pytest.mark.parametrize("name", ["prefill", "longctx"])
def test_layer_tile_heights_bitwise(name):
    """The expert GEMMs at 128- and 256-row tiles: the accumulation order of every output does not
    depend on the tile height, so the layer forward (h codes, expert rows, output) is bitwise the
    same, including groups whose last tile has a wave row of padding only."""
    cfg = synth.CONFIGS[name]
    gw = gpu_weights(cfg)
    x = synth.make_x(cfg, DEV, chunk=3)
    res = {}
    for tile in (128, 256):
        lay = MoELayer(gw, cfg.T, _act(cfg), tile_rows=tile)
        out = lay.forward(x).clone()
        assert lay.plan.tile_rows == tile
        res[tile] = (out, lay.hq.clone(), lay.hs.clone(), lay.y.clone())
        del lay
    torch.cuda.synchronize()
    n = cfg.rows
    (o1, h1, s1, y1), (o2, h2, s2, y2) = res[128], res[256]
    assert torch.equal(h1[:n], h2[:n]) and torch.equal(s1[:n].view(torch.int32), s2[:n].view(torch.int32))
    assert torch.equal(y1[:n].view(torch.int16), y2[:n].view(torch.int16))
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    del res, gw
    _free()


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill"])
def test_layer_gathered_rows_equal_permuted_copy(name):
    """GEMM1 reading its rows from xq through src_token gives bitwise the forward (and, for the
    small layers, the training backward's dx) of GEMM1 reading the dispatch's permuted copy."""
    cfg = synth.CONFIGS[name]
    gw = gpu_weights(cfg)
    outs = {}
    for gather in (True, False):
        lay = MoELayer(gw, cfg.T, _act(cfg), gather_rows=gather)
        assert (lay.disp.aq is None) == gather
        x = synth.make_x(cfg, DEV)
        o = lay.forward(x).clone()
        hq = lay.hq.clone()
        dx = None
        if name != "prefill":
            from block_scaled_fp8_top_amd.layer import prepare_backward_weights
            dx = lay.backward(x, synth.make_dout(cfg, DEV), prepare_backward_weights(gw))["dx"].clone()
        outs[gather] = (o, hq, dx)
        del lay
    torch.cuda.synchronize()
    (o1, h1, d1), (o0, h0, d0) = outs[True], outs[False]
    assert torch.equal(h1, h0)
    iv = torch.int16 if o1.dtype == torch.bfloat16 else torch.int32
    assert torch.equal(o1.view(iv), o0.view(iv))
    if d1 is not None:
        assert torch.equal(d1.view(iv), d0.view(iv))
    del outs, gw
    _free()


@pytest.mark.parametrize("name", ["tiny", "decode"])
def test_layer_graph_replay_matches_eager(name):
    """The whole forward captured in one HIP graph: every replay, with unrelated eager work and
    synchronisations in between, reproduces the eager outputs bit for bit (no memset nodes, no
    host synchronisation, all buffers preallocated)."""
    cfg = synth.CONFIGS[name]
    gw = gpu_weights(cfg)
    lay = MoELayer(gw, cfg.T, _act(cfg))
    other = MoELayer(gw, cfg.T, _act(cfg))
    x = synth.make_x(cfg, DEV)
    x2 = synth.make_x(cfg, DEV, chunk=1)
    ref = lay.forward(x).clone()
    ref_idx, ref_w = lay.idx.clone(), lay.wts.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            lay.forward(x)
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(4):
        lay.out.zero_()
        lay.idx.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(lay.out.view(torch.int16 if lay.out.dtype == torch.bfloat16 else torch.int32),
                           ref.view(torch.int16 if ref.dtype == torch.bfloat16 else torch.int32)), f"replay {rep}"
        assert torch.equal(lay.idx, ref_idx) and torch.equal(lay.wts.view(torch.int32), ref_w.view(torch.int32))
        other.forward(x2)   # eager work on other buffers between replays
        torch.cuda.synchronize()
    del g, lay, other, gw
    _free()


R3_TOKENS = 16


@pytest.fixture(scope="module")
def r3_stack():
    """The prefill layer 4 deep at 32768 tokens: pass A routes with W and records the
    [num_layers, top_k, seq_len] payload; pass B replays it on W' = W + N(0, 1e-3); pass C
    recomputes the routing on W'.  Whole-batch facts are checked here; for 16 sampled tokens every
    layer's input rows, indices, weights and output rows are kept for the oracle."""
    cfg = synth.CONFIGS["r3"]
    T, k, Lyr = cfg.T, cfg.k, cfg.layers
    act = _act(cfg)
    toks = synth.sample_tokens(T, R3_TOKENS, cfg.seed)
    payload = torch.full((Lyr, k, T), -1, dtype=torch.int32, device=DEV)
    x0 = synth.make_x(cfg, DEV)
    keep, rows = {}, {}
    stats = []
    for pas in ("A", "B", "C"):
        x = x0
        for l in range(Lyr):
            gw = gpu_weights(cfg, l, perturbed=pas != "A")
            lay = MoELayer(gw, T, act)
            if pas == "A":
                out = lay.forward(x, record=payload[l])
            elif pas == "B":
                out = lay.forward(x, replay=payload[l])
            else:
                out = lay.forward(x)
            idx = lay.idx.clone()
            if pas == "A":
                keep[("A", l)] = (idx, lay.disp.counts.clone(), lay.disp.offsets.clone(), lay.disp.dest_row.clone(),
                                  lay.disp.src_token.clone())
            if pas == "B":
                assert torch.equal(idx, payload[l].t().contiguous()), f"layer {l}: replayed idx != payload"
                a = keep[("A", l)]
                assert torch.equal(lay.disp.counts, a[1]) and torch.equal(lay.disp.offsets, a[2])
                assert torch.equal(lay.disp.dest_row, a[3]) and torch.equal(lay.disp.src_token, a[4])
                assert int(lay.bad.item()) == 0
            if pas == "C":
                ia = keep[("A", l)][0]
                slot = (idx != ia).float().mean().item()
                setd = 1.0 - (idx[:, :, None] == ia[:, None, :]).any(-1).float().mean().item()
                stats.append((slot, setd))
            if pas in ("A", "B"):
                rows[(pas, l)] = dict(x=rows_host(x, toks), idx=rows_host(idx, toks), w=rows_host(lay.wts, toks),
                                      out=rows_host(out, toks),
                                      replay=np.ascontiguousarray(host(payload[l])[:, toks]))
            x = (x.float() + out.float()).to(act)
            del lay, gw
            _free()
        keep[(pas, "final")] = x
    res = dict(cfg=cfg, toks=toks, rows=rows, stats=stats,
               dB=rel_err(host(keep[("B", "final")]), host(keep[("A", "final")])),
               dC=rel_err(host(keep[("C", "final")]), host(keep[("A", "final")])))
    del keep, payload, x0
    _free()
    return res


def test_r3_stack_record_replay(r3_stack):
    """Replay reproduces the recorded routing and dispatch at every layer (checked while the
    stack runs); recomputing the routing on W' moves slots, which is what replay prevents."""
    stats = r3_stack["stats"]
    print("pass C vs pass A per layer (slot drift, expert-set drift):",
          [f"({a:.4f}, {b:.4f})" for a, b in stats])
    assert len(stats) == r3_stack["cfg"].layers
    assert all(0.0 < b <= a < 1.0 for a, b in stats)
    print(f"stack output rel diff: B vs A {r3_stack['dB']:.3e}, C vs A {r3_stack['dC']:.3e}")
    assert r3_stack["dB"] < r3_stack["dC"]


@pytest.mark.parametrize("layer", [0, 1, 2, 3])
def test_r3_stack_layer_parity(r3_stack, layer):
    """Every layer of the stack on 16 sampled tokens, from the stack's own inputs at that layer:
    pass A (route with W, record) and pass B (replay the record on W') against the oracle -
    indices and weights bit for bit, outputs within the tolerance."""
    cfg = r3_stack["cfg"]
    a, b = r3_stack["rows"][("A", layer)], r3_stack["rows"][("B", layer)]
    olA = oracle_layer(cfg, layer)
    rA = L.forward_sampled(olA, a["x"], workers=8)
    assert_equal(f"layer {layer} pass A idx", a["idx"], rA["idx"])
    assert_equal(f"layer {layer} pass A w", a["w"], rA["w"])
    assert_equal(f"layer {layer} record", a["replay"], np.ascontiguousarray(rA["idx"].T))
    errA = rel_err(a["out"], rA["out"])
    del olA
    olB = oracle_layer(cfg, layer, perturbed=True)
    rB = L.forward_sampled(olB, b["x"], replay_rows=a["replay"], workers=8)
    assert_equal(f"layer {layer} pass B idx", b["idx"], rB["idx"])
    assert_equal(f"layer {layer} pass B w", b["w"], rB["w"])
    errB = rel_err(b["out"], rB["out"])
    print(f"layer {layer}: {len(r3_stack['toks'])} tokens, output err pass A {errA:.3e} pass B {errB:.3e}")
    assert errA < TOL and errB < TOL


@pytest.mark.parametrize("layer", [1, 2, 3])
def test_r3_deeper_layers_route_and_replay_parity(layer):
    """Layers 1..3 of the stack on identical inputs: gate logits, routing, replay on W'."""
    cfg = synth.CONFIGS["r3"]
    gcfg, ocfg = cfgs_for(cfg)
    x = synth.make_x(cfg, DEV, chunk=layer)
    wg, b = synth.make_gate(cfg, layer, DEV)
    wg2, _ = synth.make_gate(cfg, layer, DEV, perturbed=True)
    z = M.moe_gate_logits(x, wg, b)
    payload = torch.empty((cfg.k, cfg.T), dtype=torch.int32, device=DEV)
    idx, w = M.moe_route(z, gcfg, record=payload)
    z2 = M.moe_gate_logits(x, wg2, b)
    ridx, rw = M.moe_replay_route(z2, gcfg, payload)
    toks = synth.sample_tokens(cfg.T, 64, cfg.seed + layer)
    xr = rows_host(x, toks)
    oz = O.moe_gate_logits(xr, host(wg), None)
    oidx, ow = O.moe_route(oz, ocfg)
    oz2 = O.moe_gate_logits(xr, host(wg2), None)
    oridx, orw, _ = O.moe_replay_route(oz2, ocfg, np.ascontiguousarray(oidx.T))
    assert_equal("logits", rows_host(z, toks), oz)
    assert_equal("idx", rows_host(idx, toks), oidx)
    assert_equal("w", rows_host(w, toks), ow)
    assert_equal("replay idx", rows_host(ridx, toks), oridx)
    assert_equal("replay w", rows_host(rw, toks), orw)
