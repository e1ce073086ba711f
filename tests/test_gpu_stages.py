"""Per-stage parity of the HIP path against the CPU oracle, at every workload's full size.

Each stage gets the same seeded synthetic inputs on both sides.  Integer, byte and index outputs
(logits of the router's fixed chain, routing indices and weights, FP8 codes and scales, counts,
offsets, permutation) must match bit for bit; GEMM and combine outputs within a max-abs-normalised
error of 2e-2.  Large outputs are compared on sampled rows that the oracle computes one by one.
"""
import itertools

import numpy as np
import pytest
import torch

import block_scaled_fp8_top_amd as M
import oracle as O
import synth
from gpu_helpers import DEV, TOL, assert_equal, cfgs_for, host, rel_err, rows_host

pytestmark = pytest.mark.gpu
NAMES = ["tiny", "decode", "prefill", "longctx", "r3"]
TILES = [32, 48, 64, 128, 256]   # every row-tile height of the grouped GEMM, whichever the shape would pick


def _weights_for(b, epi, tile):
    """256-row tiles stream packed weights only; other heights take the row-major codes."""
    return M.moe_pack_weights_fp8(b, epi) if tile == 256 else b


def _cleanup():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


# ----------------------------------------------------------------------------- quantisation
@pytest.mark.parametrize("name", NAMES)
def test_quant_activations_1x128(name):
    cfg = synth.CONFIGS[name]
    x = synth.make_x(cfg, DEV)
    q, s = M.moe_quant_fp8_block(x, 1)
    rq, rs = O.moe_quant_fp8_block(host(x), 1)
    assert_equal("codes", host(q), rq)
    assert_equal("scales", host(s), rs)
    del x, q, s
    _cleanup()


@pytest.mark.parametrize("name", NAMES)
def test_quant_weights_128x128(name):
    cfg = synth.CONFIGS[name]
    experts = sorted({0, cfg.E - 1} | ({cfg.E} if cfg.shared else set()))
    for e in experts:
        w1, w2 = synth.make_expert(cfg, e, 0, DEV)
        for w in (w1, w2):
            q, s = M.moe_quant_fp8_block(w, 128)
            rq, rs = O.moe_quant_fp8_block(host(w), 128)
            assert_equal(f"W codes e={e}", host(q), rq)
            assert_equal(f"W scales e={e}", host(s), rs)
    # batched [2, N, K] call, bf16 input
    wb = torch.stack([synth.make_expert(cfg, e, 0, DEV)[1] for e in experts[:2]]).to(torch.bfloat16)
    q, s = M.moe_quant_fp8_block(wb, 128)
    rq, rs = O.moe_quant_fp8_block(host(wb), 128)
    assert_equal("batched codes", host(q), rq)
    assert_equal("batched scales", host(s), rs)
    _cleanup()


def test_quant_edge_values():
    """Zero blocks, signed zeros, a block whose amax is tiny, and values at code boundaries."""
    x = torch.zeros((4, 384), dtype=torch.float32)
    x[0, 128:256] = -0.0
    x[1, :128] = torch.linspace(-448, 448, 128)
    x[1, 128:256] = 1e-30
    x[2, :] = torch.tensor([1.0625, 1.1875, -3.0, 0.1] * 96)
    x[3, 256:] = synth.randn((128,), 5, synth.STAGE, part=30) * 1e4
    q, s = M.moe_quant_fp8_block(x.to(DEV), 1)
    rq, rs = O.moe_quant_fp8_block(x.numpy(), 1)
    assert_equal("codes", host(q), rq)
    assert_equal("scales", host(s), rs)


def _quotient_edge_blocks(nblocks, seed, bf16_exact):
    """Blocks of 128 whose amax A has an exponent anywhere from -133 to 127 (subnormal, tiny,
    normal and huge scales, both sides of the 2^-60 scale below which the encoders divide in
    full), filled with values spread over every bit pattern of magnitude <= A: subnormal and
    signed-zero x included."""
    rng = np.random.default_rng(seed)
    out = np.empty((nblocks, 128), np.float32)
    for b in range(nblocks):
        ex = int(rng.integers(-133, 128))
        a = np.float32(np.ldexp(1.0 + rng.random(), ex)) if ex < 127 else np.float32(np.ldexp(1.0 + 0.99 * rng.random(), ex))
        if bf16_exact:
            a = (np.array([a], np.float32).view(np.uint32) & 0xFFFF0000).view(np.float32)[0]
        if a == 0:
            a = np.float32(np.ldexp(1.0, -133))
        top = int(np.array([a], np.float32).view(np.uint32)[0])
        bits = rng.integers(0, top + 1, size=127, dtype=np.int64).astype(np.uint32)
        if bf16_exact:
            bits &= np.uint32(0xFFFF0000)
        bits |= rng.integers(0, 2, size=127).astype(np.uint32) << np.uint32(31)   # random signs
        out[b, 0] = a if b % 2 else -a
        out[b, 1:] = bits.view(np.float32)
        rng.shuffle(out[b])
    return out


@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("pow2", [False, True])
def test_quant_quotients_over_every_exponent(act, pow2):
    """The encoders' x / s (one correctly rounded reciprocal and one FMA correction per value, or a
    full division for scales below 2^-60): codes and scales bit for bit the oracle's (IEEE
    division) for block scales across the whole fp32 exponent range, 1x128 and 128x128 blocks."""
    x = _quotient_edge_blocks(4096, 41 + pow2, act == "bf16").reshape(512, 1024)
    xt = torch.from_numpy(x).to(DEV)
    if act == "bf16":
        xt = xt.to(torch.bfloat16)
    for br in (1, 128):
        q, s = M.moe_quant_fp8_block(xt, br, pow2=pow2)
        rq, rs = O.moe_quant_fp8_block(host(xt), br, pow2=pow2)
        assert_equal(f"codes {br}", host(q), rq)
        assert_equal(f"scales {br}", host(s), rs)


# ----------------------------------------------------------------------------- gate logits
@pytest.mark.parametrize("name", NAMES)
def test_gate_logits(name):
    cfg = synth.CONFIGS[name]
    x = synth.make_x(cfg, DEV)
    wg, b = synth.make_gate(cfg, 0, DEV)
    z = M.moe_gate_logits(x, wg, b)
    rows = np.arange(cfg.T) if cfg.T <= 256 else synth.sample_tokens(cfg.T, 96, cfg.seed)
    rz = O.moe_gate_logits(host(x)[rows], host(wg), None if b is None else host(b))
    assert_equal("logits", host(z)[rows], rz)
    del x, z
    _cleanup()


@pytest.mark.parametrize("T,H,E", [(77, 136, 13),       # direct (one output per thread)
                                    (700, 264, 256),     # LDS-staged 1x1 tiles
                                    (5000, 136, 200),    # 2x2 tiles, ragged
                                    (9000, 520, 130),    # 2x2 tiles, ragged, 17 chunks
                                    (8200, 136, 200),    # 4x4 tiles, ragged
                                    (16383, 136, 260),   # 8x4 tiles, ragged T, E and last chunk
                                    (8200, 160, 64),     # x broadcast: 1 expert per lane, 5 chunks
                                    (8193, 96, 128),     # x broadcast: 2 per lane, 1 token in the last workgroup
                                    (12007, 224, 256),   # x broadcast: 2 per lane, two 128-expert slices, 7 chunks
                                    (8192, 32, 256),     # x broadcast: one chunk
                                    (8250, 64, 512)])    # 512 experts: 8x4 tiles
def test_gate_logits_ragged_all_paths(T, H, E):
    """T and E not multiples of the register tiles, H not a multiple of the LDS chunk; fp32 and bf16.
    From 8192 tokens with E of 64, 128 or 256 and H a multiple of 32 (below the 8x4 tiles' size),
    the x-broadcast kernel runs: ragged last workgroups, slices of 64 or 128 experts (1 or 2 per
    lane, one or two slices), one to seven chunks."""
    x = synth.randn((T, H), 6, synth.STAGE, part=31, device=DEV)
    wg = synth.randn((E, H), 6, synth.STAGE, part=32, device=DEV, std=0.1)
    b = synth.randn((E,), 6, synth.STAGE, part=33, device=DEV)
    for xx in (x, x.to(torch.bfloat16)):
        z = M.moe_gate_logits(xx, wg, b)
        assert_equal("logits", host(z), O.moe_gate_logits(host(xx), host(wg), host(b)))
    z0 = M.moe_gate_logits(x[:0], wg)
    assert z0.shape == (0, E)


# ----------------------------------------------------------------------------- router / replay
@pytest.mark.parametrize("name", NAMES)
def test_route_and_record(name):
    cfg = synth.CONFIGS[name]
    gcfg, ocfg = cfgs_for(cfg)
    T, k = cfg.T, cfg.k
    z = synth.make_logits(cfg, device=DEV)
    payload = torch.full((2, k, T + 3), -5, dtype=torch.int32, device=DEV)
    idx, w = M.moe_route(z, gcfg, record=payload[1])
    opay = np.full((k, T + 3), -5, np.int32)
    oidx, ow = O.moe_route(host(z), ocfg, record=opay)
    assert_equal("idx", host(idx), oidx)
    assert_equal("weights", host(w), ow)
    assert_equal("record", host(payload[1]), opay)
    assert np.all(host(payload[0]) == -5)


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill"])
@pytest.mark.parametrize("pow2", [False, True])
def test_route_quant_equals_separate_calls(name, pow2):
    """moe_route_quant: the router's indices, weights and recorded payload and the 1x128 codes and
    scales of x, bitwise those of moe_route and moe_quant_fp8_block called separately."""
    cfg = synth.CONFIGS[name]
    gcfg, _ = cfgs_for(cfg)
    T, k = min(cfg.T, 2048), cfg.k
    z = synth.make_logits(cfg, device=DEV)[:T].contiguous()
    x = synth.make_x(cfg, DEV)[:T].contiguous()
    p1 = torch.full((k, T), -3, dtype=torch.int32, device=DEV)
    p2 = p1.clone()
    i1, w1 = M.moe_route(z, gcfg, record=p1)
    q1, s1 = M.moe_quant_fp8_block(x, 1, pow2=pow2)
    i2, w2, q2, s2 = M.moe_route_quant(z, gcfg, x, record=p2, pow2=pow2)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2) and torch.equal(w1.view(torch.int32), w2.view(torch.int32))
    assert torch.equal(p1, p2)
    assert torch.equal(q1, q2) and torch.equal(s1.view(torch.int32), s2.view(torch.int32))


@pytest.mark.parametrize("T", [1, 5, 67])
@pytest.mark.parametrize("H", [128, 384])
@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("pow2", [False, True])
def test_route_quant_ragged_equals_separate_calls(T, H, act, pow2):
    """The fused launch's ragged ends (a last routing workgroup with fewer than 4 tokens, a last
    quantisation workgroup with fewer blocks than it holds) give bitwise the separate calls."""
    cfg = synth.CONFIGS["prefill"]
    gcfg, _ = cfgs_for(cfg)
    z = synth.make_logits(cfg, T=T, device=DEV, part=5)
    x = synth.to_act(synth.randn((T, H), 23, synth.STAGE, part=78, device=DEV), act)
    p1 = torch.full((cfg.k, T), -3, dtype=torch.int32, device=DEV)
    p2 = p1.clone()
    i1, w1 = M.moe_route(z, gcfg, record=p1)
    q1, s1 = M.moe_quant_fp8_block(x, 1, pow2=pow2)
    i2, w2, q2, s2 = M.moe_route_quant(z, gcfg, x, record=p2, pow2=pow2)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2) and torch.equal(w1.view(torch.int32), w2.view(torch.int32))
    assert torch.equal(p1, p2)
    assert torch.equal(q1, q2) and torch.equal(s1.view(torch.int32), s2.view(torch.int32))


@pytest.mark.parametrize("name", NAMES)
def test_replay(name):
    cfg = synth.CONFIGS[name]
    gcfg, ocfg = cfgs_for(cfg)
    T, k = cfg.T, cfg.k
    z = synth.make_logits(cfg, device=DEV)
    payload = torch.empty((k, T), dtype=torch.int32, device=DEV)
    idx, w = M.moe_route(z, gcfg, record=payload)
    opay = np.empty((k, T), np.int32)
    O.moe_route(host(z), ocfg, record=opay)
    assert_equal("record", host(payload), opay)
    bad = torch.zeros(1, dtype=torch.int32, device=DEV)
    # replay of the recorded routing on the same logits reproduces the router bit for bit
    ridx, rw = M.moe_replay_route(z, gcfg, payload, bad_count=bad)
    assert_equal("replay idx", host(ridx), host(idx))
    assert_equal("replay w", host(rw), host(w))
    # on different logits: indices kept, weights from the current logits
    z2 = synth.make_logits(cfg, device=DEV, part=1)
    ridx2, rw2 = M.moe_replay_route(z2, gcfg, payload, bad_count=bad)
    oidx2, ow2, obad = O.moe_replay_route(host(z2), ocfg, opay)
    assert_equal("replay2 idx", host(ridx2), oidx2)
    assert_equal("replay2 w", host(rw2), ow2)
    assert int(bad.item()) == 0 and obad == 0
    # planted bad entries (out of range, negative, repeated) in both copies
    bad_tokens = [1, T // 2, T - 1]
    opay[0, 1] = cfg.E
    opay[k - 1, T // 2] = -3
    opay[min(1, k - 1), T - 1] = opay[0, T - 1] if k > 1 else cfg.E + 7
    gpay = torch.from_numpy(opay).to(DEV)
    ridx3, rw3 = M.moe_replay_route(z2, gcfg, gpay, bad_count=bad)
    oidx3, ow3, obad3 = O.moe_replay_route(host(z2), ocfg, opay)
    assert obad3 == len(bad_tokens) and int(bad.item()) == obad3
    assert_equal("replay3 idx", host(ridx3), oidx3)
    assert_equal("replay3 w", host(rw3), ow3)


@pytest.mark.parametrize("name,renorm,act,k", [("prefill", 1, "bf16", None), ("r3", 1, "bf16", None),
                                               ("prefill", 0, "f32", None), ("tiny", 1, "f32", 6),
                                               ("prefill", 1, "bf16", 7)])
def test_replay_gate_fused(name, renorm, act, k):
    """Sigmoid replay fused with the gate projection == moe_gate_logits + moe_replay_route, bit for
    bit, with and without renormalisation, bf16 and fp32 x, a k that does not divide 64, bias, and
    planted bad entries; and against the oracle's logits + replay on sampled tokens."""
    cfg = synth.CONFIGS[name]
    E, H = cfg.E, cfg.H
    k = k or cfg.k
    T = min(cfg.T, 8192)
    gcfg = M.router_cfg(E, k, 1, renorm)
    ocfg = O.router_cfg(E, k, 1, renorm)
    x = synth.make_x(cfg, DEV)[:T]
    x = x.float() if act == "f32" else x.to(torch.bfloat16)
    wg, b = synth.make_gate(cfg, 0, DEV)
    bias = synth.randn((E,), cfg.seed, 90, 0, 0, device=DEV) * 0.5
    rng = np.random.default_rng(cfg.seed + k)
    pay = np.stack([rng.permutation(E)[:k] for _ in range(T)], 1).astype(np.int32)   # [k, T], distinct per token
    pay[0, 5] = E
    pay[k - 1, T // 3] = -1
    pay[1, T - 1] = pay[0, T - 1]
    gpay = torch.from_numpy(pay).to(DEV)
    for bb in (None, bias):
        bad1 = torch.zeros(1, dtype=torch.int32, device=DEV)
        bad2 = torch.zeros(1, dtype=torch.int32, device=DEV)
        z = M.moe_gate_logits(x, wg, bb)
        ridx, rw = M.moe_replay_route(z, gcfg, gpay, bad_count=bad1)
        fidx, fw = M.moe_replay_gate(x, wg, bb, gcfg, gpay, bad_count=bad2)
        assert_equal("fused idx", host(fidx), host(ridx))
        assert_equal("fused w", host(fw), host(rw))
        assert int(bad1.item()) == int(bad2.item()) == 3
        toks = synth.sample_tokens(T, 64, cfg.seed + 5)
        oz = O.moe_gate_logits(host(x)[toks], host(wg), None if bb is None else host(bb))
        oidx, ow, _ = O.moe_replay_route(oz, ocfg, np.ascontiguousarray(pay[:, toks]))
        assert_equal("fused idx vs oracle", rows_host(fidx, toks), oidx)
        assert_equal("fused w vs oracle", rows_host(fw, toks), ow)


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill"])
def test_route_ties(name):
    """Logits on a coarse grid: many exact ties, broken toward the lower expert index."""
    cfg = synth.CONFIGS[name]
    gcfg, ocfg = cfgs_for(cfg)
    z = synth.tie_logits(4096, cfg.E, 5, cfg.seed, device=DEV)
    idx, w = M.moe_route(z, gcfg)
    oidx, ow = O.moe_route(host(z), ocfg)
    assert_equal("idx", host(idx), oidx)
    assert_equal("w", host(w), ow)


@pytest.mark.parametrize("score,ng", [(0, 1), (1, 1), (1, 4)])
def test_route_masked_experts(score, ng):
    """-inf logits (masked experts), including tokens with fewer finite logits than k: indices
    and weights bit for bit the oracle's (no placeholder index escapes)."""
    from test_oracle_pins import masked_logits
    T, E, k = 512, 64, 6
    z = masked_logits(T, E, 22, [1, 2, 5, 6, 7, 40] if score == 0 else [0, 1, 2, 5, 6, 7, 40])
    gcfg = M.router_cfg(E, k, score, True, ng, 2 if ng > 1 else 1, 2)
    ocfg = O.router_cfg(E, k, score, True, ng, 2 if ng > 1 else 1, 2)
    zd = torch.from_numpy(z).to(DEV)
    idx, w = M.moe_route(zd, gcfg)
    oidx, ow = O.moe_route(z, ocfg)
    assert_equal("idx", host(idx), oidx)
    assert_equal("w", host(w), ow)
    x = synth.randn((T, 256), 22, synth.STAGE, part=77, device=DEV)
    fidx, fw, _, _ = M.moe_route_quant(zd, gcfg, x)
    assert_equal("fused idx", host(fidx), oidx)
    assert_equal("fused w", host(fw), ow)


@pytest.mark.parametrize("E,k,score,ng,tg,gt", [(1024, 64, 0, 1, 1, 2), (1024, 8, 1, 64, 7, 3), (96, 5, 1, 3, 2, 1),
                                                (2, 2, 0, 1, 1, 2), (1, 1, 1, 1, 1, 2), (130, 3, 0, 1, 1, 2)])
def test_route_extreme_shapes(E, k, score, ng, tg, gt):
    """Largest supported E and k, E not a multiple of 64, many groups, k = E, one token."""
    for T in (1, 333):
        z = synth.randn((T, E), 7, synth.STAGE, part=34, device=DEV) * 3
        gcfg = M.router_cfg(E, k, score, True, ng, tg, gt)
        ocfg = O.router_cfg(E, k, score, True, ng, tg, gt)
        idx, w = M.moe_route(z, gcfg)
        oidx, ow = O.moe_route(host(z), ocfg)
        assert_equal(f"idx T={T}", host(idx), oidx)
        assert_equal(f"w T={T}", host(w), ow)


# ----------------------------------------------------------------------------- dispatch
@pytest.mark.parametrize("name", NAMES)
def test_dispatch(name):
    cfg = synth.CONFIGS[name]
    T, k, E, H = cfg.T, cfg.k, cfg.E, cfg.H
    idx = synth.routing_indices(cfg, T).numpy()
    idx[3, 0] = -1                      # a dropped slot (as left by a rejected replay token)
    idx[T - 1, :] = -1
    xq = synth.random_codes((T, H), cfg.seed, 40, device=DEV)
    xs = synth.random_scales((T, H // 128), cfg.seed, 41, device=DEV)
    d = M.moe_dispatch(torch.from_numpy(idx).to(DEV), E, cfg.shared, xq, xs)
    oc, oo, od, osrc = O.moe_dispatch(idx, E, cfg.shared)
    assert_equal("counts", host(d.counts), oc)
    assert_equal("offsets", host(d.offsets), oo)
    assert_equal("dest_row", host(d.dest_row), od)
    nrows = int(oo[-1])
    assert_equal("src_token", host(d.src_token)[:nrows], osrc)
    rows = np.arange(nrows) if nrows <= 4096 else np.unique(np.concatenate(
        [synth.sample_tokens(nrows, 2048, cfg.seed), oo[:-1][oo[:-1] < nrows], np.maximum(oo[1:] - 1, 0)]))
    xqh, xsh = host(xq), host(xs)
    assert_equal("aq rows", rows_host(d.aq, rows), O.permute_rows(xqh, osrc[rows]))
    assert_equal("as rows", rows_host(d.as_, rows), O.permute_rows(xsh, osrc[rows]))
    # index-only mode
    d2 = M.moe_dispatch(torch.from_numpy(idx).to(DEV), E, cfg.shared)
    assert_equal("dest_row (index only)", host(d2.dest_row), od)
    # scales-only mode (the GEMM gathers the codes): every row's scales
    d3 = M.moe_dispatch(torch.from_numpy(idx).to(DEV), E, cfg.shared, xq, xs, copy_codes=False)
    assert d3.aq is None
    assert_equal("as rows (scales only)", host(d3.as_)[:nrows], O.permute_rows(xsh, osrc))
    del xq, xs, d, d2, d3
    _cleanup()


@pytest.mark.parametrize("H", [128, 384, 512, 1536, 6144])
@pytest.mark.parametrize("T", [1, 61, 1000])
def test_dispatch_scales_only_ragged(H, T):
    """Scales-only permutation on row counts that are not multiples of a workgroup's rows and
    scale rows of 1..48 floats (whole 16-byte pieces or not), with the shared expert appended."""
    E, k = 64, 6
    rng = np.random.default_rng(H + T)
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    xs = synth.random_scales((T, H // 128), 7, 42, device=DEV)
    xq = synth.random_codes((T, H), 7, 43, device=DEV)
    d = M.moe_dispatch(torch.from_numpy(idx).to(DEV), E, True, xq, xs, copy_codes=False)
    _, oo, _, osrc = O.moe_dispatch(idx, E, True)
    nrows = int(oo[-1])
    assert_equal("as rows", host(d.as_)[:nrows], O.permute_rows(host(xs), osrc))


def test_dispatch_all_one_expert_and_tiny():
    """Every slot on one expert (all others empty), and a single token."""
    for T, k, E in ((5000, 4, 16), (1, 3, 7)):
        idx = np.stack([np.full(T, 2, np.int32)] + [np.full(T, (2 + j) % E, np.int32) for j in range(1, k)], 1)
        d = M.moe_dispatch(torch.from_numpy(idx).to(DEV), E, True)
        oc, oo, od, osrc = O.moe_dispatch(idx, E, True)
        assert_equal("counts", host(d.counts), oc)
        assert_equal("offsets", host(d.offsets), oo)
        assert_equal("dest", host(d.dest_row), od)
        assert_equal("src", host(d.src_token)[:oo[-1]], osrc)


@pytest.mark.parametrize("T,k,E", [(2048, 4, 64), (2049, 4, 64), (100, 8, 1024), (300, 6, 2), (1, 1, 1),
                                   (1024, 8, 256), (640, 2, 1000)])
def test_dispatch_small_and_chunked_paths(T, k, E):
    """Batches on both sides of the one-workgroup path's limits (8192 slots, 16384 piece x expert
    counters), every expert-id width, and dropped (-1) slots."""
    rng = np.random.default_rng(T * 7 + k * 3 + E)
    idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
    idx[rng.random((T, k)) < 0.05] = -1
    for shared in (False, True):
        d = M.moe_dispatch(torch.from_numpy(idx).to(DEV), E, shared)
        oc, oo, od, osrc = O.moe_dispatch(idx, E, shared)
        assert_equal("counts", host(d.counts), oc)
        assert_equal("offsets", host(d.offsets), oo)
        assert_equal("dest_row", host(d.dest_row), od)
        assert_equal("src_token", host(d.src_token)[:oo[-1]], osrc)


@pytest.mark.parametrize("T,k,E,shared", [(256, 6, 64, False), (96, 8, 32, True), (1, 8, 256, True),
                                           (0, 6, 64, False), (2048, 8, 256, True),
                                           (3, 2, 1023, True), (4, 2, 1024, True),    # G = 1024, 1025
                                           (1024, 8, 16, True), (1000, 8, 24, False),   # one workgroup, all lists
                                           (4096, 8, 64, False), (4096, 8, 8, True),   # chunked: the scan writes them
                                           (200, 8, 1023, True), (200, 8, 1024, True)])  # chunked, G = 1024, 1025
def test_dispatch_plan_equals_separate_plan(T, k, E, shared):
    """moe_dispatch_plan: the same dispatch outputs as moe_dispatch and the same tile list (every
    entry and the count) as moe_grouped_gemm_plan, for each tile height.  The dispatch's own
    one-workgroup kernel writes the plan (the whole dispatch for small batches, else the scan of the
    chunk histograms) up to 1024 groups; with more, the plan kernel runs after the dispatch."""
    rng = np.random.default_rng(T + E)
    idx = torch.from_numpy(rng.integers(0, E, size=(T, k)).astype(np.int32)).to(DEV)
    H = 256
    xq = synth.random_codes((T, H), 8, 44, device=DEV)
    xs = synth.random_scales((T, H // 128), 8, 45, device=DEV)
    G = E + (1 if shared else 0)
    max_rows = T * k + (T if shared else 0)
    ref = M.moe_dispatch(idx, E, shared, xq, xs, copy_codes=False)
    for tile in (0, 32, 48, 64, 128, 256):
        out = M.moe_dispatch(idx, E, shared, xq, xs, copy_codes=False)   # fresh buffers of the same shape
        for t_ in (out.counts, out.offsets, out.dest_row, out.src_token, out.as_):
            t_.fill_(-9)
        ws = torch.empty(M.workspace_bytes(M.MOE_OP_DISPATCH, T, k, E), dtype=torch.uint8, device=DEV)
        gws = torch.full((max(M.workspace_bytes(M.MOE_OP_GROUPED_GEMM, max_rows, 0, G, 0, 0), 256),), 0xEE,
                         dtype=torch.uint8, device=DEV)
        gws2 = gws.clone()
        plan = M.moe_dispatch_plan(idx, E, shared, xq, xs, ws, out, gws, tile_rows=tile)
        plan2 = M.moe_grouped_gemm_plan(ref.offsets, max_rows, gws2, tile_rows=tile)
        torch.cuda.synchronize()
        assert (plan.tile_rows, plan.groups, plan.max_rows) == (plan2.tile_rows, plan2.groups, plan2.max_rows)
        for name in ("counts", "offsets", "dest_row"):
            assert_equal(f"{name} tile {tile}", host(getattr(out, name)), host(getattr(ref, name)))
        n = int(host(ref.offsets)[-1])
        assert_equal(f"src tile {tile}", host(out.src_token)[:n], host(ref.src_token)[:n])
        assert_equal(f"as tile {tile}", host(out.as_)[:n], host(ref.as_)[:n])
        if max_rows == 0:
            continue
        nt = int(host(gws2[:4].view(torch.int32))[0])
        assert int(host(gws[:4].view(torch.int32))[0]) == nt
        assert_equal(f"tiles tile {tile}", host(gws[256:256 + 16 * nt]), host(gws2[256:256 + 16 * nt]))
        # both lists against their definition: group order, and (128- and 256-row tiles, when the
        # workspace holds it) every group's full tiles first, then the groups' short last tiles
        l1, l2, l3, second, third = _expected_tile_lists(host(ref.offsets), plan.tile_rows, max_rows, G)
        assert nt == len(l1)
        got1 = host(gws[256:256 + 16 * nt].view(torch.int32)).reshape(-1, 4)
        assert_equal(f"list 1 tile {tile}", got1, np.array(l1, np.int32).reshape(-1, 4))
        for w in (gws, gws2):
            head = host(w[:12].view(torch.int32))
            if second:
                assert int(head[1]) == len(l2), (tile, head, len(l2))
                got2 = host(w[256 + 16 * second:256 + 16 * (second + len(l2))].view(torch.int32)).reshape(-1, 4)
                assert_equal(f"list 2 tile {tile}", got2, np.array(l2, np.int32).reshape(-1, 4))
            if third:
                assert int(head[2]) == len(l3), (tile, head, len(l3))
                got3 = host(w[256 + 16 * third:256 + 16 * (third + len(l3))].view(torch.int32)).reshape(-1, 4)
                assert_equal(f"list 3 tile {tile}", got3, np.array(l3, np.int32).reshape(-1, 4))


def _expected_tile_lists(offsets, bm, max_rows, G):
    """The grouped GEMM's tile lists from their definition: entries {group, first row, first tile of
    the entry's block, tiles in the block}.  List 1: group order.  List 2 (128- and 256-row tiles,
    when the workspace holds it): every group's full tiles, then the short last tiles; for 256-row
    tiles with room for `groups` more entries, only the short tiles of more than 128 rows, the
    others (1 .. 128 rows) forming list 3 as 128-row tiles.  Returns (l1, l2, l3, second, third)."""
    rows = np.diff(offsets[:G + 1])
    l1 = []
    for g in range(G):
        n = -(-int(rows[g]) // bm)
        f = len(l1)
        l1 += [(g, int(offsets[g]) + i * bm, f, n) for i in range(n)]
    mt = -(-max_rows // bm) + G
    cap = -(-max_rows // 32) + G
    second = mt if bm >= 128 and 2 * mt <= cap else 0
    third = 2 * second if bm == 256 and second and 2 * second + G <= cap else 0
    l2, l3 = [], []
    if second:
        for g in range(G):
            n = int(rows[g]) // bm
            f = len(l2)
            l2 += [(g, int(offsets[g]) + i * bm, f, n) for i in range(n)]
        for g in range(G):
            r = int(rows[g]) % bm
            start = int(offsets[g]) + (int(rows[g]) // bm) * bm
            if r > (128 if third else 0):
                l2.append((g, start, len(l2), 1))
            elif third and r > 0:
                l3.append((g, start, len(l3), 1))
    return l1, l2, l3, second, third


@pytest.mark.parametrize("H", [128, 1152, 8192, 8320])
def test_dispatch_permute_widths(H):
    """Row permutation at several widths: a row shorter than one wavefront's 16-byte pieces, a
    partial last round of pieces, 8 KB and a wider row; with a shared expert and dropped slots,
    every row compared."""
    T, k, E = 300, 3, 5
    rng = np.random.default_rng(H)
    idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
    idx[rng.random((T, k)) < 0.05] = -1
    xq = synth.random_codes((T, H), 7, 42, device=DEV)
    xs = synth.random_scales((T, H // 128), 7, 43, device=DEV)
    for shared in (False, True):
        d = M.moe_dispatch(torch.from_numpy(idx).to(DEV), E, shared, xq, xs)
        _, oo, _, osrc = O.moe_dispatch(idx, E, shared)
        n = int(oo[-1])
        assert_equal(f"aq H={H}", host(d.aq)[:n], O.permute_rows(host(xq), osrc))
        assert_equal(f"as H={H}", host(d.as_)[:n], O.permute_rows(host(xs), osrc))
        # scales only (the codes are then gathered by the grouped GEMM): same indices and scales,
        # no code copy
        ds = M.moe_dispatch(torch.from_numpy(idx).to(DEV), E, shared, xq, xs, copy_codes=False)
        assert ds.aq is None
        assert_equal(f"src H={H}", host(ds.src_token)[:n], osrc)
        assert_equal(f"as only H={H}", host(ds.as_)[:n], O.permute_rows(host(xs), osrc))


# ----------------------------------------------------------------------------- grouped GEMM
def _gemm_case(cfg, which, part):
    """Random codes/scales with the workload's group sizes; offsets from the oracle dispatch of
    synthetic routing indices."""
    G = cfg.groups
    N, K = (2 * cfg.F, cfg.H) if which == "w1" else (cfg.H, cfg.F)
    idx = synth.routing_indices(cfg, cfg.T, seed_part=part).numpy()
    _, offsets, _, _ = O.moe_dispatch(idx, cfg.E, cfg.shared)
    rows = int(offsets[-1])
    a = synth.random_codes((rows, K), cfg.seed, 50 + part, device=DEV)
    as_ = synth.random_scales((rows, K // 128), cfg.seed, 51 + part, device=DEV, lo=2.0 ** -10, hi=2.0 ** -6)
    b = synth.random_codes((G, N, K), cfg.seed, 52 + part, device=DEV)
    bs = synth.random_scales((G, N // 128, K // 128), cfg.seed, 53 + part, device=DEV, lo=2.0 ** -10, hi=2.0 ** -6)
    return offsets, a, as_, b, bs, N, K


def _sample_rows(offsets, n, seed):
    rows = int(offsets[-1])
    nonempty = [g for g in range(len(offsets) - 1) if offsets[g + 1] > offsets[g]]
    pick = set()
    rng = np.random.default_rng(seed)
    for g in rng.choice(nonempty, size=min(6, len(nonempty)), replace=False):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        pick |= {lo, hi - 1} | {min(lo + d, hi - 1) for d in (31, 32, 127, 128)}   # group and tile edges
    pick |= set(synth.sample_tokens(rows, n, seed).tolist())
    return np.array(sorted(pick))


def _oracle_rows(a, as_, offsets, b, bs, rows):
    """fp64 reference rows, one group's dequantised weights at a time."""
    grp = np.searchsorted(offsets, rows, side="right") - 1
    a_h, as_h = rows_host(a, rows), rows_host(as_, rows)
    pos = {int(r): i for i, r in enumerate(rows)}
    out = {}
    for g in np.unique(grp):
        rr = rows[grp == g]
        ii = [pos[int(r)] for r in rr]
        wd = O.dequant_weight(host(b[g]), host(bs[g]))
        ref = O.dequant_act(a_h[ii], as_h[ii]) @ wd.T
        for r, v in zip(rr, ref):
            out[int(r)] = v
    return np.stack([out[int(r)] for r in rows]), grp


@pytest.mark.parametrize("name", NAMES)
@pytest.mark.parametrize("which", ["w1", "w2"])
@pytest.mark.parametrize("tile", TILES)
def test_grouped_gemm_store(name, which, tile):
    cfg = synth.CONFIGS[name]
    offsets, a, as_, b, bs, N, K = _gemm_case(cfg, which, 0 if which == "w1" else 5)
    goff = torch.from_numpy(offsets).to(DEV)
    bw = _weights_for(b, M.MOE_EPI_STORE, tile)
    y32 = M.moe_grouped_gemm_fp8(a, as_, goff, bw, bs, M.MOE_EPI_STORE, torch.float32, tile_rows=tile)
    ybf = M.moe_grouped_gemm_fp8(a, as_, goff, bw, bs, M.MOE_EPI_STORE, torch.bfloat16, tile_rows=tile)
    rows = _sample_rows(offsets, 24, cfg.seed)
    ref, _ = _oracle_rows(a, as_, offsets, b, bs, rows)
    e32 = rel_err(rows_host(y32, rows), ref)
    ebf = rel_err(rows_host(ybf, rows), ref)
    print(f"{name} {which} tile {tile}: fp32-out err {e32:.3e}, bf16-out err {ebf:.3e}")
    # uniformly random codes are heavy-tailed (log-uniform magnitudes), so fp32 accumulation error
    # relative to max |ref| reaches ~1e-4; the contract bound for GEMM outputs is TOL
    assert e32 < 1e-3 and ebf < TOL
    del a, as_, b, bs, y32, ybf
    _cleanup()


@pytest.mark.parametrize("epi", ["swiglu", "store"])
def test_grouped_gemm_split_launches(epi):
    """256-row plans run as two launches (full tiles and short tiles over 128 rows, then the short
    remainders of 1 .. 128 rows as 128-row tiles).  Every tile height computes the same sums in the
    same order, so the output equals the one-launch 128-row tiles' bit for bit on every row, with
    group sizes around each boundary (0, 1, 127 .. 129, 255 .. 257, 383 .. 385 rows); sampled rows,
    every remainder's first and last among them, against the oracle."""
    counts = np.array([0, 1, 5, 31, 64, 100, 127, 128, 129, 200, 255, 256, 257, 300, 383, 384, 385, 511, 512,
                       513, 700, 1000, 0, 1, 2, 90, 160, 1400, 30, 3, 250, 129, 128, 127, 640, 900, 17, 0, 64, 2000])
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    G, rows = len(counts), int(offsets[-1])
    N, K = 512, 256
    a = synth.random_codes((rows, K), 9, 60, device=DEV)
    as_ = synth.random_scales((rows, K // 128), 9, 61, device=DEV, lo=2.0 ** -10, hi=2.0 ** -6)
    b = synth.random_codes((G, N, K), 9, 62, device=DEV)
    bs = synth.random_scales((G, N // 128, K // 128), 9, 63, device=DEV, lo=2.0 ** -10, hi=2.0 ** -6)
    goff = torch.from_numpy(offsets).to(DEV)
    e = M.MOE_EPI_SWIGLU_QUANT if epi == "swiglu" else M.MOE_EPI_STORE
    pk = M.moe_pack_weights_fp8(b, e)
    # the plan has the third list, with the remainders of 1 .. 128 rows in it
    ws = torch.empty(M.workspace_bytes(M.MOE_OP_GROUPED_GEMM, rows, 0, G, 0, 0), dtype=torch.uint8, device=DEV)
    plan = M.moe_grouped_gemm_plan(goff, rows, ws, tile_rows=256)
    n3 = int(host(ws[:12].view(torch.int32))[2])
    assert plan.tile_rows == 256 and n3 == int(((counts % 256 > 0) & (counts % 256 <= 128)).sum())
    outs = {}
    for tile in (256, 128):
        if e == M.MOE_EPI_STORE:
            outs[tile] = (M.moe_grouped_gemm_fp8(a, as_, goff, pk, bs, e, torch.float32, tile_rows=tile),)
        else:
            outs[tile] = M.moe_grouped_gemm_fp8(a, as_, goff, pk, bs, e, tile_rows=tile)
    for x, y in zip(outs[256], outs[128]):
        assert_equal(f"{epi}: 256-row plan (two launches) against 128-row tiles", host(x), host(y))
    if e == M.MOE_EPI_STORE:
        rem0 = offsets[:-1] + counts // 256 * 256
        edge = np.concatenate([rem0[counts % 256 > 0], offsets[1:][counts > 0] - 1])
        smp = np.unique(np.concatenate([edge, synth.sample_tokens(rows, 40, 9)]))
        ref, _ = _oracle_rows(a, as_, offsets, b, bs, smp)
        assert rel_err(rows_host(outs[256][0], smp), ref) < 1e-3


def test_grouped_gemm_exact_integers():
    """Integer codes in [-8,8] with unit or common power-of-two scales: every partial and total
    is an exact fp32 integer, so the result is bitwise equal in any accumulation order."""
    offsets = np.array([0, 130, 130, 131, 400, 657], np.int64)   # an empty group, a 1-row group, ragged tails
    G, N, K = 5, 384, 1024
    rows = int(offsets[-1])
    a, ai = synth.integer_codes((rows, K), 60, 0, device=DEV)
    b, bi = synth.integer_codes((G, N, K), 60, 1, device=DEV)
    for (sa, sb), tile in itertools.product(((1.0, 1.0), (0.25, 8.0)), TILES):
        as_ = torch.full((rows, K // 128), sa, dtype=torch.float32, device=DEV)
        bs = torch.full((G, N // 128, K // 128), sb, dtype=torch.float32, device=DEV)
        goff = torch.from_numpy(offsets.astype(np.int32)).to(DEV)
        ref = O.moe_grouped_gemm_fp8(host(a), host(as_), offsets, host(b), host(bs))
        for bw in (b, M.moe_pack_weights_fp8(b, M.MOE_EPI_STORE)):   # N = 384: a zero-padded packed panel
            if tile == 256 and isinstance(bw, torch.Tensor):
                continue                                              # 256-row tiles: packed weights only
            y = M.moe_grouped_gemm_fp8(a, as_, goff, bw, bs, M.MOE_EPI_STORE, torch.float32, tile_rows=tile)
            assert_equal(f"exact integer GEMM (scales {sa},{sb}, tile {tile}, {type(bw).__name__})", host(y),
                         ref.astype(np.float32))
        assert np.array_equal(ref, sa * sb * np.concatenate(
            [ai[offsets[g]:offsets[g + 1]].numpy() @ bi[g].numpy().T for g in range(G)]))


def test_grouped_gemm_exact_integers_bf16_out():
    """The bf16 store epilogue (the tile staged through LDS in rounds of up to 64 rows, each row
    stored as one contiguous piece) on the exact-integer case with N = 384, whose second weight
    panel has only 128 valid columns: every value equals the exact result rounded to bf16 (round to
    nearest even), for every tile height, so no column past N is written (it would land in the next
    row) and no row past a group's end."""
    offsets = np.array([0, 130, 130, 131, 400, 657, 1357], np.int64)   # a 700-row group: 256-row units
    G, N, K = 6, 384, 512
    rows = int(offsets[-1])
    a, ai = synth.integer_codes((rows, K), 61, 0, device=DEV)
    b, bi = synth.integer_codes((G, N, K), 61, 1, device=DEV)
    as_ = torch.full((rows, K // 128), 0.5, dtype=torch.float32, device=DEV)
    bs = torch.full((G, N // 128, K // 128), 4.0, dtype=torch.float32, device=DEV)
    goff = torch.from_numpy(offsets.astype(np.int32)).to(DEV)
    exact = 2.0 * np.concatenate([ai[offsets[g]:offsets[g + 1]].numpy().astype(np.int64) @
                                  bi[g].numpy().astype(np.int64).T for g in range(G)])
    want = torch.from_numpy(exact.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    packed = M.moe_pack_weights_fp8(b, M.MOE_EPI_STORE)
    for tile in TILES:
        for bw in (b, packed):
            if tile == 256 and isinstance(bw, torch.Tensor):
                continue                                              # 256-row tiles: packed weights only
            y = M.moe_grouped_gemm_fp8(a, as_, goff, bw, bs, M.MOE_EPI_STORE, torch.bfloat16, tile_rows=tile)
            assert_equal(f"exact integer GEMM, bf16 out (tile {tile}, {type(bw).__name__})",
                         host(y.view(torch.int16)), want)


def _expected_pack(b: np.ndarray, epi: int) -> np.ndarray:
    """The packed layout written out: block (g, panel, K step) = 2048 units of 16 bytes; unit
    64 i + L holds 16-byte chunk 2 (L // 16) + i % 2 of panel row r = 16 (i // 2) + L % 16."""
    G, N, K = b.shape
    KB, F = K // 128, N // 2
    ny = N // 256 if epi == M.MOE_EPI_SWIGLU_QUANT else -(-N // 256)
    u = np.arange(2048)
    i, lane = u >> 6, u & 63
    r = 16 * (i >> 1) + (lane & 15)
    chunk = 2 * (lane >> 4) + (i & 1)
    out = np.zeros((G, ny, KB, 2048, 16), np.uint8)
    for nt in range(ny):
        if epi == M.MOE_EPI_SWIGLU_QUANT:
            n = np.where(r < 128, nt * 128 + r, F + nt * 128 + r - 128)
        else:
            n = nt * 256 + r
        ok = n < N
        for kb in range(KB):
            cols = kb * 128 + chunk[:, None] * 16 + np.arange(16)
            out[:, nt, kb, ok] = b[:, n[ok][:, None], cols[ok]]
    return out.reshape(G, -1)


@pytest.mark.parametrize("epi,N", [(M.MOE_EPI_STORE, 384), (M.MOE_EPI_STORE, 512), (M.MOE_EPI_SWIGLU_QUANT, 512)])
def test_pack_weights_layout(epi, N):
    G, K = 3, 384
    b = synth.random_codes((G, N, K), 7, N + epi, device=DEV)
    pw = M.moe_pack_weights_fp8(b, epi)
    assert_equal(f"packed weight (epilogue {epi}, N {N})", host(pw.data), _expected_pack(host(b), epi))


@pytest.mark.parametrize("name", NAMES)
@pytest.mark.parametrize("tile", TILES)
def test_grouped_gemm_packed_equals_rowmajor(name, tile):
    """Packing only moves bytes: every output, code and scale is bitwise the row-major result."""
    cfg = synth.CONFIGS[name]
    for which, epi in (("w1", M.MOE_EPI_SWIGLU_QUANT), ("w2", M.MOE_EPI_STORE)):
        offsets, a, as_, b, bs, N, K = _gemm_case(cfg, which, 11)
        goff = torch.from_numpy(offsets).to(DEV)
        pw = M.moe_pack_weights_fp8(b, epi)
        # 256-row tiles take packed weights only: their result is compared with the row-major
        # weights at 128-row tiles (the accumulation order of an output does not depend on the
        # tile height, so the two are bitwise equal)
        r0 = M.moe_grouped_gemm_fp8(a, as_, goff, b, bs, epi, torch.float32, tile_rows=128 if tile == 256 else tile)
        r1 = M.moe_grouped_gemm_fp8(a, as_, goff, pw, bs, epi, torch.float32, tile_rows=tile)
        rows = int(offsets[-1])
        if epi == M.MOE_EPI_STORE:
            assert torch.equal(r0[:rows].view(torch.int32), r1[:rows].view(torch.int32)), f"{name} {which}"
        else:
            assert torch.equal(r0[0][:rows], r1[0][:rows]) and torch.equal(r0[1][:rows], r1[1][:rows]), f"{name} {which}"
        del a, as_, b, bs, pw, r0, r1
        _cleanup()


def test_grouped_gemm_gathered_rows_clamped():
    """Row ids outside [0, a_count) are clamped into it (the documented safety net): the group rows
    that name -5 and a_count + 7 get exactly the results of rows 0 and a_count - 1."""
    G, N, K, T = 2, 256, 256, 40
    offsets = np.array([0, 20, 33], np.int32)
    rows = 33
    rng = np.random.default_rng(9)
    src = rng.integers(0, T, rows).astype(np.int32)
    bad = src.copy()
    bad[3], bad[25] = -5, T + 7
    want = src.copy()
    want[3], want[25] = 0, T - 1
    x = synth.randn((T, K), 42, synth.STAGE, part=1, device=DEV)
    xq, xs = M.moe_quant_fp8_block(x, 1)
    w = synth.randn((G, N, K), 42, synth.STAGE, part=2, device=DEV, std=K ** -0.5)
    bq, bsc = M.moe_quant_fp8_block(w, 128)
    goff = torch.from_numpy(offsets).to(DEV)
    ws = torch.empty(M.workspace_bytes(M.MOE_OP_GROUPED_GEMM, rows, 0, G, 0, 0), dtype=torch.uint8, device=DEV)
    plan = M.moe_grouped_gemm_plan(goff, rows, ws)
    pk = M.moe_pack_weights_fp8(bq, M.MOE_EPI_STORE)
    as_ = xs[torch.from_numpy(want).long().to(DEV)].contiguous()
    got = M.moe_grouped_gemm_fp8(xq, as_, goff, pk, bsc, M.MOE_EPI_STORE, torch.float32, plan=plan,
                                 a_rows=torch.from_numpy(bad).to(DEV))
    ref = M.moe_grouped_gemm_fp8(xq, as_, goff, pk, bsc, M.MOE_EPI_STORE, torch.float32, plan=plan,
                                 a_rows=torch.from_numpy(want).to(DEV))
    torch.cuda.synchronize()
    assert_equal("clamped rows", host(got), host(ref))


@pytest.mark.parametrize("tile", [32, 48, 64, 128, 256])
@pytest.mark.parametrize("pow2", [False, True])
def test_grouped_gemm_gathered_rows(tile, pow2):
    """A rows gathered from a token-order matrix through a row-id list (repeats, any order) give
    bitwise the GEMM of the explicitly permuted copy: store (bf16, fp32) and SwiGLU epilogues, and
    FP4 weights with power-of-two scales."""
    rng = np.random.default_rng(tile + 7 * pow2)
    G, N, K, T = 5, 512, 768, 300
    counts = np.array([0, 130, 1, 257, 77])
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rows = int(offsets[-1]) + 9                               # a few rows past the last group
    src = torch.from_numpy(rng.integers(0, T, rows).astype(np.int32)).to(DEV)
    x = synth.randn((T, K), 41, synth.STAGE, part=tile, device=DEV)
    xq, xs = M.moe_quant_fp8_block(x, 1, pow2=pow2)
    aq = xq[src.long()].contiguous()
    as_ = xs[src.long()].contiguous()
    w = synth.randn((G, N, K), 41, synth.STAGE, part=100 + tile, device=DEV, std=K ** -0.5)
    bq, bsc = M.moe_quant_fp8_block(w, 128, pow2=pow2)
    goff = torch.from_numpy(offsets).to(DEV)
    ws = torch.empty(M.workspace_bytes(M.MOE_OP_GROUPED_GEMM, rows, 0, G, 0, 0), dtype=torch.uint8, device=DEV)
    plan = M.moe_grouped_gemm_plan(goff, rows, ws, tile_rows=tile)
    n = int(offsets[-1])
    for epi in (M.MOE_EPI_STORE, M.MOE_EPI_SWIGLU_QUANT):
        pk = M.moe_pack_weights_fp8(bq, epi)
        for od in ((torch.bfloat16, torch.float32) if epi == M.MOE_EPI_STORE else (None,)):
            kw = dict(out_dtype=od) if od is not None else {}
            ref = M.moe_grouped_gemm_fp8(aq, as_, goff, pk, bsc, epi, plan=plan, pow2=pow2, **kw)
            got = M.moe_grouped_gemm_fp8(xq, as_, goff, pk, bsc, epi, plan=plan, pow2=pow2, a_rows=src, **kw)
            if epi == M.MOE_EPI_STORE:
                assert_equal(f"store {od}", host(got)[:n], host(ref)[:n])
            else:
                assert_equal("h codes", host(got[0])[:n], host(ref[0])[:n])
                assert_equal("h scales", host(got[1])[:n], host(ref[1])[:n])
    if pow2:
        q4, e8 = M.moe_quant_mxfp4(w)
        pk4 = M.moe_pack_weights_fp4(q4, e8, M.MOE_EPI_STORE)
        ref = M.moe_grouped_gemm_fp8(aq, as_, goff, pk4, None, M.MOE_EPI_STORE, torch.float32, plan=plan, pow2=True)
        got = M.moe_grouped_gemm_fp8(xq, as_, goff, pk4, None, M.MOE_EPI_STORE, torch.float32, plan=plan, pow2=True,
                                     a_rows=src)
        assert_equal("fp4 store", host(got)[:n], host(ref)[:n])
    torch.cuda.synchronize()


@pytest.mark.parametrize("name", ["tiny", "decode", "longctx"])
def test_grouped_gemm_plan_shared_by_two_gemms(name):
    """One plan, two GEMMs (SwiGLU over W1, then store over W2), bitwise equal to the one-call path
    for the automatic and every explicit tile height."""
    cfg = synth.CONFIGS[name]
    offsets, a, as_, b1, bs1, N1, K1 = _gemm_case(cfg, "w1", 13)
    goff = torch.from_numpy(offsets).to(DEV)
    rows = int(offsets[-1])
    G = cfg.groups
    b2 = synth.random_codes((G, K1, N1 // 2), cfg.seed, 60, device=DEV)
    bs2 = synth.random_scales((G, K1 // 128, N1 // 256), cfg.seed, 61, device=DEV, lo=2.0 ** -10, hi=2.0 ** -6)
    p1, p2 = M.moe_pack_weights_fp8(b1, M.MOE_EPI_SWIGLU_QUANT), M.moe_pack_weights_fp8(b2, M.MOE_EPI_STORE)
    ws = torch.empty(M.workspace_bytes(M.MOE_OP_GROUPED_GEMM, rows, 0, G), dtype=torch.uint8, device=DEV)
    for tile in [0] + TILES:
        plan = M.moe_grouped_gemm_plan(goff, rows, ws, tile_rows=tile)
        hq, hs = M.moe_grouped_gemm_fp8(a, as_, goff, p1, bs1, M.MOE_EPI_SWIGLU_QUANT, plan=plan)
        y = M.moe_grouped_gemm_fp8(hq, hs, goff, p2, bs2, M.MOE_EPI_STORE, torch.bfloat16, plan=plan)
        hq0, hs0 = M.moe_grouped_gemm_fp8(a, as_, goff, p1, bs1, M.MOE_EPI_SWIGLU_QUANT, tile_rows=plan.tile_rows)
        y0 = M.moe_grouped_gemm_fp8(hq0, hs0, goff, p2, bs2, M.MOE_EPI_STORE, torch.bfloat16, tile_rows=plan.tile_rows)
        assert torch.equal(hq[:rows], hq0[:rows]) and torch.equal(hs[:rows], hs0[:rows]), (name, tile)
        assert torch.equal(y[:rows].view(torch.int16), y0[:rows].view(torch.int16)), (name, tile)
    del a, as_, b1, b2, p1, p2
    _cleanup()


@pytest.mark.parametrize("name", NAMES)
@pytest.mark.parametrize("tile", TILES)
def test_grouped_gemm_swiglu_quant(name, tile):
    cfg = synth.CONFIGS[name]
    offsets, a, as_, b, bs, N, K = _gemm_case(cfg, "w1", 9)
    F = N // 2
    goff = torch.from_numpy(offsets).to(DEV)
    hq, hs = M.moe_grouped_gemm_fp8(a, as_, goff, _weights_for(b, M.MOE_EPI_SWIGLU_QUANT, tile), bs,
                                    M.MOE_EPI_SWIGLU_QUANT, tile_rows=tile)
    rows = _sample_rows(offsets, 16, cfg.seed + 1)
    g1, _ = _oracle_rows(a, as_, offsets, b, bs, rows)
    h = O.swiglu(g1, F)
    rq, rs = O.moe_quant_fp8_block(h, 1)
    gq, gs = rows_host(hq, rows), rows_host(hs, rows)
    # h depends on the GEMM's last bits (fp32 accumulation of heavy-tailed random codes, ~1e-4
    # relative to the block max), so scales agree to that level and codes to within one e4m3 step
    assert np.max(np.abs(gs / rs - 1)) < 1e-3
    tab = O.e4m3_table()
    dg = tab[gq] * np.repeat(gs, 128, 1)
    dr = tab[rq] * np.repeat(rs, 128, 1)
    # one e4m3 step (1/8 relative, or the subnormal step of the larger scale) plus the scale mismatch
    smax = np.repeat(np.maximum(rs, gs), 128, 1)
    # plus GEMM1's absolute error, ~1e-4 of the block max (amax = 448 s), which dominates for h near 0
    step = np.abs(dr) / 8 + smax * 2.0 ** -9 + np.abs(dr) * np.abs(np.repeat(gs / rs, 128, 1) - 1) + 448 * smax * 1e-3
    viol = np.argwhere(np.abs(dg - dr) > step * 1.0001)
    assert viol.size == 0, [(tuple(v), float(dg[tuple(v)]), float(dr[tuple(v)]), hex(gq[tuple(v)]), hex(rq[tuple(v)]),
                             float(gs[v[0], v[1] // 128]), float(rs[v[0], v[1] // 128]), float(h[tuple(v)]))
                            for v in viol[:6]]
    frac = np.mean(gq != rq)
    print(f"{name}: h code mismatch fraction {frac:.2e}, deq(h) err vs fp64 h {rel_err(dg, h):.3e}")
    assert frac < 1e-2
    del a, as_, b, bs, hq, hs
    _cleanup()


# ----------------------------------------------------------------------------- combine
@pytest.mark.parametrize("name", NAMES)
def test_combine(name):
    cfg = synth.CONFIGS[name]
    T, k, E, H = cfg.T, cfg.k, cfg.E, cfg.H
    idx = synth.routing_indices(cfg, T, seed_part=3).numpy()
    idx[2, 1 % k] = -1
    _, offsets, dest, _ = O.moe_dispatch(idx, E, cfg.shared)
    rows = int(offsets[-1])
    act = torch.bfloat16 if cfg.act == "bf16" else torch.float32
    y = synth.randn((rows, H), cfg.seed, synth.STAGE, part=70, device=DEV).to(act)
    w = torch.rand((T, k), generator=torch.Generator().manual_seed(cfg.seed), dtype=torch.float32)
    gdest = torch.from_numpy(dest).to(DEV)
    goff = torch.from_numpy(offsets).to(DEV)
    shared = goff[E:E + 1] if cfg.shared else None
    out = M.moe_combine(y, gdest, w.to(DEV), shared)
    toks = np.arange(T) if T <= 512 else synth.sample_tokens(T, 256, cfg.seed)
    # the rows those tokens read, gathered on the device and renumbered
    need = np.unique(dest[toks][dest[toks] >= 0])
    yh = rows_host(y, need)
    ren = np.full(rows, -1, np.int64)
    ren[need] = np.arange(len(need))
    dsub = np.where(dest[toks] >= 0, ren[np.maximum(dest[toks], 0)], -1).astype(np.int32)
    ysh = rows_host(y, offsets[E] + toks) if cfg.shared else None
    ref = O.moe_combine(yh, dsub, w.numpy()[toks], ysh)
    err = rel_err(rows_host(out, toks), ref)
    print(f"{name}: combine err {err:.3e}")
    assert err < TOL
    # fp32 in/out is accurate to fp32 rounding
    out32 = M.moe_combine(y.float(), gdest, w.to(DEV), shared, out_dtype=torch.float32)
    assert rel_err(rows_host(out32, toks), ref) < 1e-5
    del y, out, out32
    _cleanup()


def test_combine_pure_gather_is_exact():
    T, H = 300, 256
    y = synth.randn((T, H), 8, synth.STAGE, part=71, device=DEV)
    perm = torch.randperm(T, generator=torch.Generator().manual_seed(8)).to(torch.int32)
    out = M.moe_combine(y, perm[:, None].contiguous().to(DEV), torch.ones((T, 1), device=DEV), None,
                        out_dtype=torch.float32)
    assert_equal("gather", host(out), host(y)[perm.numpy()])


@pytest.mark.parametrize("act", ["bf16", "f32"])
@pytest.mark.parametrize("shared", [False, True])
def test_combine_residual(act, shared):
    """The combine on a residual branch: its layer output is bitwise moe_combine's, and
    x_next = act(residual + output) bitwise the oracle's residual rule on those same values;
    in place (x_next is the residual) gives the same bits."""
    import oracle.layer as OL
    cfg = synth.CONFIGS["prefill"]
    T, k, E, H = 777, cfg.k, cfg.E, 384
    idx = synth.routing_indices(cfg, T, seed_part=9).numpy()
    idx[3, 2] = -1
    _, offsets, dest, _ = O.moe_dispatch(idx, E, shared)
    rows = int(offsets[-1])
    dt = torch.bfloat16 if act == "bf16" else torch.float32
    y = synth.randn((rows, H), 31, synth.STAGE, part=72, device=DEV).to(dt)
    w = torch.rand((T, k), generator=torch.Generator().manual_seed(31), dtype=torch.float32).to(DEV)
    res = synth.to_act(synth.randn((T, H), 31, synth.STAGE, part=73, device=DEV) * 4, act)
    gdest = torch.from_numpy(dest).to(DEV)
    goff = torch.from_numpy(offsets).to(DEV)
    sh = goff[E:E + 1] if shared else None
    ref_out = M.moe_combine(y, gdest, w, sh)
    x_next, out = M.moe_combine_residual(y, gdest, w, sh, res, write_out=True)
    iv = torch.int16 if act == "bf16" else torch.int32
    assert torch.equal(out.view(iv), ref_out.view(iv))
    want = OL.residual_add(host(res), host(ref_out), act)
    assert_equal("x_next", host(x_next), want)
    inplace = res.clone()
    M.moe_combine_residual(y, gdest, w, sh, inplace, x_next=inplace)
    assert torch.equal(inplace.view(iv), x_next.view(iv))


def _signed_zero_tie_logits(T, E, seed):
    """Logits with exact ties, +0.0 / -0.0 mixtures (equal values, so ties by index) and a few -inf."""
    rng = np.random.default_rng(seed)
    z = rng.integers(-3, 4, size=(T, E)).astype(np.float32) * np.float32(0.5)
    zero = z == 0
    z[zero & (rng.random((T, E)) < 0.5)] = np.float32(-0.0)
    z[rng.random((T, E)) < 0.01] = -np.inf
    z[:, 0] = np.float32(7.0)   # at least one finite logit per token
    return z


@pytest.mark.parametrize("E", [64, 128, 256, 512])
@pytest.mark.parametrize("score", [0, 1])
@pytest.mark.parametrize("ng,tg,gt", [(1, 1, 2), (2, 1, 1), (4, 2, 3), (8, 4, 2), (16, 5, 2)])
def test_route_sixteen_lane_path(E, score, ng, tg, gt):
    """The 16-lanes-per-token router (E of 64..512, group limits of 2..16 groups): indices, weights
    and record bit for bit the oracle's on random logits, on tie-heavy logits with signed zeros and
    -inf, for k of 1, 8 and up to the groups' capacity; the fused launch gives the same; a
    misaligned logits view (the general path) gives the same."""
    gs = E // ng
    for k in sorted({1, 8, min(17, tg * gs), min(40, tg * gs)}):
        gcfg = M.router_cfg(E, k, score, k > 1, ng, tg, gt)
        ocfg = O.router_cfg(E, k, score, k > 1, ng, tg, gt)
        for T, kind in ((257, "rand"), (67, "ties")):
            if kind == "rand":
                z = (synth.randn((T, E), 11, synth.STAGE, part=E + k, device=DEV) * 2).cpu().numpy()
            else:
                z = _signed_zero_tie_logits(T, E, E * 100 + k)
            zd = torch.from_numpy(z).to(DEV)
            rec = torch.full((k, T + 1), -4, dtype=torch.int32, device=DEV)
            idx, w = M.moe_route(zd, gcfg, record=rec)
            orec = np.full((k, T + 1), -4, np.int32)
            oidx, ow = O.moe_route(z, ocfg, record=orec)
            tag = f"E={E} k={k} ng={ng} {kind}"
            assert_equal(f"idx {tag}", host(idx), oidx)
            assert_equal(f"w {tag}", host(w), ow)
            assert_equal(f"record {tag}", host(rec), orec)
            x = synth.randn((T, 256), 3, synth.STAGE, part=k, device=DEV).to(torch.bfloat16)
            fidx, fw, fq, fs = M.moe_route_quant(zd, gcfg, x)
            q1, s1 = M.moe_quant_fp8_block(x, 1)
            assert_equal(f"fused idx {tag}", host(fidx), oidx)
            assert_equal(f"fused w {tag}", host(fw), ow)
            assert torch.equal(fq, q1) and torch.equal(fs.view(torch.int32), s1.view(torch.int32))
            buf = torch.empty(T * E + 1, dtype=torch.float32, device=DEV)
            zm = buf[1:].view(T, E)    # 4-byte aligned only: the general path
            zm.copy_(zd)
            midx, mw = M.moe_route(zm, gcfg)
            assert_equal(f"misaligned idx {tag}", host(midx), oidx)
            assert_equal(f"misaligned w {tag}", host(mw), ow)
