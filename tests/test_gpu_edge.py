"""Degenerate cases of the forward path on the GPU, through the C ABI, against the oracle: an empty
batch through every stage and through the layer, a grouped GEMM whose groups are all empty (it must
write nothing), one-token layers, and a replay whose payload holds bad expert ids for some tokens
(their slots go to no expert: index -1, weight 0; a shared expert still contributes)."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import block_scaled_fp8_top_amd as M
import oracle.layer as L
import synth
from block_scaled_fp8_top_amd.layer import MoELayer
from gpu_helpers import DEV, TOL, assert_equal, cfgs_for, gpu_weights, host, oracle_layer, rel_err

pytestmark = pytest.mark.gpu


def test_empty_batch_every_stage_and_layer():
    cfg = synth.CONFIGS["decode"]
    gcfg, _ = cfgs_for(cfg)
    H, E, k = cfg.H, cfg.E, cfg.k
    x = torch.empty((0, H), dtype=torch.bfloat16, device=DEV)
    wg = synth.randn((E, H), 9, synth.STAGE, part=1, device=DEV, std=0.02)
    z = M.moe_gate_logits(x, wg)
    assert z.shape == (0, E)
    payload = torch.zeros((k, 4), dtype=torch.int32, device=DEV)
    idx, w = M.moe_route(z, gcfg, record=payload[:, :0])
    assert idx.shape == (0, k) and w.shape == (0, k)
    bad = torch.zeros(1, dtype=torch.int32, device=DEV)
    ridx, rw = M.moe_replay_route(z, gcfg, payload[:, :0], bad_count=bad)
    assert ridx.shape == (0, k) and int(bad.item()) == 0
    for pow2 in (False, True):
        xq, xs = M.moe_quant_fp8_block(x, 1, pow2=pow2)
        assert xq.shape == (0, H) and xs.shape == (0, H // 128)
    for shared in (False, True):
        d = M.moe_dispatch(idx, E, shared, xq, xs)
        assert np.all(host(d.counts) == 0) and np.all(host(d.offsets) == 0)
        assert d.aq.shape[0] == 0
    out = M.moe_combine(torch.empty((0, H), dtype=torch.bfloat16, device=DEV), idx, w)
    assert out.shape == (0, H)
    # the whole layer at T = 0 (nothing to route, no rows, no GEMM work)
    gw = gpu_weights(synth.CONFIGS["tiny"])
    lay = MoELayer(gw, 0, torch.float32)
    y = lay.forward(torch.empty((0, gw.H), dtype=torch.float32, device=DEV))
    torch.cuda.synchronize()
    assert y.shape == (0, gw.H)


@pytest.mark.parametrize("epi", [M.MOE_EPI_STORE, M.MOE_EPI_SWIGLU_QUANT])
@pytest.mark.parametrize("pow2", [False, True])
def test_gemm_all_groups_empty_writes_nothing(epi, pow2):
    """max_rows > 0 but every group empty: the plan has no tiles and no output byte changes."""
    G, N, K, rows = 5, 512, 256, 96
    b = torch.randint(0, 0x7E, (G, N, K), dtype=torch.uint8, device=DEV)
    bs = torch.ones((G, N // 128, K // 128), dtype=torch.float32, device=DEV)
    a = torch.randint(0, 0x7E, (rows, K), dtype=torch.uint8, device=DEV)
    as_ = torch.ones((rows, K // 128), dtype=torch.float32, device=DEV)
    offsets = torch.zeros(G + 1, dtype=torch.int32, device=DEV)
    pk = M.moe_pack_weights_fp8(b, epi)
    for tile in (32, 48, 64, 128):
        if epi == M.MOE_EPI_STORE:
            out = torch.full((rows, N), 7.0, dtype=torch.float32, device=DEV)
            M.moe_grouped_gemm_fp8(a, as_, offsets, pk, bs, epi, torch.float32, out=out, tile_rows=tile, pow2=pow2)
            torch.cuda.synchronize()
            assert np.all(host(out) == 7.0), f"tile {tile}: rows written"
        else:
            hq = torch.full((rows, N // 2), 0x55, dtype=torch.uint8, device=DEV)
            hs = torch.full((rows, N // 256), 3.0, dtype=torch.float32, device=DEV)
            M.moe_grouped_gemm_fp8(a, as_, offsets, pk, bs, epi, out=hq, out_scales=hs, tile_rows=tile, pow2=pow2)
            torch.cuda.synchronize()
            assert np.all(host(hq) == 0x55) and np.all(host(hs) == 3.0), f"tile {tile}: rows written"


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill"])
def test_layer_single_token(name):
    """T = 1: k rows (plus the shared row) spread over k different experts, every other group empty."""
    cfg = synth.CONFIGS[name]
    gw = gpu_weights(cfg)
    act = torch.bfloat16 if cfg.act == "bf16" else torch.float32
    lay = MoELayer(gw, 1, act)
    x = synth.make_x(cfg, DEV)[3:4].contiguous()
    out = lay.forward(x)
    torch.cuda.synchronize()
    ol = oracle_layer(cfg)
    # the tiny layer through the dispatch path; the large ones per token (only the used experts)
    r = L.forward_dispatch(ol, host(x)) if name == "tiny" else L.forward_sampled(ol, host(x))
    assert_equal("idx", host(lay.idx), r["idx"])
    want = np.bincount(r["idx"].reshape(-1), minlength=cfg.E)
    if cfg.shared:
        want = np.concatenate([want, [1]])
    assert_equal("counts", host(lay.disp.counts), want)
    err = rel_err(host(out), r["out"])
    print(f"{name} one-token layer err {err:.3e}")
    assert err < TOL
    del lay, gw
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["tiny", "prefill_small"])
def test_layer_replay_with_bad_ids(name):
    """Replayed payload with an out-of-range id, a negative id and a repeated id in three tokens:
    those tokens' slots go to no expert (counted once each), the rest replays normally."""
    if name == "prefill_small":
        cfg = replace(synth.CONFIGS["prefill"], name="prefill_small", T=96, H=256, E=32, F=256, k=8)
    else:
        cfg = synth.CONFIGS[name]
    gw = gpu_weights(cfg)
    lay = MoELayer(gw, cfg.T, torch.bfloat16 if cfg.act == "bf16" else torch.float32)
    x = synth.make_x(cfg, DEV)
    payload = torch.zeros((cfg.k, cfg.T), dtype=torch.int32, device=DEV)
    lay.forward(x, record=payload)
    pay = host(payload).copy()
    pay[0, 1] = cfg.E + 3
    pay[min(1, cfg.k - 1), cfg.T // 2] = -2
    pay[cfg.k - 1, cfg.T - 1] = pay[0, cfg.T - 1]
    gpay = torch.from_numpy(pay).to(DEV)
    if cfg.score_fn == "sigmoid":
        # the fused replay gate drops the same tokens, bit for bit
        lay.bad.zero_()
        fused = lay.forward(x, replay=gpay).clone()
        fidx, fw, fbad = host(lay.idx), host(lay.wts), int(lay.bad.item())
    lay.bad.zero_()
    out = lay.forward(x, replay=gpay, fused_replay=False)
    torch.cuda.synchronize()
    if cfg.score_fn == "sigmoid":
        assert fbad == 3 and np.array_equal(fidx, host(lay.idx))
        assert np.array_equal(fw.view(np.uint32), host(lay.wts).view(np.uint32))
        assert np.array_equal(host(fused), host(out))
    ol = oracle_layer(cfg)
    r = L.forward_dispatch(ol, host(x), replay=pay)
    assert r["bad"] == 3 and int(lay.bad.item()) == 3
    assert_equal("idx", host(lay.idx), r["idx"])
    assert_equal("w", host(lay.wts).view(np.uint32), r["w"].view(np.uint32))
    assert_equal("counts", host(lay.disp.counts), r["counts"])
    err = rel_err(host(out), r["out"])
    print(f"{name} replay with bad ids err {err:.3e}")
    assert err < TOL
    # the bad tokens: no routed contribution (only the shared expert's row, if any)
    if not cfg.shared:
        for t in (1, cfg.T // 2, cfg.T - 1):
            assert np.all(host(out)[t] == 0)


def test_dispatch_rejects_missized_outputs():
    """Caller-provided dispatch outputs are checked against the extents the kernels write, before
    any launch (a short src_token or a wrong counts length would otherwise be written past)."""
    T, k, E, H = 16, 2, 8, 256
    idx = torch.randint(0, E, (T, k), dtype=torch.int32, device=DEV)
    xq = torch.zeros((T, H), dtype=torch.uint8, device=DEV)
    xs = torch.ones((T, H // 128), dtype=torch.float32, device=DEV)
    good = M.moe_dispatch(idx, E, False, xq, xs)
    ws = torch.empty(M.workspace_bytes(M.MOE_OP_DISPATCH, T, k, E), dtype=torch.uint8, device=DEV)
    gws = torch.empty(M.workspace_bytes(M.MOE_OP_GROUPED_GEMM, T * k, 0, E, 0, 0), dtype=torch.uint8, device=DEV)
    for field, bad in (("counts", torch.empty(E - 1, dtype=torch.int32, device=DEV)),
                       ("src_token", torch.empty(T * k - 1, dtype=torch.int32, device=DEV)),
                       ("as_", torch.empty((T * k, 1), dtype=torch.float32, device=DEV))):
        out = replace(good, **{field: bad})
        with pytest.raises(ValueError):
            M.moe_dispatch(idx, E, False, xq, xs, out=out)
        with pytest.raises(ValueError):
            M.moe_dispatch_plan(idx, E, False, xq, xs, ws, out, gws)
