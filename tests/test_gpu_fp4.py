"""FP4 expert weights on the GPU against the oracle, through the C ABI: the MX quantisation bit for
bit (codes and E8M0 scales), the grouped GEMM with packed FP4 weights exactly on integer cases for
every tile height (every product and partial sum is exact), against the oracle's fp64 product on
random weights, the SwiGLU epilogue's h codes, and the MoE layer forward with FP4 experts (the tiny
layer's every intermediate, sampled tokens of the full-size decode and prefill layers)."""
import itertools

import numpy as np
import pytest
import torch

import block_scaled_fp8_top_amd as M
import oracle as O
import oracle.layer as L
import synth
from block_scaled_fp8_top_amd.layer import MoELayer
from gpu_helpers import DEV, TOL, assert_equal, gpu_weights, host, oracle_layer, rel_err, rows_host

pytestmark = pytest.mark.gpu
TILES = [32, 48, 64, 128]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_quant_mxfp4_bit_exact(dt):
    rows, cols = 300, 2048
    x = synth.randn((rows, cols), 31, synth.STAGE, 0, 0, 81, device=DEV)
    x[0, :32] = 0                                      # an all-zero block
    x[1, 32:64] *= 1e-38                               # scales near the bottom of the E8M0 range
    x[2] *= 1e4
    x = synth.to_act(x, dt)
    q, e8 = M.moe_quant_mxfp4(x)
    rq, re8 = O.quant_mxfp4(host(x))
    assert_equal("fp4 codes", host(q), rq)
    assert_equal("fp4 scales", host(e8), re8)


def _int_fp4_weights(G, N, K, seed):
    """FP4-representable weights: integers in {0, +-1, +-2, +-3, +-4, +-6} (scale 1 where a block
    holds a 4 or 6, else the scale halves the codes' range but keeps the integers exact)."""
    rng = np.random.default_rng(seed)
    w = rng.choice([-6, -4, -3, -2, -1, 0, 1, 2, 3, 4, 6], size=(G, N, K)).astype(np.float32)
    return w


@pytest.mark.parametrize("epi", ["store"])
def test_fp4_gemm_exact_integers(epi):
    offsets = np.array([0, 130, 130, 131, 400, 657], np.int64)
    G, N, K = 5, 512, 1024
    rows = int(offsets[-1])
    wv = _int_fp4_weights(G, N, K, 7)
    w = torch.from_numpy(wv).to(DEV)
    q, e8 = M.moe_quant_mxfp4(w)
    pk = M.moe_pack_weights_fp4(q, e8, M.MOE_EPI_STORE)
    a, av = synth.integer_codes((rows, K), 61, 0, device=DEV)
    rng = np.random.default_rng(5)
    as_ = torch.from_numpy(np.exp2(rng.integers(-1, 2, (rows, K // 128))).astype(np.float32)).to(DEV)
    goff = torch.from_numpy(offsets.astype(np.int32)).to(DEV)
    ref = O.moe_grouped_gemm_fp4w(host(a), host(as_), offsets, host(q), host(e8))
    # the oracle itself is exact here: integer activations times integer weights
    grp = np.repeat(np.arange(G), np.diff(offsets))
    exact = np.stack([((av[r].double() * torch.from_numpy(host(as_)[r]).double().repeat_interleave(128)).numpy()
                       @ wv[grp[r]].astype(np.float64).T) for r in range(rows)])
    assert np.array_equal(ref, exact)
    for tile in TILES:
        y = M.moe_grouped_gemm_fp8(a, as_, goff, pk, None, M.MOE_EPI_STORE, torch.float32, tile_rows=tile, pow2=True)
        assert_equal(f"fp4 exact integers tile {tile}", host(y), ref.astype(np.float32))


@pytest.mark.parametrize("name,tile", [(n, t) for n in ("decode", "prefill") for t in (48, 128)])
def test_fp4_gemm_random(name, tile):
    cfg = synth.CONFIGS[name]
    G, N, K = 6, 2 * cfg.F, cfg.H
    counts = np.array([0, 70, 1, 300, 129, 33])
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    rows = int(offsets[-1])
    w = synth.randn((G, N, K), 33, synth.STAGE, 0, 0, 82, device=DEV, std=1.0 / np.sqrt(K))
    q, e8 = M.moe_quant_mxfp4(w)
    del w
    x = synth.randn((rows, K), 33, synth.STAGE, 0, 0, 83, device=DEV)
    a, as_ = M.moe_quant_fp8_block(x, 1, pow2=True)
    goff = torch.from_numpy(offsets.astype(np.int32)).to(DEV)
    y = M.moe_grouped_gemm_fp8(a, as_, goff, M.moe_pack_weights_fp4(q, e8, M.MOE_EPI_STORE), None, M.MOE_EPI_STORE,
                               torch.float32, tile_rows=tile, pow2=True)
    ref = O.moe_grouped_gemm_fp4w(host(a), host(as_), offsets, host(q), host(e8))
    # exact products, fp32 accumulation over K: ~1e-6 of the largest output
    assert rel_err(host(y), ref) < 1e-4
    # SwiGLU epilogue: h codes against the oracle's quantisation of swiglu(ref)
    hq, hs = M.moe_grouped_gemm_fp8(a, as_, goff, M.moe_pack_weights_fp4(q, e8, M.MOE_EPI_SWIGLU_QUANT), None,
                                    M.MOE_EPI_SWIGLU_QUANT, tile_rows=tile, pow2=True)
    h = O.swiglu(ref, N // 2)
    rq, rs = O.moe_quant_fp8_block(h, 1, pow2=True)
    gq, gs = host(hq), host(hs)
    ratio = gs / rs
    assert np.all((ratio == 1) | (ratio == 2) | (ratio == 0.5)) and np.mean(ratio != 1) < 1e-2
    tab = O.e4m3_table()
    same = np.repeat(ratio == 1, 128, 1)
    dg, dr = tab[gq] * np.repeat(gs, 128, 1), tab[rq] * np.repeat(rs, 128, 1)
    step = np.abs(dr) / 8 + np.repeat(rs, 128, 1) * (2.0 ** -9 + 448 * 1e-3)
    assert np.all(np.abs(dg - dr)[same] <= step[same] * 1.0001)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_fp4_layer_tiny_every_intermediate():
    cfg = synth.CONFIGS["tiny"]
    gw = gpu_weights(cfg, fp4=True)
    lay = MoELayer(gw, cfg.T, torch.float32)
    x = synth.make_x(cfg, DEV)
    out = lay.forward(x)
    ol = oracle_layer(cfg, fp4=True)
    r = L.forward_dispatch(ol, host(x))
    assert_equal("idx", host(lay.idx), r["idx"])
    assert_equal("xq", host(lay.xq), r["xq"])
    assert_equal("xs", host(lay.xs), r["xs"])
    n = int(r["offsets"][-1])
    # the rows GEMM1 reads: xq gathered through src_token (the layer keeps no permuted copy)
    assert_equal("gathered rows", host(lay.xq)[host(lay.disp.src_token)[:n]], r["aq"])
    assert rel_err(host(lay.y)[:n], r["y_act"]) < TOL
    err = rel_err(host(out), r["out"])
    print(f"tiny fp4 layer output err {err:.3e}")
    assert err < TOL
    with pytest.raises(ValueError):
        lay.forward(x, training=True)


@pytest.mark.parametrize("name,samples", [("decode", 32), ("prefill", 4)])
def test_fp4_layer_sampled(name, samples):
    cfg = synth.CONFIGS[name]
    gw = gpu_weights(cfg, fp4=True)
    act = torch.bfloat16 if cfg.act == "bf16" else torch.float32
    lay = MoELayer(gw, cfg.T, act)
    x = synth.make_x(cfg, DEV)
    out = lay.forward(x)
    torch.cuda.synchronize()
    toks = synth.sample_tokens(cfg.T, samples, cfg.seed)
    ol = oracle_layer(cfg, fp4=True)
    r = L.forward_sampled(ol, rows_host(x, toks))
    assert_equal("idx", rows_host(lay.idx, toks), r["idx"])
    assert_equal("xq", rows_host(lay.xq, toks), r["xq"])
    err = rel_err(rows_host(out, toks), r["out"])
    print(f"{name} fp4 layer output err {err:.3e}")
    assert err < TOL
    del lay, gw, x, out
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
