"""Power-of-two block scales on the GPU (the form gfx950's matrix cores apply as E8M0 exponents),
through the C-ABI, against the oracle in the same mode: quantisation bit-exact, GEMM outputs within
the tolerance, exact-integer GEMMs bitwise, the SwiGLU epilogue's power-of-two h scales, and the
whole layer."""
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


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _is_pow2(s: np.ndarray) -> bool:
    bits = np.asarray(s, np.float32).view(np.uint32)
    e, m = (bits >> 23) & 0xFF, bits & 0x7FFFFF
    return bool(np.all(np.where(e == 0, (m != 0) & ((m & (m - 1)) == 0), m == 0)))


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill"])
def test_pow2_quant_activations_and_weights(name):
    cfg = synth.CONFIGS[name]
    x = synth.make_x(cfg, DEV)
    x[0, :128] = 0                                   # an all-zero block
    x[1, 128:256] *= 1e-38                            # scales near the bottom of the E8M0 range
    q, s = M.moe_quant_fp8_block(x, 1, pow2=True)
    rq, rs = O.moe_quant_fp8_block(host(x), 1, pow2=True)
    assert_equal("codes", host(q), rq)
    assert_equal("scales", host(s), rs)
    assert _is_pow2(host(s))
    w1, w2 = synth.make_expert(cfg, 0, 0, DEV)
    for w in (w1, w2.to(torch.bfloat16)):
        q, s = M.moe_quant_fp8_block(w, 128, pow2=True)
        rq, rs = O.moe_quant_fp8_block(host(w), 128, pow2=True)
        assert_equal("W codes", host(q), rq)
        assert_equal("W scales", host(s), rs)
    del x, q, s, w1, w2
    _free()


def _case(cfg, which, part):
    """Random codes, power-of-two scales, the workload's group sizes."""
    G = cfg.groups
    N, K = (2 * cfg.F, cfg.H) if which == "w1" else (cfg.H, cfg.F)
    idx = synth.routing_indices(cfg, cfg.T, seed_part=part).numpy()
    _, offsets, _, _ = O.moe_dispatch(idx, cfg.E, cfg.shared)
    rows = int(offsets[-1])
    a = synth.random_codes((rows, K), cfg.seed, 70 + part, device=DEV)
    as_ = torch.exp2(torch.round(torch.log2(
        synth.random_scales((rows, K // 128), cfg.seed, 71 + part, device=DEV, lo=2.0 ** -10, hi=2.0 ** -6))))
    b = synth.random_codes((G, N, K), cfg.seed, 72 + part, device=DEV)
    bs = torch.exp2(torch.round(torch.log2(
        synth.random_scales((G, N // 128, K // 128), cfg.seed, 73 + part, device=DEV, lo=2.0 ** -10, hi=2.0 ** -6))))
    return offsets, a, as_, b, bs, N, K


def _rows(offsets, n, seed):
    nonempty = [g for g in range(len(offsets) - 1) if offsets[g + 1] > offsets[g]]
    rng = np.random.default_rng(seed)
    pick = set()
    for g in rng.choice(nonempty, size=min(6, len(nonempty)), replace=False):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        pick |= {lo, hi - 1} | {min(lo + d, hi - 1) for d in (31, 32, 47, 48, 127, 128)}
    pick |= set(synth.sample_tokens(int(offsets[-1]), n, seed).tolist())
    return np.array(sorted(pick))


def _ref_rows(a, as_, offsets, b, bs, rows):
    grp = np.searchsorted(offsets, rows, side="right") - 1
    a_h, as_h = rows_host(a, rows), rows_host(as_, rows)
    out = np.zeros((len(rows), b.shape[1]))
    for g in np.unique(grp):
        sel = np.nonzero(grp == g)[0]
        out[sel] = O.dequant_act(a_h[sel], as_h[sel]) @ O.dequant_weight(host(b[g]), host(bs[g])).T
    return out


@pytest.mark.parametrize("name,which,tile", [(n, w, t) for n in ("tiny", "decode", "prefill") for w in ("w1", "w2")
                                             for t in TILES])
def test_pow2_gemm_store(name, which, tile):
    cfg = synth.CONFIGS[name]
    offsets, a, as_, b, bs, N, K = _case(cfg, which, 0 if which == "w1" else 5)
    goff = torch.from_numpy(offsets).to(DEV)
    rows = _rows(offsets, 24, cfg.seed)
    ref = _ref_rows(a, as_, offsets, b, bs, rows)
    for bw in (b, M.moe_pack_weights_fp8(b, M.MOE_EPI_STORE)):
        y = M.moe_grouped_gemm_fp8(a, as_, goff, bw, bs, M.MOE_EPI_STORE, torch.float32, tile_rows=tile, pow2=True)
        err = rel_err(rows_host(y, rows), ref)
        assert err < 1e-3, (name, which, tile, type(bw).__name__, err)
    del a, as_, b, bs
    _free()


def test_pow2_gemm_exact_integers():
    """Integer codes with power-of-two scales: every sum is an exact fp32 value in any order, so the
    hardware-scaled accumulation equals the oracle bitwise, for every tile height and layout."""
    offsets = np.array([0, 130, 130, 131, 400, 657], np.int64)
    G, N, K = 5, 384, 1024
    rows = int(offsets[-1])
    a, _ = synth.integer_codes((rows, K), 61, 0, device=DEV)
    b, _ = synth.integer_codes((G, N, K), 61, 1, device=DEV)
    goff = torch.from_numpy(offsets.astype(np.int32)).to(DEV)
    rng = np.random.default_rng(4)
    # per-row activation scales in {1/2, 1, 2} and per-block weight scales in {1, 2}: products of
    # codes in [-8, 8] summed over K = 1024 need 17 bits, the scale exponents span 3 more, so every
    # partial sum is exact in fp32 and the result cannot depend on the summation order
    as_ = torch.from_numpy(np.exp2(rng.integers(-1, 2, (rows, K // 128))).astype(np.float32)).to(DEV)
    bs = torch.from_numpy(np.exp2(rng.integers(0, 2, (G, N // 128, K // 128))).astype(np.float32)).to(DEV)
    ref = O.moe_grouped_gemm_fp8(host(a), host(as_), offsets, host(b), host(bs))
    for tile, bw in itertools.product(TILES, (b, M.moe_pack_weights_fp8(b, M.MOE_EPI_STORE))):
        y = M.moe_grouped_gemm_fp8(a, as_, goff, bw, bs, M.MOE_EPI_STORE, torch.float32, tile_rows=tile, pow2=True)
        assert_equal(f"pow2 exact integers tile {tile} {type(bw).__name__}", host(y), ref.astype(np.float32))


@pytest.mark.parametrize("name,tile", [(n, t) for n in ("tiny", "decode", "prefill") for t in TILES])
def test_pow2_gemm_swiglu_quant(name, tile):
    """h scales are powers of two and equal the oracle's except where GEMM1's last bits move a row
    block's amax / 448 across a power of two (then they differ by exactly 2x); codes agree to one
    e4m3 step where the scales agree."""
    cfg = synth.CONFIGS[name]
    offsets, a, as_, b, bs, N, K = _case(cfg, "w1", 9)
    F = N // 2
    goff = torch.from_numpy(offsets).to(DEV)
    hq, hs = M.moe_grouped_gemm_fp8(a, as_, goff, M.moe_pack_weights_fp8(b, M.MOE_EPI_SWIGLU_QUANT), bs,
                                    M.MOE_EPI_SWIGLU_QUANT, tile_rows=tile, pow2=True)
    rows = _rows(offsets, 16, cfg.seed + 1)
    h = O.swiglu(_ref_rows(a, as_, offsets, b, bs, rows), F)
    rq, rs = O.moe_quant_fp8_block(h, 1, pow2=True)
    gq, gs = rows_host(hq, rows), rows_host(hs, rows)
    assert _is_pow2(gs)
    ratio = gs / rs
    assert np.all((ratio == 1) | (ratio == 2) | (ratio == 0.5))
    assert np.mean(ratio != 1) < 1e-2
    tab = O.e4m3_table()
    same = np.repeat(ratio == 1, 128, 1)
    dg = tab[gq] * np.repeat(gs, 128, 1)
    dr = tab[rq] * np.repeat(rs, 128, 1)
    step = np.abs(dr) / 8 + np.repeat(rs, 128, 1) * (2.0 ** -9 + 448 * 1e-3)
    assert np.all(np.abs(dg - dr)[same] <= step[same] * 1.0001)
    del a, as_, b, bs, hq, hs
    _free()


def test_pow2_layer_tiny_every_intermediate():
    cfg = synth.CONFIGS["tiny"]
    gw = gpu_weights(cfg, pow2=True)
    lay = MoELayer(gw, cfg.T, torch.float32)
    x = synth.make_x(cfg, DEV)
    out = lay.forward(x)
    ol = oracle_layer(cfg, pow2=True)
    r = L.forward_dispatch(ol, host(x))
    for g in range(cfg.groups):
        ew = ol.get(g)
        assert_equal(f"w1q[{g}]", host(gw.w1q[g]), ew.w1q)
        assert_equal(f"w2s[{g}]", host(gw.w2s[g]), ew.w2s)
    assert_equal("xq", host(lay.xq), r["xq"])
    assert_equal("xs", host(lay.xs), r["xs"])
    n = int(r["offsets"][-1])
    # the rows GEMM1 reads: xq gathered through src_token (the layer keeps no permuted copy)
    assert_equal("gathered rows", host(lay.xq)[host(lay.disp.src_token)[:n]], r["aq"])
    assert rel_err(host(lay.y)[:n], r["y_act"]) < TOL
    err = rel_err(host(out), r["out"])
    print(f"tiny pow2 layer output err {err:.3e}")
    assert err < TOL


@pytest.mark.parametrize("name,samples", [("decode", 32), ("prefill", 4)])
def test_pow2_layer_sampled(name, samples):
    cfg = synth.CONFIGS[name]
    gw = gpu_weights(cfg, pow2=True)
    act = torch.bfloat16 if cfg.act == "bf16" else torch.float32
    lay = MoELayer(gw, cfg.T, act)
    x = synth.make_x(cfg, DEV)
    out = lay.forward(x)
    torch.cuda.synchronize()
    toks = synth.sample_tokens(cfg.T, samples, cfg.seed)
    ol = oracle_layer(cfg, pow2=True)
    r = L.forward_sampled(ol, rows_host(x, toks))
    assert_equal("idx", rows_host(lay.idx, toks), r["idx"])
    assert_equal("xq", rows_host(lay.xq, toks), r["xq"])
    assert_equal("xs", rows_host(lay.xs, toks), r["xs"])
    err = rel_err(rows_host(out, toks), r["out"])
    print(f"{name} pow2 layer output err {err:.3e}")
    assert err < TOL
    del lay, gw, x, out
    _free()
