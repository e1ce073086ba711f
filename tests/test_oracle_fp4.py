"""Pins of the oracle's FP4 weight format (OCP E2M1 elements in 1x32 blocks with power-of-two
scales), CPU only: the code values and hand-worked rounding cases of tests/golden/e2m1.txt, a
brute-force nearest-value search with ties to the even code on a dense grid, the block-scale
definition, the packing order, and an exact integer case of the grouped GEMM with FP4 weights."""
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e2m1.txt")


def _golden():
    vals, enc = None, []
    for line in open(GOLDEN):
        line = line.strip()
        if line.startswith("values"):
            vals = [float(t) for t in line.split()[1:]]
        elif line.startswith("encode"):
            enc = [(float(a), int(b)) for a, b in (t.split(":") for t in line.split()[1:])]
    return vals, enc


def test_e2m1_values_and_worked_cases():
    vals, enc = _golden()
    tab = O.e2m1_table()
    assert np.array_equal(tab, np.array(vals))
    assert np.signbit(tab[8]) and not np.signbit(tab[0])
    for v, code in enc:
        assert int(O.e2m1_encode(np.array([v], np.float32))[0]) == code, (v, code)


def test_e2m1_encode_brute_force():
    tab = O.e2m1_table()
    grid = np.concatenate([np.arange(-8 * 256, 8 * 256 + 1) / 256.0,
                           np.random.default_rng(1).uniform(-7, 7, 20000)]).astype(np.float32)
    got = O.e2m1_encode(grid)
    for v, c in zip(grid.tolist(), got.tolist()):
        cand = range(8, 16) if (np.signbit(np.float32(v))) else range(0, 8)
        a = min(abs(v), 6.0)
        d = [abs(abs(tab[k]) - a) for k in cand]
        best = min(d)
        ties = [k for k, dk in zip(cand, d) if dk == best]
        want = next(k for k in ties if k % 2 == 0) if len(ties) > 1 else ties[0]
        assert c == want, (v, c, want)


def test_fp4_scale_definition():
    rng = np.random.default_rng(2)
    for amax in np.concatenate([rng.uniform(1e-6, 1e3, 2000), [6.0, 3.0, 12.0, 1e-40, 0.0]]).astype(np.float32):
        s = O.fp4_scale(float(amax))
        if amax == 0:
            assert s == 1.0
            continue
        m, e = np.frexp(s)
        assert m == 0.5                                  # a power of two
        t = np.float32(amax) / np.float32(6.0)
        lo = 2.0 ** -127
        assert s >= t or s == lo                         # at or above amax / 6
        assert s / 2 < t or s == lo                      # and the smallest such
    assert O.fp4_scale(6.0) == 1.0 and O.fp4_scale(6.000001) == 2.0


def test_quant_mxfp4_packing_and_round_trip():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((5, 96)) * np.exp2(rng.integers(-20, 20, (5, 1)))).astype(np.float32)
    x[1, 32:64] = 0.0                                   # an all-zero block
    q, e8 = O.quant_mxfp4(x)
    assert q.shape == (5, 48) and e8.shape == (5, 3)
    tab = O.e2m1_table()
    for r in range(5):
        for b in range(3):
            blk = x[r, 32 * b:32 * b + 32]
            s = O.fp4_scale(float(np.max(np.abs(blk))))
            assert e8[r, b] == int(np.frexp(s)[1]) - 1 + 127
            codes = O.e2m1_encode((blk / np.float32(s)).astype(np.float32))
            packed = q[r, 16 * b:16 * b + 16]
            assert np.array_equal(packed & 15, codes[0::2]) and np.array_equal(packed >> 4, codes[1::2])
            # the largest element keeps at least code 5 (3): amax / s is in (3, 6]
            assert np.max(np.abs(tab[codes])) >= 3.0 or np.max(np.abs(blk)) == 0
    deq = O.dequant_mxfp4(q, e8)
    assert np.all(deq[1, 32:64] == 0)
    # error at most half the spacing of the element's binade (1/4 of its power of two, 1/4 of s in the subnormal range)
    s_full = np.repeat(np.exp2(e8.astype(np.float64) - 127), 32, axis=1)
    err = np.abs(deq - x)
    assert np.all(err <= 0.25 * np.maximum(np.exp2(np.floor(np.log2(np.maximum(np.abs(x) / s_full, 1.0)))), 1.0) * s_full + 1e-30)


def test_grouped_gemm_fp4_weights_exact_integers():
    """FP4 codes are small integers and halves; with power-of-two scales every product and sum is
    exact in fp64, so the oracle must equal the integer matmul scaled back."""
    rng = np.random.default_rng(4)
    G, N, K = 3, 64, 256
    offsets = np.array([0, 5, 5, 12], np.int32)
    rows = int(offsets[-1])
    wv = rng.choice([-6, -4, -3, -2, -1, 0, 1, 2, 3, 4, 6], size=(G, N, K)).astype(np.float32)
    wv[:, :, :32] *= 0.5                                 # a block with scale 1/2... halves stay exact
    wq = np.zeros((G, N, K // 2), np.uint8)
    we8 = np.zeros((G, N, K // 32), np.uint8)
    for g in range(G):
        wq[g], we8[g] = O.quant_mxfp4(wv[g])
    av = rng.integers(-8, 9, (rows, K)).astype(np.float32)
    aq, as_ = O.moe_quant_fp8_block(av, 1, True)
    got = O.moe_grouped_gemm_fp4w(aq, as_, offsets, wq, we8)
    for g in range(G):
        r0, r1 = offsets[g], offsets[g + 1]
        ref = O.dequant_act(aq[r0:r1], as_[r0:r1]) @ O.dequant_mxfp4(wq[g], we8[g]).T
        assert np.array_equal(got[r0:r1], ref)
        assert np.array_equal(O.dequant_mxfp4(wq[g], we8[g]), wv[g].astype(np.float64))   # exactly representable
        assert np.array_equal(got[r0:r1], av[r0:r1].astype(np.float64) @ wv[g].astype(np.float64).T)


def _fp4_layer_pair(cfg, int_weights: bool):
    """The same small layer with FP4 experts and, for int_weights, with power-of-two FP8 experts
    too.  int_weights: masters are 2^-5 times integers in {0, +-1, +-2, +-3, +-4, +-6}, which
    both formats hold exactly (FP4 with a 1x32 scale of 2^-5 or 2^-6; e4m3 with a 128x128 scale)."""
    import oracle.layer as L
    import synth
    wg, b = synth.make_gate(cfg, 0, "cpu")
    rc = O.router_cfg(cfg.E, cfg.k, O.SOFTMAX if cfg.score_fn == "softmax" else O.SIGMOID, cfg.renorm,
                      cfg.n_group, cfg.topk_group, cfg.group_score_topk)

    def master(e):
        if not int_weights:
            w1, w2 = synth.make_expert(cfg, e, 0, "cpu")
            return w1.numpy(), w2.numpy()
        rng = np.random.default_rng(100 + e)
        vals = [-6, -4, -3, -2, -1, 0, 1, 2, 3, 4, 6]
        w1 = rng.choice(vals, size=(2 * cfg.F, cfg.H)).astype(np.float32) * 2.0 ** -5
        w2 = rng.choice(vals, size=(cfg.H, cfg.F)).astype(np.float32) * 2.0 ** -5
        return w1, w2

    def mk(expert):
        return L.OracleLayer(wg=wg.numpy(), bias=None if b is None else b.numpy(), cfg=rc, shared=cfg.shared,
                             act=cfg.act, F=cfg.F, expert=expert, pow2=True)

    fp4 = mk(lambda e: L.quantize_expert_fp4(*master(e)))
    fp8 = mk(lambda e: L.quantize_expert(*master(e), pow2=True))
    return fp4, fp8, master


@pytest.mark.parametrize("name", ["tiny", "prefill_small"])
def test_fp4_layer_dispatch_equals_per_token(name):
    """The FP4-expert layer's dispatch path equals per-token evaluation with no dispatch (the same
    composition pin as for FP8 experts: the grouped FP4 GEMM and the per-expert products agree)."""
    import oracle.layer as L
    from test_oracle_layer import SMALL, x_f32
    cfg = SMALL[name]
    lay, _, _ = _fp4_layer_pair(cfg, False)
    x = x_f32(cfg)
    full = L.forward_dispatch(lay, x)
    tok = L.forward_token(lay, x)
    assert np.array_equal(full["idx"], tok["idx"])
    assert L.rel_err(full["out"], tok["out"]) < 1e-13


def test_fp4_layer_equals_fp8_layer_on_shared_values():
    """On weights both formats represent exactly, the FP4-expert layer and the power-of-two FP8
    layer hold the same expert values, so the two layers agree to fp64 rounding; a wrong E2M1
    value, nibble order, scale exponent or GEMM operand in the FP4 side would break this."""
    import oracle.layer as L
    from test_oracle_layer import SMALL, x_f32
    cfg = SMALL["decode_small"]
    l4, l8, master = _fp4_layer_pair(cfg, True)
    for e in range(3):
        w1, w2 = master(e)
        assert np.array_equal(l4.get(e).w1(), w1.astype(np.float64))
        assert np.array_equal(l8.get(e).w2(), w2.astype(np.float64))
    x = x_f32(cfg)
    a, c = L.forward_dispatch(l4, x), L.forward_dispatch(l8, x)
    assert np.array_equal(a["hq"], c["hq"]) and np.array_equal(a["hs"], c["hs"])
    assert L.rel_err(a["out"], c["out"]) < 1e-13


def test_fp4_quantisation_error_is_moderate_context_only():
    """Context, not parity: FP4 experts move the tiny layer more than FP8 experts do, but stay
    within tens of percent of the unquantised layer."""
    import oracle.layer as L
    from test_oracle_layer import SMALL, x_f32
    cfg = SMALL["tiny"]
    l4, l8, master = _fp4_layer_pair(cfg, False)
    x = x_f32(cfg)
    u = L.forward_unquantized(l4, x, master)
    e4 = L.rel_err(L.forward_dispatch(l4, x)["out"], u)
    e8 = L.rel_err(L.forward_dispatch(l8, x)["out"], u)
    print(f"fp4 layer err {e4:.3e}, fp8 pow2 layer err {e8:.3e}")
    assert e8 < e4 < 0.4
