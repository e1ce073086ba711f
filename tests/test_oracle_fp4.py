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
