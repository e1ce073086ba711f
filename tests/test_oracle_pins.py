"""Pins of the CPU oracle against things other than itself (CPU only).

Each test ties one oracle step to the format definition, a library routine, a closed form, an
invariant or brute force, chosen so that a plausible mistake (dropped term, wrong sign or index,
transposed operand, wrong rounding) fails at least one of them.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")
U = 2.0 ** -24  # fp32 unit roundoff


# ----------------------------------------------------------------------------- FP8 e4m3
def _format_value(code: int) -> float:
    """e4m3fn value from the bit fields, written independently of the oracle."""
    s, e, m = (code >> 7) & 1, (code >> 3) & 0xF, code & 7
    if e == 0xF and m == 7:
        return float("nan")
    mag = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -mag if s else mag


def test_e4m3_decode_table_matches_format_and_torch():
    tab = O.e4m3_table()
    fmt = np.array([_format_value(c) for c in range(256)])
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(tab), np.isnan(fmt))
    assert np.isnan(tab[0x7F]) and np.isnan(tab[0xFF]) and np.isnan(tab).sum() == 2
    ok = ~np.isnan(fmt)
    assert np.array_equal(tab[ok], fmt[ok]) and np.array_equal(tab[ok], lib[ok])
    assert tab[0x7E] == 448.0 and tab[0x01] == 2.0 ** -9 and tab[0x08] == 2.0 ** -6


def test_e4m3_encode_golden_cases():
    rows = [l.split() for l in open(os.path.join(GOLD, "e4m3_encode.txt")) if l.strip() and not l.startswith("#")]
    vals = np.array([float(r[0]) for r in rows], np.float32)
    want = np.array([int(r[1], 16) for r in rows], np.uint8)
    got = O.e4m3_encode(vals)
    assert np.array_equal(got, want), [(v, hex(g), hex(w)) for v, g, w in zip(vals, got, want) if g != w]


@pytest.mark.slow
def test_e4m3_encode_exhaustive_vs_torch_cast():
    """Every non-negative fp32 up to 448 (1.14e9 values) and a strided sweep of negatives
    against torch's float8_e4m3fn cast (round to nearest even; agrees with saturation there)."""
    hi = 0x43E00000  # 448.0
    step = 1 << 26
    for start in range(0, hi + 1, step):
        stop = min(hi + 1, start + step)
        v = np.arange(start, stop, dtype=np.uint32).view(np.float32)
        got = O.e4m3_encode(v)
        ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(got, ref), f"mismatch in bit range [{start:#x},{stop:#x})"
    neg = np.arange(0x80000000, 0x80000000 + hi + 1, 4099, dtype=np.uint64).astype(np.uint32).view(np.float32)
    assert np.array_equal(O.e4m3_encode(neg), torch.from_numpy(neg).to(torch.float8_e4m3fn).view(torch.uint8).numpy())


def test_e4m3_encode_saturates_and_keeps_sign():
    v = np.array([464.0, 465.0, 480.0, 1e30, -465.0, -1e30, -0.0, 0.0, -1e-30], np.float32)
    assert O.e4m3_encode(v).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x80, 0x00, 0x80]


def test_e4m3_encode_is_nearest():
    """Random fp32 in range: the chosen code is a nearest finite value (brute force)."""
    rng = np.random.default_rng(0)
    v = (rng.standard_normal(20000) * rng.choice([1e-3, 1e-1, 10, 100], 20000)).astype(np.float32)
    v = np.clip(v, -448, 448)
    codes = O.e4m3_encode(v)
    tab = np.array([_format_value(c) for c in range(256)])
    fin = np.where(~np.isnan(tab))[0]
    d = np.abs(v.astype(np.float64)[:, None] - tab[fin][None, :])
    best = d.min(1)
    assert np.all(np.abs(v.astype(np.float64) - tab[codes]) == best)


# ----------------------------------------------------------------------------- pinned exp
def test_pinned_exp_accuracy_and_special_values():
    x = np.linspace(-86.0, 88.0, 2_000_001).astype(np.float32)
    got = O.pinned_exp(x).astype(np.float64)
    ref = np.exp(x.astype(np.float64))
    ulp = np.spacing(ref.astype(np.float32)).astype(np.float64)
    assert np.max(np.abs(got - ref) / ulp) < 3.0
    assert O.pinned_exp(np.array([0.0], np.float32))[0] == 1.0
    assert O.pinned_exp(np.array([1.0], np.float32))[0] == np.float32(math.e)
    assert np.all(np.isfinite(O.pinned_exp(np.array([-1e30, 1e30, -87, 89], np.float32))))
    assert O.pinned_sigmoid(np.array([0.0], np.float32))[0] == 0.5
    s = O.pinned_sigmoid(np.linspace(-30, 30, 100001).astype(np.float32)).astype(np.float64)
    r = 1.0 / (1.0 + np.exp(-np.linspace(-30, 30, 100001).astype(np.float32).astype(np.float64)))
    # exp within 3 ulp, then one add and one division: a few units of fp32 roundoff
    assert np.max(np.abs(s - r) / r) < 8 * U


# ----------------------------------------------------------------------------- gate logits
def test_gate_logits_within_rounding_bound():
    rng = np.random.default_rng(1)
    T, H, E = 17, 1000, 9
    x = rng.standard_normal((T, H)).astype(np.float32)
    wg = (rng.standard_normal((E, H)) * 0.03).astype(np.float32)
    b = rng.standard_normal(E).astype(np.float32)
    z = O.moe_gate_logits(x, wg, b).astype(np.float64)
    xd, wd = x.astype(np.float64), wg.astype(np.float64)
    ref = xd @ wd.T + b.astype(np.float64)
    gam = H * U / (1 - H * U)
    bound = gam * (np.abs(xd) @ np.abs(wd).T) + 2 * U * (np.abs(ref) + np.abs(b))
    assert np.all(np.abs(z - ref) <= bound)


def test_gate_logits_exact_on_integers_and_orientation():
    rng = np.random.default_rng(2)
    T, H, E = 5, 300, 7
    x = rng.integers(-20, 21, (T, H))
    w = rng.integers(-20, 21, (E, H))
    z = O.moe_gate_logits(x.astype(np.float32), w.astype(np.float32))
    assert np.array_equal(z.astype(np.int64), x @ w.T)
    # bias enters once per logit
    z2 = O.moe_gate_logits(x.astype(np.float32), w.astype(np.float32), np.arange(E, dtype=np.float32))
    assert np.array_equal(z2.astype(np.int64), x @ w.T + np.arange(E))


def test_gate_logits_fixed_chain_order():
    """The logit is the ascending-h chain: with x = [1e8, 1, -1e8, 1] and w = 1 the chain gives
    ((1e8 + 1 -> 1e8) - 1e8) + 1 = 1, while a reversed or pairwise order gives 0."""
    x = np.array([[1e8, 1.0, -1e8, 1.0]], np.float32)
    w = np.array([[1.0, 1.0, 1.0, 1.0]], np.float32)
    # ascending chain: ((1e8 + 1) -> 1e8) - 1e8 = 0, + 1 = 1 ; a different order would give 2 or 0
    assert O.moe_gate_logits(x, w)[0, 0] == 1.0


# ----------------------------------------------------------------------------- router
def _cases():
    for line in open(os.path.join(GOLD, "router_cases.txt")):
        if not line.strip() or line.startswith("#"):
            continue
        d = dict(kv.split("=") for kv in line.split())
        yield d


@pytest.mark.parametrize("case", list(_cases()), ids=lambda d: d["name"])
def test_router_golden(case):
    z = np.array([float(v) for v in case["z"].split(",")], np.float32)[None]
    cfg = O.router_cfg(len(z[0]), int(case["k"]), O.SOFTMAX if case["score"] == "softmax" else O.SIGMOID,
                       int(case["renorm"]), int(case["n_group"]), int(case["topk_group"]), 2)
    idx, w = O.moe_route(z, cfg)
    assert idx[0].tolist() == [int(v) for v in case["idx"].split(",")]
    np.testing.assert_allclose(w[0], [float(v) for v in case["w"].split(",")], rtol=1e-6)


@pytest.mark.parametrize("score,renorm", [("softmax", False), ("softmax", True), ("sigmoid", True), ("sigmoid", False)])
def test_router_matches_torch_on_distinct_keys(score, renorm):
    T, E, k = 300, 64, 6
    z = synth.randn((T, E), 11, synth.STAGE, part=7) * 2.0
    cfg = O.router_cfg(E, k, O.SOFTMAX if score == "softmax" else O.SIGMOID, renorm)
    idx, w = O.moe_route(z.numpy(), cfg)
    tv, ti = torch.topk(z.double(), k, dim=1)
    assert np.array_equal(idx, ti.numpy())
    sc = torch.softmax(z.double(), 1) if score == "softmax" else torch.sigmoid(z.double())
    ref = torch.gather(sc, 1, ti)
    if renorm:
        ref = ref / ref.sum(1, keepdim=True)
    # the un-renormalised softmax carries the rounding of a 64-term fp32 denominator
    np.testing.assert_allclose(w, ref.numpy(), rtol=1e-6 if (renorm or score == "sigmoid") else 5e-6, atol=0)


def _brute_grouped(z, E, k, n_group, topk_group, gtop):
    """Group-limited top-k by exhaustive rules, in fp64 for scores (distinct keys assumed)."""
    T = z.shape[0]
    gs = E // n_group
    s = 1.0 / (1.0 + np.exp(-z.astype(np.float64)))
    out = np.empty((T, k), np.int64)
    for t in range(T):
        gsc = []
        for g in range(n_group):
            zz = z[t, g * gs:(g + 1) * gs]
            top = np.argsort(-zz, kind="stable")[:gtop]
            gsc.append(s[t, g * gs + top].sum())
        keep = np.argsort(-np.array(gsc), kind="stable")[:topk_group]
        allowed = np.concatenate([np.arange(g * gs, (g + 1) * gs) for g in sorted(keep)])
        order = allowed[np.argsort(-z[t, allowed], kind="stable")]
        out[t] = order[:k]
    return out


@pytest.mark.parametrize("gtop", [1, 2])
def test_router_group_limited_brute_force(gtop):
    T, E, k = 200, 64, 6
    z = (synth.randn((T, E), 12, synth.STAGE, part=8) * 1.5).numpy()
    cfg = O.router_cfg(E, k, O.SIGMOID, True, n_group=8, topk_group=3, group_score_topk=gtop)
    idx, w = O.moe_route(z, cfg)
    assert np.array_equal(idx, _brute_grouped(z, E, k, 8, 3, gtop))
    s = 1.0 / (1.0 + np.exp(-np.take_along_axis(z, idx, 1).astype(np.float64)))
    np.testing.assert_allclose(w, s / s.sum(1, keepdims=True), rtol=1e-6)


def test_router_ties_go_to_lower_index_and_full_sort():
    T, E = 100, 16
    z = synth.tie_logits(T, E, 5, 3).numpy()
    cfg = O.router_cfg(E, E, O.SOFTMAX, False)
    idx, _ = O.moe_route(z, cfg)
    assert np.array_equal(idx, np.argsort(-z, axis=1, kind="stable"))
    cfg4 = O.router_cfg(E, 4, O.SIGMOID, True)
    idx4, _ = O.moe_route(z, cfg4)
    assert np.array_equal(idx4, np.argsort(-z, axis=1, kind="stable")[:, :4])


def masked_logits(T, E, seed, finite_per_token):
    """Logits where each token keeps only a few finite entries and the rest are -inf (experts
    masked out, e.g. by a -inf bias)."""
    rng = np.random.default_rng(seed)
    z = np.full((T, E), -np.inf, np.float32)
    for t in range(T):
        keep = rng.choice(E, size=finite_per_token[t % len(finite_per_token)], replace=False)
        z[t, keep] = rng.standard_normal(len(keep)).astype(np.float32)
    return z


@pytest.mark.parametrize("score", [O.SOFTMAX, O.SIGMOID])
def test_router_masked_experts_take_lowest_index(score):
    """A token with fewer than k finite logits fills its remaining slots with the lowest-index
    allowed experts of -inf logit (the same key order: -inf below every finite value, ties to the
    lower index), never with an invalid index; checked against an exhaustive sort."""
    T, E, k = 64, 32, 6
    # a softmax over a token with no finite logit is undefined (its maximum is -inf), so softmax
    # tokens keep at least one; sigmoid scores of -inf are fine (the exp input is clamped)
    z = masked_logits(T, E, 21, [1, 3, 5, 6, 9] if score == O.SOFTMAX else [0, 1, 3, 5, 6, 9])
    idx, w = O.moe_route(z, O.router_cfg(E, k, score, True))
    for t in range(T):
        ref = sorted(range(E), key=lambda e: (-float(z[t, e]), e))[:k]   # -(-inf) = inf sorts last
        assert idx[t].tolist() == ref
    assert np.all(idx >= 0) and np.all(idx < E) and np.all(np.isfinite(w))
    # group-limited: the same rule inside the kept groups
    cfg = O.router_cfg(E, 4, O.SIGMOID, True, n_group=4, topk_group=2, group_score_topk=2)
    gidx, _ = O.moe_route(z, cfg)
    assert np.all(gidx >= 0) and np.all(gidx < E)
    assert all(len(set(r)) == 4 for r in gidx.tolist())


def test_router_degenerate_cases():
    T, E = 64, 32
    z = synth.randn((T, E), 13, synth.STAGE, part=9).numpy()
    # k = 1 with renormalisation: weight exactly 1
    _, w1 = O.moe_route(z, O.router_cfg(E, 1, O.SIGMOID, True))
    assert np.all(w1 == 1.0)
    _, w1s = O.moe_route(z, O.router_cfg(E, 1, O.SOFTMAX, True))
    assert np.all(w1s == 1.0)
    # n_group == topk_group is the ungrouped router
    a = O.moe_route(z, O.router_cfg(E, 5, O.SIGMOID, True, n_group=4, topk_group=4))
    b = O.moe_route(z, O.router_cfg(E, 5, O.SIGMOID, True))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    # renormalised weights sum to 1 within k rounding steps
    _, w = O.moe_route(z, O.router_cfg(E, 8, O.SOFTMAX, True))
    assert np.all(np.abs(w.astype(np.float64).sum(1) - 1.0) <= 8 * 2 * U)


def test_record_and_replay_roundtrip():
    T, E, k = 257, 64, 6
    z = synth.randn((T, E), 14, synth.STAGE, part=10).numpy()
    cfg = O.router_cfg(E, k, O.SIGMOID, True, n_group=8, topk_group=4)
    payload = np.full((3, k, T + 5), -7, np.int32)   # [num_layers, top_k, seq_len] with slack columns
    idx, w = O.moe_route(z, cfg, record=payload[1])
    assert np.array_equal(payload[1][:, :T], idx.T) and np.all(payload[1][:, T:] == -7)
    assert np.all(payload[0] == -7) and np.all(payload[2] == -7)
    ridx, rw, bad = O.moe_replay_route(z, cfg, payload[1])
    assert bad == 0 and np.array_equal(ridx, idx) and np.array_equal(rw, w)
    # on different logits the indices are kept and the weights follow the current logits
    z2 = z + synth.randn((T, E), 14, synth.STAGE, part=11).numpy() * 0.5
    ridx2, rw2, _ = O.moe_replay_route(z2, cfg, payload[1])
    assert np.array_equal(ridx2, idx)
    s = 1.0 / (1.0 + np.exp(-np.take_along_axis(z2, idx, 1).astype(np.float64)))
    np.testing.assert_allclose(rw2, s / s.sum(1, keepdims=True), rtol=1e-6)


def test_replay_rejects_bad_indices():
    T, E, k = 6, 8, 3
    z = synth.randn((T, E), 15, synth.STAGE, part=12).numpy()
    rec = np.array([[0, 1, 2, 3, 4, 5], [1, 1, 8, 0, 5, 6], [2, 3, 4, -1, 6, 7]], np.int32)
    cfg = O.router_cfg(E, k, O.SOFTMAX, False)
    idx, w, bad = O.moe_replay_route(z, cfg, rec)
    # token 1: duplicate 1, token 2: 8 out of range, token 3: -1 out of range
    assert bad == 3
    for t in (1, 2, 3):
        assert np.all(idx[t] == -1) and np.all(w[t] == 0)
    for t in (0, 4, 5):
        assert idx[t].tolist() == rec[:, t].tolist()


# ----------------------------------------------------------------------------- quantisation
def _torch_quant(x: torch.Tensor, br: int):
    """Library reference for in-range values: torch fp32 division and the float8_e4m3fn cast."""
    R, C = x.shape
    xb = x.reshape(R // br, br, C // 128, 128)
    amax = xb.abs().amax(dim=(1, 3))
    s = torch.where(amax == 0, torch.ones_like(amax), amax / 448.0)
    q = (xb / s[:, None, :, None]).to(torch.float8_e4m3fn).view(torch.uint8).reshape(R, C)
    return q.numpy(), s.numpy()


@pytest.mark.parametrize("br", [1, 128])
def test_quant_matches_torch_cast(br):
    x = synth.randn((256, 512), 16, synth.STAGE, part=13) * 3.0
    x[5] = 0.0                                  # an all-zero row
    q, s = O.moe_quant_fp8_block(x.numpy(), br)
    rq, rs = _torch_quant(x, br)
    assert np.array_equal(q, rq) and np.array_equal(s, rs)


@pytest.mark.parametrize("br", [1, 128])
def test_quant_roundtrip_bound_and_block_max(br):
    x = (synth.randn((256, 384), 17, synth.STAGE, part=14) * 0.7).numpy()
    x[:, :128] *= 1e-3
    q, s = O.moe_quant_fp8_block(x, br)
    tab = O.e4m3_table()
    srow = np.repeat(np.repeat(s, br, 0), 128, 1).astype(np.float64)
    v = x.astype(np.float64) / srow            # exact-ish ratio
    deq = tab[q] * srow
    # per element: |x - deq| <= s * (half a grid step at |x/s|) + fp32 slack of the division
    e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -6)))
    half_step = np.where(np.abs(v) < 2.0 ** -6, 2.0 ** -10, 2.0 ** (e - 4))
    assert np.all(np.abs(x - deq) <= srow * (half_step + np.abs(v) * 2 * U) + 1e-30)
    # every non-zero block holds a code of magnitude 448
    blocks = (q.reshape(q.shape[0] // br, br, -1, 128) & 0x7F) == 0x7E
    assert np.all(blocks.any(axis=(1, 3)))


def test_quant_zero_block_and_signed_zero():
    x = np.zeros((128, 256), np.float32)
    x[:, 128:] = -0.0
    q, s = O.moe_quant_fp8_block(x, 128)
    assert np.all(s == 1.0) and np.all(q[:, :128] == 0x00) and np.all(q[:, 128:] == 0x80)


def test_quant_weight_block_transpose_and_batch():
    w = synth.randn((2, 256, 384), 18, synth.STAGE, part=15).numpy()
    q, s = O.moe_quant_fp8_block(w, 128)
    qt, st = O.moe_quant_fp8_block(np.ascontiguousarray(w.transpose(0, 2, 1)), 128)
    assert np.array_equal(qt, q.transpose(0, 2, 1)) and np.array_equal(st, s.transpose(0, 2, 1))
    q1, s1 = O.moe_quant_fp8_block(w[1], 128)
    assert np.array_equal(q1, q[1]) and np.array_equal(s1, s[1])


def test_quantise_then_permute_equals_permute_then_quantise():
    x = synth.randn((50, 256), 19, synth.STAGE, part=16).numpy()
    src = np.random.default_rng(3).integers(0, 50, 120).astype(np.int32)
    q, s = O.moe_quant_fp8_block(x, 1)
    q2, s2 = O.moe_quant_fp8_block(x[src], 1)
    assert np.array_equal(O.permute_rows(q, src), q2) and np.array_equal(O.permute_rows(s, src), s2)


# ----------------------------------------------------------------------------- dispatch
@pytest.mark.parametrize("shared", [False, True])
def test_dispatch_is_stable_argsort(shared):
    cfg = synth.CONFIGS["decode"]
    T, E, k = 300, cfg.E, cfg.k
    idx = synth.routing_indices(cfg, T).numpy()
    counts, offsets, dest, src = O.moe_dispatch(idx, E, shared)
    flat = idx.reshape(-1)
    order = np.argsort(flat, kind="stable")
    assert np.array_equal(src[:T * k], order // k)
    assert np.array_equal(dest.reshape(-1)[order], np.arange(T * k))
    assert np.array_equal(counts[:E], np.bincount(flat, minlength=E))
    assert counts.sum() == T * k + (T if shared else 0) and offsets[-1] == counts.sum()
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
    for t in range(T):
        for j in range(k):
            assert src[dest[t, j]] == t
    for e in range(E):
        seg = src[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)         # strictly ascending tokens within a group
    if shared:
        assert np.array_equal(src[offsets[E]:offsets[E + 1]], np.arange(T))


def test_dispatch_empty_groups_and_dropped_slots():
    idx = np.array([[3, 1], [3, -1], [-1, -1], [1, 3]], np.int32)
    counts, offsets, dest, src = O.moe_dispatch(idx, 5, False)
    assert counts.tolist() == [0, 2, 0, 3, 0]
    assert offsets.tolist() == [0, 0, 2, 2, 5, 5]
    assert dest.tolist() == [[2, 0], [3, -1], [-1, -1], [1, 4]]
    assert src.tolist() == [0, 3, 0, 1, 3]


# ----------------------------------------------------------------------------- GEMM
def test_gemm_exact_integer_case():
    M, N, K = 37, 256, 512
    a, ai = synth.integer_codes((M, K), 20, 0)
    b, bi = synth.integer_codes((N, K), 20, 1)
    ai, bi = ai.numpy(), bi.numpy()
    as_ = np.ones((M, K // 128), np.float32)
    bs = np.ones((N // 128, K // 128), np.float32)
    got = O.moe_grouped_gemm_fp8(a.numpy(), as_, np.array([0, M]), b.numpy()[None], bs[None])
    assert np.array_equal(got, (ai @ bi.T).astype(np.float64))
    # a common power-of-two scale stays exact
    got2 = O.moe_grouped_gemm_fp8(a.numpy(), as_ * 0.25, np.array([0, M]), b.numpy()[None], bs[None] * 8)
    assert np.array_equal(got2, 2.0 * (ai @ bi.T))


def test_gemm_block_form_and_brute_force():
    M, N, K = 3, 256, 256
    a = synth.random_codes((M, K), 21, 0).numpy()
    b = synth.random_codes((N, K), 21, 1).numpy()
    as_ = synth.random_scales((M, K // 128), 21, 2).numpy()
    bs = synth.random_scales((N // 128, K // 128), 21, 3).numpy()
    fast = O.moe_grouped_gemm_fp8(a, as_, np.array([0, M]), b[None], bs[None])
    blk = O.gemm_block_form(a, as_, b, bs)
    np.testing.assert_allclose(fast, blk, rtol=1e-12, atol=1e-12 * np.abs(blk).max())
    tab = np.array([_format_value(c) for c in range(256)])
    for m in range(M):
        for n in (0, 1, 127, 128, 255):
            ref = sum(tab[a[m, kk]] * as_[m, kk // 128] * tab[b[n, kk]] * bs[n // 128, kk // 128] for kk in range(K))
            assert abs(fast[m, n] - ref) <= 1e-12 * max(1.0, abs(ref))


def test_grouped_gemm_uses_each_groups_weights():
    K, N = 128, 128
    offsets = np.array([0, 2, 2, 5])             # group 1 empty
    a, ai = synth.integer_codes((5, K), 22, 0)
    b, bi = synth.integer_codes((3, N, K), 22, 1)
    ai, bi = ai.numpy(), bi.numpy()
    out = O.moe_grouped_gemm_fp8(a.numpy(), np.ones((5, 1), np.float32), offsets, b.numpy(),
                                 np.ones((3, 1, 1), np.float32))
    assert np.array_equal(out[:2], ai[:2] @ bi[0].T) and np.array_equal(out[2:], ai[2:] @ bi[2].T)


# ----------------------------------------------------------------------------- SwiGLU, combine
def test_swiglu_closed_form():
    g = synth.randn((7, 256), 23, synth.STAGE, part=17).double().numpy() * 4
    h = O.swiglu(g, 128)
    ref = torch.nn.functional.silu(torch.from_numpy(g[:, :128])) * torch.from_numpy(g[:, 128:])
    np.testing.assert_allclose(h, ref.numpy().astype(np.float32), rtol=2 * U)
    g[:, :128] = 0.0
    assert np.all(O.swiglu(g, 128) == 0.0)


def test_combine_gather_and_weighted_sum():
    rows, H, T, k = 12, 8, 4, 3
    y = synth.randn((rows, H), 24, synth.STAGE, part=18).numpy()
    dest = np.array([[0, 5, -1], [3, 3 + 1, 6], [11, 10, 9], [2, 7, 8]], np.int32)
    w = synth.randn((T, k), 24, synth.STAGE, part=19).numpy()
    out = O.moe_combine(y, dest, w)
    for t in range(T):
        ref = sum(float(w[t, j]) * y[dest[t, j]].astype(np.float64) for j in range(k) if dest[t, j] >= 0)
        np.testing.assert_allclose(out[t], ref, rtol=1e-15, atol=1e-15)
    # k = 1, w = 1: a pure gather; shared rows add
    d1 = np.array([[4], [0], [7], [7]], np.int32)
    g = O.moe_combine(y, d1, np.ones((T, 1), np.float32), y_shared=y[:T])
    assert np.array_equal(g, y[d1[:, 0]].astype(np.float64) + y[:T].astype(np.float64))


# ----------------------------------------------------------------------------- R3 payload codec
import oracle.payload as OP  # noqa: E402


def _payload_golden():
    cases = []
    with open(os.path.join(GOLD, "payload_pack.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            kv = dict(tok.split("=", 1) for tok in line.split())
            cases.append((int(kv["E"]), [int(v) for v in kv["idx"].split(",")],
                          [int(v) for v in kv["bytes"].split(",")]))
    return cases


@pytest.mark.parametrize("case", _payload_golden(), ids=lambda c: f"E{c[0]}")
def test_payload_pack_golden(case):
    E, idx, expect = case
    packed, bad = OP.payload_pack(np.array(idx, np.int32), E)
    assert bad == 0 and packed.tolist() == expect and OP.payload_pack_slow(idx, E) == expect
    assert len(expect) == OP.payload_bytes(len(idx), E)
    assert OP.payload_unpack(packed, len(idx), E).tolist() == idx


def test_payload_bits_closed_form():
    for E in list(range(1, 300)) + [1023, 1024, 1025, 65535, 65536]:
        b = OP.payload_bits(E)
        assert (1 << b) >= E and (b == 1 or (1 << (b - 1)) < E)
        assert b == max(1, math.ceil(math.log2(E)))


def test_payload_brute_force_and_round_trip():
    """Random payloads of every width up to 16 bits against the bit-by-bit construction; the 8-bit
    code of E <= 256 is the plain uint8 array; out-of-range indices are counted."""
    rng = np.random.default_rng(5)
    for E in (2, 3, 5, 8, 9, 31, 64, 100, 256, 257, 1000, 4097, 65536):
        for n in (1, 31, 32, 33, 95):
            idx = rng.integers(0, E, size=n).astype(np.int32)
            packed, bad = OP.payload_pack(idx, E)
            assert bad == 0 and packed.tolist() == OP.payload_pack_slow(idx, E)
            assert np.array_equal(OP.payload_unpack(packed, n, E), idx)
            if OP.payload_bits(E) == 8:
                assert np.array_equal(packed[:n], idx.astype(np.uint8)) and not packed[n:].any()
    idx = np.array([3, -1, 7, 8, 2], np.int32)
    _, bad = OP.payload_pack(idx, 8)
    assert bad == 2


# ----------------------------------------------------------------------------- power-of-two scales
def _is_pow2_f32(v: np.ndarray) -> np.ndarray:
    bits = np.asarray(v, np.float32).view(np.uint32)
    e, m = (bits >> 23) & 0xFF, bits & 0x7FFFFF
    return np.where(e == 0, (m != 0) & ((m & (m - 1)) == 0), m == 0)


def test_pow2_scale_definition():
    """s is a power of two, s >= t = fl32(amax / 448) and s / 2 < t (unless clamped at 2^-127);
    amax = 0 gives 1.  Checked on powers of two, their fp32 neighbours, subnormals and a wide sweep."""
    rng = np.random.default_rng(3)
    amax = [0.0, 448.0, 449.0, 224.0, 1.0, 2.0 ** -140, 2.0 ** -120, 3.4e38, 1e-45]
    for k in range(-140, 120, 7):
        p = np.float32(2.0 ** k)
        amax += [float(p), float(np.nextafter(p, np.float32(np.inf))), float(np.nextafter(p, np.float32(0)))]
    amax += list((10.0 ** rng.uniform(-44, 38, 2000)).astype(np.float32).astype(float))
    lo = np.float32(2.0 ** -127)
    for a in amax:
        s = np.float32(O.pow2_scale(a))
        if a == 0.0:
            assert s == 1.0
            continue
        t = np.float32(a) / np.float32(448.0)
        assert _is_pow2_f32(s), (a, s)
        assert s >= t and (s == lo or s / 2 < t), (a, s, t)
        assert s >= lo


def test_quant_pow2_codes_and_range():
    """Codes equal the library route (torch fp32 division, float8 cast) with the oracle's scales;
    every scale is a power of two; every non-zero block reaches the upper half of the e4m3 range
    (amax / s > 224, so its largest code is at least 224: the scale was rounded up to the next power
    of two, not down, which would saturate)."""
    x = synth.randn((2, 256, 384), 31, synth.STAGE, part=20).numpy() * np.float32(3.0)
    x[0, 0, :128] = 0.0
    x[1, 5, 128:256] *= np.float32(1e-30)
    for br in (1, 128):
        q, s = O.moe_quant_fp8_block(x, br, pow2=True)
        assert _is_pow2_f32(s).all()
        se = np.repeat(np.repeat(s, br, axis=1), 128, axis=2)
        lib = (torch.from_numpy(x) / torch.from_numpy(se)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(q, lib)
        vals = torch.from_numpy(q).view(torch.float8_e4m3fn).float().abs().numpy()
        bmax = vals.reshape(2, 256 // br, br, 3, 128).max(axis=(2, 4))
        nz = np.abs(x).reshape(2, 256 // br, br, 3, 128).max(axis=(2, 4)) > 0
        amax = np.abs(x).reshape(2, 256 // br, br, 3, 128).max(axis=(2, 4))
        assert (amax[nz] / s[nz] > 224).all() and (amax[nz] / s[nz] <= 448).all()
        assert (bmax[nz] >= 224).all() and (bmax[~nz] == 0).all()
        assert np.array_equal(s[~nz], np.ones(int((~nz).sum()), np.float32))
