"""C-ABI checks that need no GPU: the library loads, exports every function include/moe_fp8.h
declares, and rejects bad arguments on the host with the documented status codes before any
launch (so null device pointers are never touched)."""
import ctypes
import os
import re

import pytest
import torch

import block_scaled_fp8_top_amd as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_fp8.h")
OK, NULL, SHAPE, DTYPE, ARG, HIP, WS = 0, -1, -2, -3, -4, -5, -6


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(M.LIB_PATH):
        from block_scaled_fp8_top_amd import build
        build.build(verbose=False)
    return M.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), f"{n} declared in moe_fp8.h but not exported"
    assert set(names) == set(M.EXPORTED)


def test_status_strings_and_version(L):
    for code in (OK, NULL, SHAPE, DTYPE, ARG, HIP, WS):
        assert M.status_str(code)
    assert M.status_str(-99) == "unknown status"
    assert "gfx950" in M.version()


def test_workspace_sizes(L):
    a = M.workspace_bytes(M.MOE_OP_DISPATCH, 16384, 8, 256)
    b = M.workspace_bytes(M.MOE_OP_DISPATCH, 16385, 8, 256)
    assert 0 < a <= b
    assert M.workspace_bytes(M.MOE_OP_GROUPED_GEMM, 147456, 0, 257, 4096, 6144) > 0
    assert M.workspace_bytes(99, 1, 1, 1) == 0 and M.workspace_bytes(M.MOE_OP_DISPATCH, -1, 1, 1) == 0


def _cfg(**kw):
    d = dict(num_experts=256, top_k=8, score_fn=1, renormalize=1, n_group=8, topk_group=4, group_score_topk=2)
    d.update(kw)
    return M.RouterCfg(*[d[f] for f, _ in M.RouterCfg._fields_])


@pytest.mark.parametrize("kw,code", [
    ({}, NULL),                                        # valid cfg, null pointers
    ({"num_experts": 0}, ARG), ({"num_experts": 1025}, ARG), ({"top_k": 0}, ARG), ({"top_k": 65}, ARG),
    ({"num_experts": 4, "top_k": 5, "n_group": 1}, ARG), ({"score_fn": 2}, ARG), ({"n_group": 7}, ARG),
    ({"n_group": 0}, ARG), ({"topk_group": 9}, ARG), ({"topk_group": 0}, ARG), ({"group_score_topk": 0}, ARG),
    ({"group_score_topk": 33}, ARG), ({"topk_group": 1, "top_k": 33}, ARG), ({"n_group": 128, "num_experts": 1024}, ARG),
])
def test_route_validation(L, kw, code):
    cfg = _cfg(**kw)
    assert L.moe_route(None, 10, ctypes.byref(cfg), None, None, None, 0, None) == code
    assert L.moe_replay_route(None, 10, ctypes.byref(cfg), None, 10, None, None, None, None) == code


def test_route_validation_other(L):
    cfg = _cfg()
    assert L.moe_route(None, 10, None, None, None, None, 0, None) == NULL
    assert L.moe_route(None, -1, ctypes.byref(cfg), None, None, None, 0, None) == SHAPE
    assert L.moe_route(None, 0, ctypes.byref(cfg), None, None, None, 0, None) == OK          # empty: no-op
    assert L.moe_route(None, 10, ctypes.byref(cfg), None, None, ctypes.c_void_p(16), 9, None) == ARG  # record_ld < T
    assert L.moe_replay_route(None, 10, ctypes.byref(cfg), None, 9, None, None, None, None) == ARG
    assert L.moe_router_score_eval(None, 5, 2, None, None) == ARG
    assert L.moe_router_score_eval(None, 5, 0, None, None) == NULL
    assert L.moe_router_score_eval(None, 0, 0, None, None) == OK


def test_gate_logits_validation(L):
    assert L.moe_gate_logits(None, 0, None, None, 4, 128, 8, None, None) == NULL
    assert L.moe_gate_logits(None, 0, None, None, 4, 100, 8, None, None) == SHAPE     # H % 8
    assert L.moe_gate_logits(None, 0, None, None, 4, 128, 0, None, None) == SHAPE
    assert L.moe_gate_logits(None, 2, None, None, 4, 128, 8, None, None) == DTYPE
    assert L.moe_gate_logits(None, 1, None, None, 0, 128, 8, None, None) == OK


def test_quant_validation(L):
    assert L.moe_quant_fp8_block(None, 0, 1, 4, 100, 1, 0, None, None, None) == SHAPE     # cols % 128
    assert L.moe_quant_fp8_block(None, 0, 1, 100, 128, 128, 0, None, None, None) == SHAPE # rows % 128
    assert L.moe_quant_fp8_block(None, 0, 1, 128, 128, 64, 0, None, None, None) == ARG
    assert L.moe_quant_fp8_block(None, 0, 1, 128, 128, 1, 2, None, None, None) == ARG     # scale mode
    assert L.moe_quant_fp8_block(None, 2, 1, 128, 128, 1, 0, None, None, None) == DTYPE
    assert L.moe_quant_fp8_block(None, 0, 1, 128, 128, 1, 1, None, None, None) == NULL
    assert L.moe_quant_fp8_block(None, 0, 0, 128, 128, 1, 1, None, None, None) == OK


def test_dispatch_validation(L):
    P = ctypes.c_void_p(256)  # never dereferenced: every case fails on the host first
    args = lambda T=10, k=2, E=8, H=256, xq=None, ws=None, wsb=0: (P, T, k, E, 0, xq, xq, H, P, P, P, P, xq, xq, ws, wsb, None)
    assert L.moe_dispatch(*args(E=1025)) == SHAPE
    assert L.moe_dispatch(*args(k=0)) == SHAPE
    assert L.moe_dispatch(*args(xq=P, H=200)) == SHAPE
    assert L.moe_dispatch(*args()) == WS
    assert L.moe_dispatch(*args(ws=P, wsb=16)) == WS
    assert L.moe_dispatch(P, 10, 2, 8, 0, P, None, 256, P, P, P, P, P, P, P, 1 << 20, None) == NULL


def test_gemm_validation(L):
    P = ctypes.c_void_p(256)
    g = lambda N=256, K=256, epi=0, od=1, ws=P, wsb=1 << 20, osc=None, groups=4, tr=0, rows=100, bl=0, sm=0: (
        P, P, P, groups, rows, P, bl, P, N, K, epi, sm, tr, P, od, osc, ws, wsb, None)
    assert L.moe_grouped_gemm_fp8(*g(N=200)) == SHAPE
    assert L.moe_grouped_gemm_fp8(*g(K=100)) == SHAPE
    assert L.moe_grouped_gemm_fp8(*g(od=2)) == DTYPE
    assert L.moe_grouped_gemm_fp8(*g(epi=1, od=1)) == DTYPE
    assert L.moe_grouped_gemm_fp8(*g(epi=1, od=2, N=384)) == SHAPE    # F = 192 not a multiple of 128
    assert L.moe_grouped_gemm_fp8(*g(epi=1, od=2)) == NULL            # out_scales missing
    assert L.moe_grouped_gemm_fp8(*g(epi=7)) == ARG
    assert L.moe_grouped_gemm_fp8(*g(groups=0)) == SHAPE
    assert L.moe_grouped_gemm_fp8(*g(wsb=8)) == WS
    assert L.moe_grouped_gemm_fp8(*g(tr=40)) == ARG                   # tile height not 32, 48, 64, 128 or 256
    assert L.moe_grouped_gemm_fp8(*g(tr=256, bl=0)) == ARG            # 256-row tiles need packed weights
    assert L.moe_grouped_gemm_fp8(*g(rows=1 << 20, K=4096)) == SHAPE   # 2^32 bytes of activations
    assert L.moe_grouped_gemm_fp8(*g(N=1 << 17, K=1 << 15)) == SHAPE   # 2^32 bytes of one group's weights
    assert L.moe_grouped_gemm_fp8(*g(bl=3)) == ARG                    # unknown weight layout
    assert L.moe_grouped_gemm_fp8(*g(bl=2)) == ARG                    # FP4 weights need power-of-two scales
    assert L.moe_grouped_gemm_fp8(*g(sm=2)) == ARG                    # unknown scale mode
    assert L.moe_grouped_gemm_fp8(*g(sm=1, wsb=8)) == WS


def test_replay_gate_validation(L):
    P = ctypes.c_void_p(256)
    sig = M.router_cfg(256, 8, 1, 1, 8, 4, 2)
    soft = M.router_cfg(64, 6, 0, 0)
    f = lambda cfg=sig, T=100, H=512, dt=1, ld=100, x=P: (x, dt, P, None, T, H, ctypes.byref(cfg), P, ld, P, P, None, None)
    assert L.moe_replay_gate(*f(cfg=soft)) == ARG          # softmax weights need every logit
    assert L.moe_replay_gate(*f(H=100)) == SHAPE
    assert L.moe_replay_gate(*f(dt=2)) == DTYPE
    assert L.moe_replay_gate(*f(ld=50)) == ARG
    assert L.moe_replay_gate(*f(x=None)) == NULL
    assert L.moe_replay_gate(*f(T=0)) == OK


def test_gemm_plan_validation(L):
    P = ctypes.c_void_p(256)
    plan = M.GemmPlan()
    assert L.moe_grouped_gemm_plan(P, 4, 100, 40, P, 1 << 20, ctypes.byref(plan), None) == ARG   # tile height
    assert L.moe_grouped_gemm_plan(P, 0, 100, 0, P, 1 << 20, ctypes.byref(plan), None) == SHAPE
    assert L.moe_grouped_gemm_plan(P, 4, 100, 0, P, 8, ctypes.byref(plan), None) == WS
    assert L.moe_grouped_gemm_plan(P, 4, 100, 0, P, 1 << 20, None, None) == NULL
    assert L.moe_grouped_gemm_plan(P, 4, 0, 0, None, 0, ctypes.byref(plan), None) == OK          # nothing to plan
    assert plan.tile_rows == 32 and plan.groups == 4 and plan.max_rows == 0
    # automatic tile height: the smallest of 32/48/64/128 holding twice the average group, 256 for
    # groups averaging 256 rows or more
    for rows, groups, tr in ((100, 8, 32), (1536, 64, 48), (2000, 64, 64), (65280, 256, 128), (65536, 256, 256),
                             (147456, 257, 256)):
        L.moe_grouped_gemm_plan(P, groups, rows, 0, None, 0, ctypes.byref(plan), None)
        assert plan.tile_rows == tr, (rows, groups, plan.tile_rows)
    planned = lambda N=256, K=256, epi=0, od=1, bl=0, pl=True, sm=0: (
        ctypes.byref(plan) if pl else None, P, P, P, P, bl, P, N, K, epi, sm, P, od, None, None)
    plan.tile_rows, plan.groups, plan.max_rows, plan.workspace = 32, 4, 100, 256
    assert L.moe_grouped_gemm_fp8_planned(*planned(pl=False)) == NULL
    assert L.moe_grouped_gemm_fp8_planned(*planned(N=200)) == SHAPE
    assert L.moe_grouped_gemm_fp8_planned(*planned(od=2)) == DTYPE
    assert L.moe_grouped_gemm_fp8_planned(*planned(bl=3)) == ARG
    assert L.moe_grouped_gemm_fp8_planned(*planned(sm=5)) == ARG
    assert L.moe_grouped_gemm_fp8_planned(*planned(epi=1, od=2)) == NULL   # out_scales missing
    plan.tile_rows = 256
    assert L.moe_grouped_gemm_fp8_planned(*planned(bl=0)) == ARG           # 256-row plan, row-major weights
    plan.tile_rows = 40
    assert L.moe_grouped_gemm_fp8_planned(*planned()) == ARG


def test_pack_validation(L):
    P = ctypes.c_void_p(256)
    assert L.moe_pack_weights_fp8(P, 4, 256, 256, 7, P, None) == ARG
    assert L.moe_pack_weights_fp8(P, 4, 384, 256, 1, P, None) == SHAPE      # SwiGLU panels need N % 256
    assert L.moe_pack_weights_fp8(P, 4, 200, 256, 0, P, None) == SHAPE
    assert L.moe_pack_weights_fp8(P, 0, 256, 256, 0, P, None) == SHAPE
    assert L.moe_pack_weights_fp8(None, 4, 256, 256, 0, P, None) == NULL
    assert L.moe_pack_weights_fp8(P, 4, 1 << 17, 1 << 15, 0, P, None) == SHAPE


def test_packed_weight_bytes(L):
    assert M.packed_weight_bytes(4, 256, 512, M.MOE_EPI_STORE) == 4 * 256 * 512
    assert M.packed_weight_bytes(4, 384, 512, M.MOE_EPI_STORE) == 4 * 512 * 512      # padded to 2 panels
    assert M.packed_weight_bytes(257, 4096, 6144, M.MOE_EPI_SWIGLU_QUANT) == 257 * 4096 * 6144
    assert M.packed_weight_bytes(4, 384, 512, M.MOE_EPI_SWIGLU_QUANT) == 0
    assert M.packed_weight_bytes(4, 256, 100, M.MOE_EPI_STORE) == 0


def test_payload_validation_and_size(L):
    """Sizes follow the format (the oracle's formula); bad sizes, NULLs and misaligned pointers are
    rejected on the host."""
    import oracle.payload as OP
    for n, E in ((0, 8), (1, 1), (31, 5), (32, 256), (33, 257), (4 * 8 * 32768, 256), (10 ** 9, 1024), (7, 65536)):
        assert M.payload_bytes(n, E) == OP.payload_bytes(n, E)
    assert M.payload_bytes(-1, 8) == 0 and M.payload_bytes(5, 0) == 0 and M.payload_bytes(5, 65537) == 0
    P = ctypes.c_void_p(256)
    assert L.moe_payload_pack(P, -1, 8, P, None, None) == SHAPE
    assert L.moe_payload_pack(P, 5, 0, P, None, None) == SHAPE
    assert L.moe_payload_pack(P, 5, 65537, P, None, None) == SHAPE
    assert L.moe_payload_pack(None, 5, 8, P, None, None) == NULL
    assert L.moe_payload_pack(P, 5, 8, None, None, None) == NULL
    assert L.moe_payload_pack(ctypes.c_void_p(260), 5, 8, P, None, None) == ARG
    assert L.moe_payload_pack(None, 0, 8, None, None, None) == OK
    assert L.moe_payload_unpack(P, 5, 8, ctypes.c_void_p(264), None) == ARG
    assert L.moe_payload_unpack(None, 5, 8, P, None) == NULL
    assert L.moe_payload_to_host(P, 5, 8, P, None, None, None) == NULL
    assert L.moe_payload_from_host(None, 5, 8, P, P, None) == NULL
    assert L.moe_payload_from_host(P, 5, 8, None, P, None) == NULL


def test_combine_validation(L):
    P = ctypes.c_void_p(256)
    assert L.moe_combine(P, 1, P, P, 4, 2, 100, None, P, 1, None) == SHAPE
    assert L.moe_combine(P, 2, P, P, 4, 2, 128, None, P, 1, None) == DTYPE
    assert L.moe_combine(None, 1, P, P, 4, 2, 128, None, P, 1, None) == NULL
    assert L.moe_combine(None, 1, None, None, 0, 2, 128, None, None, 1, None) == OK


def test_binding_rejects_host_tensors(L):
    x = torch.zeros(4, 128)
    with pytest.raises(ValueError):
        M.moe_quant_fp8_block(x, 1)
    with pytest.raises(ValueError):
        M.moe_gate_logits(x, torch.zeros(8, 128))


def test_product_package_does_not_touch_the_oracle():
    """The HIP path's package never imports or loads the oracle."""
    pkg = os.path.join(ROOT, "block_scaled_fp8_top_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in src and "from oracle" not in src and "moe_oracle" not in src, f


def test_backward_validation(L):
    P = ctypes.c_void_p(16)   # never dereferenced: every case fails (or is empty) before a launch
    cfgp = ctypes.byref(_cfg())
    # combine backward: (dout, dt, y, yt, dest, w, T, k, H, shared, mode, dyq, dys, dw, row_w, stream)
    assert L.moe_combine_backward(P, 1, P, 1, P, P, 4, 17, 256, None, 0, P, P, P, None, None) == SHAPE   # k > 16
    assert L.moe_combine_backward(P, 1, P, 1, P, P, 4, 8, 200, None, 0, P, P, P, None, None) == SHAPE    # H % 128
    assert L.moe_combine_backward(P, 2, P, 1, P, P, 4, 8, 256, None, 0, P, P, P, None, None) == DTYPE
    assert L.moe_combine_backward(P, 1, P, 1, P, P, 4, 8, 256, None, 2, P, P, P, None, None) == ARG
    assert L.moe_combine_backward(None, 1, P, 1, P, P, 4, 8, 256, None, 0, P, P, P, None, None) == NULL
    assert L.moe_combine_backward(None, 1, None, 1, None, None, 0, 8, 256, None, 0, None, None, None, None, None) == OK
    # SwiGLU backward: (dh, g, rows, F, mode, dgq, dgs, stream)
    assert L.moe_swiglu_backward_quant(P, P, 4, 100, 0, P, P, None) == SHAPE
    assert L.moe_swiglu_backward_quant(P, P, 4, 128, 3, P, P, None) == ARG
    assert L.moe_swiglu_backward_quant(P, None, 4, 128, 0, P, P, None) == NULL
    assert L.moe_swiglu_backward_quant(None, None, 0, 128, 0, None, None, None) == OK
    # router backward: (logits, idx, dw, T, cfg, dz, stream)
    assert L.moe_route_backward(P, P, P, 4, None, P, None) == NULL
    assert L.moe_route_backward(P, P, P, 4, ctypes.byref(_cfg(top_k=300)), P, None) == SHAPE
    assert L.moe_route_backward(P, P, P, 4, ctypes.byref(_cfg(score_fn=5)), P, None) == ARG
    assert L.moe_route_backward(P, None, P, 4, cfgp, P, None) == NULL
    assert L.moe_route_backward(None, None, None, 0, cfgp, None, None) == OK
    # gate backward: (dz, x, xt, wg, T, H, E, dx_in, dx, dxt, dwg, db, ws, ws_bytes, stream)
    need = L.moe_gate_backward_workspace(16384, 256, 6144)
    assert need == 16 * (256 * 6144 + 256) * 4 and L.moe_gate_backward_workspace(256, 64, 4096) == 4 * (64 * 4096 + 64) * 4
    assert L.moe_gate_backward(P, P, 1, P, 4, 100, 8, None, P, 1, P, None, P, 1 << 20, None) == SHAPE
    assert L.moe_gate_backward(P, P, 2, P, 4, 128, 8, None, P, 1, P, None, P, 1 << 20, None) == DTYPE
    assert L.moe_gate_backward(P, P, 1, P, 16384, 6144, 256, None, P, 1, P, None, P, need - 1, None) == WS
    assert L.moe_gate_backward(P, None, 1, P, 4, 128, 8, None, P, 1, P, None, P, 1 << 20, None) == NULL
    assert L.moe_gate_backward(None, None, 1, None, 0, 128, 8, None, None, 1, None, None, None, 0, None) == OK
    # transpose: (q, s, G, N, K, qt, st, stream)
    assert L.moe_transpose_fp8_blocks(P, P, 2, 200, 256, ctypes.c_void_p(32), P, None) == SHAPE
    assert L.moe_transpose_fp8_blocks(P, P, 2, 256, 256, P, P, None) == ARG          # in place
    assert L.moe_transpose_fp8_blocks(P, None, 2, 256, 256, ctypes.c_void_p(32), P, None) == NULL
    assert L.moe_transpose_fp8_blocks(None, None, 0, 256, 256, None, None, None) == OK


def test_swiglu_save_validation(L):
    P = ctypes.c_void_p(16)
    plan = M.GemmPlan(128, 4, 1000, P)
    args = lambda g: (ctypes.byref(plan), P, P, P, P, 1, P, 512, 256, 0, P, P, g, None)
    assert L.moe_grouped_gemm_fp8_swiglu_save(*args(None)) == NULL
    assert L.moe_grouped_gemm_fp8_swiglu_save(None, P, P, P, P, 1, P, 512, 256, 0, P, P, P, None) == NULL
    bad = (ctypes.byref(plan), P, P, P, P, 1, P, 384, 256, 0, P, P, P, None)   # SwiGLU needs N % 256
    assert L.moe_grouped_gemm_fp8_swiglu_save(*bad) == SHAPE


def test_wgrad_validation(L):
    P = ctypes.c_void_p(16)
    assert L.moe_wgrad_max_tiles(147456, 257) == 1152 + 257 and L.moe_wgrad_max_tiles(-1, 4) == 0
    assert L.moe_wgrad_tiles(P, 0, P, None) == SHAPE and L.moe_wgrad_tiles(None, 4, P, None) == NULL
    # colwise rows: (x, xt, src, scale, offsets, tile_first, G, max_tiles, C, mode, qt, st, stream)
    assert L.moe_colwise_quant_rows(P, 1, None, None, P, P, 4, 10, 200, 0, P, P, None) == SHAPE
    assert L.moe_colwise_quant_rows(P, 2, None, None, P, P, 4, 10, 256, 0, P, P, None) == DTYPE
    assert L.moe_colwise_quant_rows(P, 1, None, None, P, P, 4, 10, 256, 7, P, P, None) == ARG
    assert L.moe_colwise_quant_rows(P, 1, None, None, None, P, 4, 10, 256, 0, P, P, None) == NULL
    assert L.moe_colwise_quant_rows(None, 1, None, None, None, None, 4, 0, 256, 0, None, None, None) == OK
    # colwise swiglu: (g, dh, F, offsets, tile_first, G, max_tiles, mode, qt, st, stream)
    assert L.moe_colwise_quant_swiglu(P, None, 100, P, P, 4, 10, 0, P, P, None) == SHAPE
    assert L.moe_colwise_quant_swiglu(P, None, 128, P, P, 4, 10, 9, P, P, None) == ARG
    assert L.moe_colwise_quant_swiglu(None, None, 128, P, P, 4, 10, 0, P, P, None) == NULL
    # wgrad GEMM: (a, as, M, b, bs, N, tile_first, G, max_tiles, mode, c, stream)
    assert L.moe_grouped_gemm_wgrad(P, P, 200, P, P, 256, P, 4, 10, 0, P, None) == SHAPE
    assert L.moe_grouped_gemm_wgrad(P, P, 256, P, P, 256, P, 0, 10, 0, P, None) == SHAPE
    assert L.moe_grouped_gemm_wgrad(P, P, 256, P, P, 256, P, 4, 10, 3, P, None) == ARG
    assert L.moe_grouped_gemm_wgrad(P, P, 256, P, None, 256, P, 4, 10, 0, P, None) == NULL


def test_fp4_validation(L):
    P = ctypes.c_void_p(256)
    # quant: (w, w_dtype, rows, cols, q, e8, stream)
    assert L.moe_quant_mxfp4(P, 1, 4, 48, P, P, None) == SHAPE        # cols not a multiple of 32
    assert L.moe_quant_mxfp4(P, 1, -1, 64, P, P, None) == SHAPE
    assert L.moe_quant_mxfp4(P, 2, 4, 64, P, P, None) == DTYPE        # FP8 input
    assert L.moe_quant_mxfp4(P, 1, 4, 64, None, P, None) == NULL
    assert L.moe_quant_mxfp4(None, 1, 0, 64, None, None, None) == OK  # empty
    sb = ctypes.c_size_t(0)
    assert M.lib().moe_packed_fp4_bytes(4, 512, 1024, 0, ctypes.byref(sb)) == 4 * 2 * 8 * 16384
    assert sb.value == 4 * 2 * 8 * 1024
    assert M.lib().moe_packed_fp4_bytes(4, 384, 1024, 0, None) == 4 * 2 * 8 * 16384   # padded to 2 panels
    assert M.lib().moe_packed_fp4_bytes(4, 384, 1024, 1, None) == 0                   # SwiGLU: N % 256
    assert M.lib().moe_packed_fp4_bytes(4, 512, 100, 0, None) == 0
    # pack: (q, e8, groups, N, K, epilogue, packed_q, packed_e8, stream)
    assert L.moe_pack_weights_fp4(P, P, 4, 512, 100, 0, P, P, None) == SHAPE
    assert L.moe_pack_weights_fp4(P, P, 0, 512, 128, 0, P, P, None) == SHAPE
    assert L.moe_pack_weights_fp4(P, P, 4, 512, 128, 5, P, P, None) == ARG
    assert L.moe_pack_weights_fp4(P, None, 4, 512, 128, 0, P, P, None) == NULL


def test_gather_validation(L):
    P = ctypes.c_void_p(16)
    plan = M.GemmPlan(128, 4, 1000, P)
    # (plan, a, a_count, a_rows, as, offsets, b, b_layout, bs, N, K, epilogue, scale_mode, out, out_dtype,
    #  out_scales, g_out, stream)
    g = lambda a_count=100, a_rows=P, g_out=None, K=256: (ctypes.byref(plan), P, a_count, a_rows, P, P, P, 1, P, 512,
                                                          K, 0, 0, P, 1, None, g_out, None)
    assert L.moe_grouped_gemm_fp8_gather(*g(a_rows=None)) == NULL
    assert L.moe_grouped_gemm_fp8_gather(*g(g_out=P)) == ARG          # G is kept only by the SwiGLU epilogue
    assert L.moe_grouped_gemm_fp8_gather(*g(a_count=0)) == SHAPE
    assert L.moe_grouped_gemm_fp8_gather(*g(a_count=1 << 24, K=512)) == SHAPE   # 2^33 bytes of gathered rows
    empty = M.GemmPlan(128, 4, 0, P)
    assert L.moe_grouped_gemm_fp8_gather(ctypes.byref(empty), None, 0, None, None, None, None, 1, None, 512, 256, 0, 0,
                                         None, 1, None, None, None) == OK
    # dispatch: scales only (aq NULL) needs xs and as; codes need xq
    assert L.moe_dispatch(P, 10, 2, 8, 0, None, None, 256, P, P, P, P, None, P, P, 1 << 20, None) == NULL
    assert L.moe_dispatch(P, 10, 2, 8, 0, None, P, 256, P, P, P, P, P, P, P, 1 << 20, None) == NULL


def test_dispatch_plan_validation(L):
    P = ctypes.c_void_p(256)
    plan = M.GemmPlan()
    # (idx, T, k, E, shared, xq, xs, H, counts, offsets, dest, src, aq, as, ws, ws_bytes, tile_rows, gws,
    #  gws_bytes, plan, stream)
    a = lambda tr=0, gwsb=1 << 20, pl=ctypes.byref(plan), E=8: (P, 10, 2, E, 0, None, None, 0, P, P, P, P, None, None,
                                                               P, 1 << 20, tr, P, gwsb, pl, None)
    assert L.moe_dispatch_plan(*a(pl=None)) == NULL
    assert L.moe_dispatch_plan(*a(tr=40)) == ARG
    assert L.moe_dispatch_plan(*a(gwsb=8)) == WS
    assert L.moe_dispatch_plan(*a(E=2000)) == SHAPE
