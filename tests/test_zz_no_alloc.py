"""The grouped GEMM entry point that allocates nothing (its tile plan in the library's own device
scratch) against the workspace entry point: bitwise the same outputs, on two calls in a row, the
second with fewer rows and groups than the first (the scratch keeps the previous call's plan)."""
import ctypes

import numpy as np
import pytest
import torch

import block_scaled_fp8_top_amd as M
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(seed, counts, N, K):
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rows = int(offsets[-1])
    G = len(counts)
    a = synth.random_codes((rows, K), seed, 80, device=DEV)
    as_ = synth.random_scales((rows, K // 128), seed, 81, device=DEV, lo=2.0 ** -10, hi=2.0 ** -6)
    b = synth.random_codes((G, N, K), seed, 82, device=DEV)
    bs = synth.random_scales((G, N // 128, K // 128), seed, 83, device=DEV, lo=2.0 ** -10, hi=2.0 ** -6)
    return torch.from_numpy(offsets).to(DEV), a, as_, b, bs, rows


def _check(offsets, a, as_, b, bs, rows, N, tile):
    for epi in (M.MOE_EPI_SWIGLU_QUANT, M.MOE_EPI_STORE):
        pk = M.moe_pack_weights_fp8(b, epi)
        if epi == M.MOE_EPI_STORE:
            ref = M.moe_grouped_gemm_fp8(a, as_, offsets, pk, bs, epi, torch.bfloat16, tile_rows=tile)
            out = torch.full((rows, N), 7.0, dtype=torch.bfloat16, device=DEV)
            got = M.moe_grouped_gemm_fp8_noalloc(a, as_, offsets, pk, bs, epi, out=out, tile_rows=tile)
            torch.cuda.synchronize()
            assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), (rows, tile, "store")
        else:
            hq, hs = M.moe_grouped_gemm_fp8(a, as_, offsets, pk, bs, epi, tile_rows=tile)
            oq = torch.full((rows, N // 2), 0x55, dtype=torch.uint8, device=DEV)
            osc = torch.full((rows, N // 256), -1.0, dtype=torch.float32, device=DEV)
            gq, gs = M.moe_grouped_gemm_fp8_noalloc(a, as_, offsets, pk, bs, epi, out=oq, out_scales=osc, tile_rows=tile)
            torch.cuda.synchronize()
            assert torch.equal(gq, hq) and torch.equal(gs.view(torch.int32), hs.view(torch.int32)), (rows, tile, "swiglu")


@pytest.mark.parametrize("tile", [0, 128])
def test_noalloc_equals_workspace_entry_two_calls(tile):
    rng = np.random.default_rng(5 + tile)
    N, K = 1024, 1024
    # first call: 33 groups (an empty one, a one-row one), ~20k rows: 256-row tiles when automatic
    big = rng.integers(300, 900, 33)
    big[3], big[17] = 0, 1
    c1 = _case(11, big, N, K)
    _check(*c1, N, tile)
    # second call: fewer groups and rows (128-row tiles when automatic)
    small = rng.integers(0, 200, 9)
    small[0] = 1
    c2 = _case(12, small, N, K)
    _check(*c2, N, tile)


def test_noalloc_rejects_plans_beyond_its_scratch():
    L = M.lib()
    P = ctypes.c_void_p(256)   # never dereferenced: the size check comes first
    rows = M.NOALLOC_SCRATCH_BYTES // 16 * 32   # more 32-row tiles than the scratch holds
    rc = L.moe_grouped_gemm_fp8_noalloc(P, P, P, 4, rows, P, M.MOE_B_PACKED, P, 256, 256, M.MOE_EPI_STORE,
                                        M.MOE_SCALE_AMAX, 0, P, M.MOE_BF16, None, None)
    assert rc == -6 and M.status_str(rc) == "workspace missing or too small"
    # the largest accepted plan still passes the check (rows up to the scratch's tile capacity)
    ok_rows = (M.NOALLOC_SCRATCH_BYTES - 256) // 16 * 32 - 32 * 4
    assert M.workspace_bytes(M.MOE_OP_GROUPED_GEMM, ok_rows, 0, 4, 0, 0) <= M.NOALLOC_SCRATCH_BYTES
