"""Exhaustive equality of the router's fixed exp and sigmoid between the GPU and the oracle.

Every finite fp32 in [-90, 90] (about 2.2e9 values; outside that range both clamp to the same
ends) is evaluated on the GPU and by the oracle and compared bit for bit, in chunks of 2^28.
"""
import numpy as np
import pytest
import torch

import block_scaled_fp8_top_amd as M
import oracle as O

pytestmark = pytest.mark.gpu

HI = 0x42B40000  # bit pattern of 90.0


def _sweep(score_fn):
    step = 1 << 28
    checked = 0
    for sign in (0, 0x80000000):
        for start in range(0, HI + 1, step):
            stop = min(HI + 1, start + step)
            bits = torch.arange(start, stop, dtype=torch.int64, device="cuda").add_(sign).to(torch.int32)
            x = bits.view(torch.float32)
            y = M.moe_router_score_eval(x, score_fn).cpu().numpy()
            xh = (np.arange(start, stop, dtype=np.uint64) + sign).astype(np.uint32).view(np.float32)
            ref = O.pinned_exp(xh) if score_fn == "softmax" else O.pinned_sigmoid(xh)
            bad = np.flatnonzero(y.view(np.uint32) != ref.view(np.uint32))
            assert bad.size == 0, f"{bad.size} mismatches, first x={xh[bad[0]]!r} gpu={y[bad[0]]!r} ref={ref[bad[0]]!r}"
            checked += stop - start
            del bits, x
    # beyond the clamp
    x = torch.tensor([-1e30, -90.5, 90.5, 3e38, -3e38], device="cuda")
    y = M.moe_router_score_eval(x, score_fn).cpu().numpy()
    ref = (O.pinned_exp if score_fn == "softmax" else O.pinned_sigmoid)(x.cpu().numpy())
    assert np.array_equal(y.view(np.uint32), ref.view(np.uint32))
    return checked


def test_router_exp_exhaustive():
    n = _sweep("softmax")
    print(f"exp: {n} values equal")


def test_router_sigmoid_exhaustive():
    n = _sweep("sigmoid")
    print(f"sigmoid: {n} values equal")
