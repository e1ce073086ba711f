"""Router-replay payload codec on the GPU against the oracle's bit stream (bit-exact), through the
C-ABI.  Widths 1..16 bits, sizes around the 32-index group and the 8192-index workgroup tile,
out-of-range indices, the replay-stack payload shape with indices recorded by the router, and the
pinned-host round trip."""
import numpy as np
import pytest
import torch

import block_scaled_fp8_top_amd as M
import oracle.payload as OP
import synth
from gpu_helpers import DEV, assert_equal, host

pytestmark = pytest.mark.gpu

EXPERTS = [1, 2, 3, 5, 8, 9, 64, 100, 256, 257, 1000, 1024, 4097, 65536]   # b = 1, 1, 2, 3, 3, 4, 6, 7, 8, 9, 10, 10, 13, 16
SIZES = [1, 31, 32, 33, 8191, 8192, 8193, 100003]


@pytest.mark.parametrize("E", EXPERTS)
def test_payload_pack_matches_oracle(E):
    rng = np.random.default_rng(E)
    for n in SIZES:
        idx = rng.integers(0, E, size=n).astype(np.int32)
        packed = M.moe_payload_pack(torch.from_numpy(idx).to(DEV), E)
        ref, bad = OP.payload_pack(idx, E)
        assert bad == 0 and packed.numel() == ref.size
        assert_equal(f"packed E={E} n={n}", host(packed), ref)
        back = M.moe_payload_unpack(packed, (n,), E)
        assert_equal(f"unpacked E={E} n={n}", host(back), idx)


def test_payload_out_of_range_counted():
    E, n = 100, 5000
    rng = np.random.default_rng(1)
    idx = rng.integers(0, E, size=n).astype(np.int32)
    idx[[0, 17, 4999]] = [-1, 100, 127]
    bad = torch.zeros(1, dtype=torch.int32, device=DEV)
    packed = M.moe_payload_pack(torch.from_numpy(idx).to(DEV), E, bad_count=bad)
    ref, rbad = OP.payload_pack(idx, E)
    assert int(host(bad)[0]) == rbad == 3
    assert_equal("packed with bad indices", host(packed), ref)


def test_payload_replay_stack_round_trip_through_pinned_host():
    """The replay stack's payload [num_layers, top_k, seq_len] (here from routing indices of the
    prefill-shaped router, 4 layers) goes device -> pinned host as 1 byte per index and back."""
    cfg = synth.CONFIGS["r3"]
    L, k, T = 4, cfg.k, 4096
    payload = torch.stack([synth.routing_indices(cfg, T, seed_part=l).t().contiguous() for l in range(L)])
    payload = payload.to(torch.int32).to(DEV)
    assert tuple(payload.shape) == (L, k, T)
    nb = M.payload_bytes(payload.numel(), cfg.E)
    assert nb == payload.numel()          # 256 experts: one byte per index
    staging = torch.empty(nb, dtype=torch.uint8, device=DEV)
    hostbuf = torch.empty(nb, dtype=torch.uint8, pin_memory=True)
    M.moe_payload_to_host(payload, cfg.E, staging, hostbuf)
    torch.cuda.synchronize()
    ref, _ = OP.payload_pack(host(payload), cfg.E)
    assert np.array_equal(hostbuf.numpy(), ref)
    staging2 = torch.empty(nb, dtype=torch.uint8, device=DEV)
    back = M.moe_payload_from_host(hostbuf, (L, k, T), cfg.E, staging2)
    torch.cuda.synchronize()
    assert torch.equal(back, payload)


def test_payload_empty():
    packed = M.moe_payload_pack(torch.empty(0, dtype=torch.int32, device=DEV), 8)
    assert packed.numel() == 0
    back = M.moe_payload_unpack(packed, (0,), 8)
    assert back.numel() == 0
