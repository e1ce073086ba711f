"""CPU oracle of the router-replay payload codec.

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` and the CPU baseline leg of ``bench.py``; never by
the product package, and it shares no code with the HIP library.

"RL at 1T Scale: prime-rl Performance Deep Dive", section "Router replay": the routing decisions
recorded at inference form a ``[num_layers, top_k, seq_len]`` integer payload that reaches tens of
Gbps and hundreds of GB, and is handled as an opaque tensor by tensor operations only.  The pages
give no storage format.  The reading used here (a lossless fixed-width code): every index of an
E-expert router fits in b = max(1, ceil(log2 E)) bits; index i of the flattened payload occupies
bits [i*b, (i+1)*b) of a little-endian bit stream, least significant bit first (stream bit j is
bit j % 8 of byte j // 8); the stream is zero-padded to whole groups of 32 indices, so a packed
payload has ceil(n / 32) * 4 * b bytes.  Indices outside [0, E) are not representable: they are
counted, and their low b bits are stored.
"""
from __future__ import annotations

import numpy as np


def payload_bits(E: int) -> int:
    """b = max(1, ceil(log2 E)): the fewest bits that hold every index 0 .. E-1."""
    if E < 1:
        raise ValueError("E >= 1")
    b = 1
    while (1 << b) < E:
        b += 1
    return b


def payload_bytes(n: int, E: int) -> int:
    """Packed size: whole 32-index groups of b 32-bit words each."""
    return -(-n // 32) * 4 * payload_bits(E)


def payload_pack(idx: np.ndarray, E: int) -> tuple[np.ndarray, int]:
    """Bit stream of the flattened indices (definition above) and the count of indices outside [0, E)."""
    b = payload_bits(E)
    v = np.asarray(idx, dtype=np.int64).reshape(-1)
    bad = int(np.count_nonzero((v < 0) | (v >= E)))
    n = v.size
    ngroups = -(-n // 32)
    padded = np.zeros(ngroups * 32, dtype=np.int64)
    padded[:n] = v & ((1 << b) - 1)
    # bit j of index i -> stream position i*b + j
    bits = ((padded[:, None] >> np.arange(b, dtype=np.int64)[None, :]) & 1).astype(np.uint8).reshape(-1)
    return np.packbits(bits, bitorder="little"), bad


def payload_unpack(packed: np.ndarray, n: int, E: int) -> np.ndarray:
    """Inverse of payload_pack for indices in [0, E): read b bits per index, least significant first."""
    b = payload_bits(E)
    bits = np.unpackbits(np.asarray(packed, dtype=np.uint8), bitorder="little")[: n * b]
    bits = bits.reshape(n, b).astype(np.int64)
    return (bits << np.arange(b, dtype=np.int64)[None, :]).sum(axis=1).astype(np.int32)


def payload_pack_slow(idx, E: int) -> list[int]:
    """The same stream built one bit at a time with plain integers (small inputs only)."""
    b = payload_bits(E)
    flat = [int(x) for x in np.asarray(idx).reshape(-1)]
    nbytes = payload_bytes(len(flat), E)
    out = [0] * nbytes
    for i, x in enumerate(flat):
        for j in range(b):
            if (x >> j) & 1:
                pos = i * b + j
                out[pos // 8] |= 1 << (pos % 8)
    return out
