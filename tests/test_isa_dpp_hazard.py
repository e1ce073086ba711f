"""The gate projection's x-broadcast kernel feeds its fmas through DPP row broadcasts written as
inline assembly (v_fmac_f32_dpp).  A DPP source register needs two wait states after a VALU
instruction writes it, and the compiler does not insert them for inline assembly, so the kernel
routes its widened x through an s_nop.  This test compiles the kernel's source to gfx950 assembly
with the library's flags (no GPU needed) and checks every DPP instruction of it: walking back from
it through straight-line code, no VALU instruction within two wait states writes its DPP source."""
import os
import re
import shutil
import subprocess

import pytest

from block_scaled_fp8_top_amd import build

SRC = os.path.join(build.CSRC, "gate_logits.hip")


def _vregs(op: str) -> set:
    op = op.strip()
    m = re.match(r"v\[(\d+):(\d+)\]", op)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", op)
    return {int(m.group(1))} if m else set()


def dpp_hazards(asm: str):
    """(kernel, dpp instruction count, list of (writer, reader)) over every kernel of `asm`."""
    found, count, kernel, insts = [], 0, None, []
    for line in asm.splitlines():
        if re.match(r"^_Z\S*:", line):
            kernel, insts = line[:-1], []
            continue
        s = line.split(";")[0].strip()
        if kernel is None or not s or s.startswith("."):
            continue
        if s.endswith(":"):
            insts.append(None)   # a branch target: the window must close before it
            continue
        insts.append(s)
        mnem = s.split()[0]
        if not mnem.endswith("_dpp"):
            continue
        count += 1
        src0 = _vregs(s.split(None, 1)[1].split(",")[1])
        states = 0
        for prev in reversed(insts[:-1]):
            if prev is None:
                found.append((kernel, "label", s))
                break
            pm = prev.split()[0]
            if pm.startswith("v_") and " " in prev and _vregs(prev.split(None, 1)[1].split(",")[0]) & src0:
                found.append((kernel, prev, s))
                break
            n = re.match(r"s_nop\s+(\d+)", prev)
            states += int(n.group(1)) + 1 if n else 1
            if states >= 2:
                break
    return count, found


def test_scanner_flags_a_planted_hazard():
    """The scanner itself: a VALU write one instruction before the DPP read is reported, an s_nop 1
    in between clears it."""
    bad = "_Zk:\n v_add_f32_e32 v1, v1, v1\n v_fmac_f32_dpp v3, v1, v2 row_newbcast:0\n"
    good = "_Zk:\n v_add_f32_e32 v1, v1, v1\n s_nop 1\n v_fmac_f32_dpp v3, v1, v2 row_newbcast:0\n"
    assert dpp_hazards(bad)[1] and not dpp_hazards(good)[1]


@pytest.mark.skipif(not shutil.which(build.HIPCC) and not os.path.exists(build.HIPCC), reason="hipcc not found")
def test_gate_logits_dpp_sources_settled():
    cmd = [build.HIPCC, *build.CFLAGS, "--cuda-device-only", "-S", "-o", "-", SRC]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    count, found = dpp_hazards(r.stdout)
    assert count >= 2 * (128 + 256), count   # the broadcast kernels are all there (slices of 64 and 128 experts, bf16/fp32)
    assert not found, found[:5]
