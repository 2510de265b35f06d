"""The copy kernels' stores, read from their gfx950 assembly (no GPU).

A gather or scatter call ends when its last workgroups finish, and each
workgroup ends with the remainder of its share: a partial block of 16-byte
units.  On gfx9-family GPUs one counter (vmcnt) tracks loads and stores alike,
so a store that waits for vmcnt(0) waits for every earlier store of the wave
to complete as well.  When the remainder was copied round by round behind a
branch per round, the compiler put such a wait before each of its stores and
they went out one at a time (gather / scatter 1.5-2 % slower).  The remainder
is now one unguarded block whose rounds past the end fall outside the buffer
resources.  This test compiles the copy kernels and checks that no store of
the gather / scatter kernels has a wait for all memory operations in its own
basic block.

The remainder's lanes past the end rely on the buffer range check, which
for the raw buffer intrinsics covers the VGPR offset of an access but not its
SGPR offset; so the
remainder's loads must carry their whole offset in the VGPR (a zero SGPR
offset), or lanes past the end would read up to a block beyond the region.
"""
import os
import re
import subprocess
import tempfile

import pytest

from hybrid_linear_attention_slot_amd import build as b

SRC = os.path.join(b.CSRC, "copy_kernels.hip")


@pytest.fixture(scope="module")
def copy_asm():
    try:
        hipcc = b._hipcc()
    except RuntimeError as e:
        pytest.skip(str(e))
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "copy.s")
        cmd = [hipcc, "-x", "hip", *b.common_flags(), "--cuda-device-only", "-S", SRC, "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        with open(out) as f:
            return f.read()


def kernel_lines(asm, pattern):
    out = {}
    for name in re.findall(r"^(_Z\S*" + pattern + r"\S*E):", asm, re.M):
        body = asm[asm.index(name + ":"):]
        body = body[:body.index(".Lfunc_end")]
        lines = [l.split(";")[0].strip() for l in body.splitlines()]
        out[name] = [l for l in lines if l and (l.endswith(":") or not l.startswith("."))]
    return out


def stores_after_full_wait(lines):
    """Stores with an s_waitcnt vmcnt(0) earlier in their own basic block."""
    bad, waited = [], False
    for i, l in enumerate(lines):
        if l.endswith(":") or l.startswith(("s_branch", "s_cbranch")):
            waited = False
        elif l.startswith("s_waitcnt") and "vmcnt(0)" in l:
            waited = True
        elif l.startswith("buffer_store"):
            if waited:
                bad.append((i, l))
            waited = False
    return bad


def test_both_directions_are_found(copy_asm):
    assert len(kernel_lines(copy_asm, "rows_balanced_kernel")) == 2


def test_no_store_waits_for_all_memory_operations(copy_asm):
    for name, lines in kernel_lines(copy_asm, "rows_balanced_kernel").items():
        assert sum(l.startswith("buffer_store") for l in lines) >= 16, name
        assert stores_after_full_wait(lines) == [], name


def test_remainder_loads_are_range_checked_in_full(copy_asm):
    # eight loads per lane in the remainder block, each with a zero SGPR offset
    for name, lines in kernel_lines(copy_asm, "rows_balanced_kernel").items():
        loads = [l for l in lines if l.startswith("buffer_load")]
        zero_soffset = [l for l in loads if re.search(r"\], 0 offen", l)]
        assert len(zero_soffset) >= 8, (name, loads)
