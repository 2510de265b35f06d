"""The prefill kernel's matrix instructions, read from its gfx950 assembly (no GPU).

Every product in the prefill runs as bf16 hi/lo halves on 16x16x32 bf16 MFMAs,
including the three-term 16x16 products that a 16x16x16 instruction would also
fit.  A 16x16x16 bf16 MFMA that accumulates onto a 16x16x32 one's result gave
wrong sums on gfx950 with the wait states the compiler put between them (a
one-wave probe sweeping the nop count between them: exact from 3 wait states
on), so the kernel keeps every dependent chain on one instruction.  This test
compiles the kernel to device assembly and checks that no other MFMA form
appears in any of its instantiations, and that every instantiation uses the
16x16x32 bf16 form.
"""
import os
import re
import subprocess
import tempfile

import pytest

from hybrid_linear_attention_slot_amd import build as b

SRC = os.path.join(b.CSRC, "prefill_kernel.hip")


@pytest.fixture(scope="module")
def prefill_asm():
    try:
        hipcc = b._hipcc()
    except RuntimeError as e:
        pytest.skip(str(e))
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "prefill.s")
        cmd = [hipcc, "-x", "hip", *b.common_flags(), "--cuda-device-only", "-S", SRC, "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        with open(out) as f:
            return f.read()


def kernels(asm):
    """{kernel symbol: its instruction lines} for every prefill_kernel instantiation."""
    out = {}
    for name in re.findall(r"^(_Z\S*prefill_kernel\S*E):", asm, re.M):
        body = asm[asm.index(name + ":"):]
        body = body[:body.index(".Lfunc_end")]
        out[name] = [l.strip() for l in body.splitlines()
                     if l.strip() and not l.strip().startswith((";", "."))]
    return out


def test_every_instantiation_is_found(prefill_asm):
    ks = kernels(prefill_asm)
    # head sizes 16, 32, 64, 128 at conv widths 2-4 in 64-column workgroups,
    # and head size 128 in whole-head ones
    assert len(ks) == 15, sorted(ks)


def test_only_16x16x32_bf16_mfmas(prefill_asm):
    for name, lines in kernels(prefill_asm).items():
        ops = {l.split()[0] for l in lines if l.startswith("v_mfma")}
        assert ops == {"v_mfma_f32_16x16x32_bf16"}, (name, ops)
