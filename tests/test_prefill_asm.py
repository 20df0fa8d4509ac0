"""Build check of the prefill attention kernel's hand-issued global->LDS
copies (sas_device.h copy16), on the CPU.

The copies are written as inline asm (M0 write, one wait state, the load) so
that the compiler does not drain every load before each later LDS read, and
they are awaited by explicit vmcnt waits the compiler cannot see.  That is
only sound when (1) nothing else in the kernel uses M0, which the asm clobbers,
and (2) no other vector-memory instruction is issued between the first copy
and the final drain, so that each vmcnt wait counts copies only.  This test
compiles prefill.hip for gfx950 with the library's flags and checks both on
the generated AMD assembly of every prefill_attend_kernel instance and of
prefill_grad_kernel (the backward's walk, which copies the same way).
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "learned_block_sparse_tok_amd", "csrc")

VMEM = re.compile(r"^\s*(global|buffer|flat|scratch)_\w+")


def kernel_bodies(asm: str):
    """(name, [instruction lines]) of every prefill_attend_kernel instance and
    of prefill_grad_kernel."""
    lines = asm.splitlines()
    out, cur, name = [], None, None
    for ln in lines:
        m = re.match(r"^(_Z\w*prefill_(?:attend|grad)_kernel\w*):", ln)
        if m:
            cur, name = [], m.group(1)
            continue
        if cur is not None:
            s = ln.split(";")[0].strip()
            if s and not s.startswith(".") and not s.endswith(":"):
                cur.append(s)
            if s.startswith("s_endpgm"):
                out.append((name, cur))
                cur = None
    return out


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not installed")
def test_prefill_copies_own_m0_and_the_load_counter(tmp_path):
    from learned_block_sparse_tok_amd import build as hip_build
    flags = [f for f in hip_build.FLAGS if f not in ("-shared", "-fPIC")]
    out = tmp_path / "prefill.s"
    subprocess.check_call(["hipcc", *flags, "--cuda-device-only", "-S", "-I", os.path.join(ROOT, "include"),
                           os.path.join(CSRC, "prefill.hip"), "-o", str(out)],
                          stderr=subprocess.DEVNULL)
    bodies = kernel_bodies(out.read_text())
    assert len(bodies) >= 9  # plain and gated forward and the backward's walk, for 1, 2 and 4 heads per column group
    assert any("prefill_grad_kernel" in name for name, _ in bodies)
    for name, ins in bodies:
        copies = [i for i, s in enumerate(ins) if s.startswith("global_load_lds_dwordx4")]
        assert copies, name
        # (1) M0: written only right before a copy, read by nothing else
        for i, s in enumerate(ins):
            if re.search(r"\bm0\b", s):
                assert s.startswith("s_mov_b32 m0,"), (name, s)
                nxt = [t for t in ins[i + 1:i + 4] if not t.startswith("s_nop")]
                assert nxt and nxt[0].startswith("global_load_lds_dwordx4"), (name, ins[i:i + 4])
        # (2) between the first copy and the drain after the last one, the
        # only vector-memory instructions are copies, and the waits are the
        # walk's own, all alike: vmcnt(0) when the blocks are taken in pairs
        # (the prologue issues two blocks' copies before the first wait), or
        # at most two later stages' copies outstanding when they are taken one
        # at a time (three blocks' copies before the first wait)
        drain = next(i for i in range(copies[-1], len(ins)) if re.match(r"s_waitcnt .*vmcnt\(0\)", ins[i]))
        first_wait = next(i for i in range(copies[0], drain + 1) if re.match(r"s_waitcnt .*vmcnt\(", ins[i]))
        prologue = sum(1 for s in ins[copies[0]:first_wait] if s.startswith("global_load_lds_dwordx4"))
        waits = set()
        for s in ins[copies[0]:drain]:
            if VMEM.match(s):
                assert s.startswith("global_load_lds_dwordx4"), (name, s)
            m = re.match(r"s_waitcnt .*vmcnt\((\d+)\)", s)
            if m:
                waits.add(int(m.group(1)))
        assert len(waits) == 1, (name, waits)
        w = waits.pop()
        if w == 0:
            assert prologue > 0 and prologue % 2 == 0, (name, prologue)
        else:
            assert prologue % 3 == 0 and w == 2 * prologue // 3, (name, prologue, w)
