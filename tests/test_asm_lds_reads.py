"""The kernels' inline-assembly LDS reads, checked in the code the compiler generates.

Several kernels issue LDS reads as inline assembly and wait for them later (or at the end of
a multi-read block), so that the compiler's own waits do not also wait for unrelated memory
operations.  The compiler takes an asm read's destination as written when the asm statement
executes, but the data lands only when the read returns.  Until a `s_waitcnt lgkmcnt` covers
it, no instruction may read that register (a copy would copy stale data), use it as an
address (a later read of the same block), or write it (the returning data would overwrite the
new value).  Both happened in builds of this library: a four-read block whose outputs were not
early-clobber let the compiler give one read's destination to the next read's address, and a
key's validity flag then came from the wrong LDS word on some runs.

This compiles every source that holds such reads to gfx950 assembly and checks each
inline-asm LDS read against the instructions that follow it, up to the first lgkmcnt wait or
the end of the basic block.
"""

import os
import re
import subprocess
import tempfile

import pytest

from sparse_attention_qsa_amd import build as B


def _regs(tok: str):
    tok = tok.strip().rstrip(",")
    m = re.match(r"([va])\[(\d+):(\d+)\]$", tok)
    if m:
        return {(m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    if m:
        return {(m.group(1), int(m.group(2)))}
    return set()


def early_uses(asm_text: str):
    """(read, later instruction) pairs where the later instruction touches the read's
    destination before an lgkmcnt wait or a block boundary."""
    lines, in_asm = [], False
    for raw in asm_text.splitlines():
        s = raw.strip()
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not s or s.startswith((".", ";")):
            if s.endswith(":") and not s.startswith(";"):
                lines.append((s, False))
            continue
        lines.append((s, in_asm))
    found = []
    for i, (s, from_asm) in enumerate(lines):
        if not (from_asm and s.startswith("ds_read")):
            continue
        dst = _regs(s.split()[1])
        for later, _ in lines[i + 1:]:
            if later.endswith(":") or (later.startswith("s_waitcnt") and "lgkmcnt" in later):
                break
            parts = later.split(None, 1)
            if len(parts) < 2 or later.startswith("s_"):
                continue
            touched = set()
            for op in parts[1].split(","):
                touched |= _regs(op)
            if dst & touched:
                found.append((s, later))
    return found


def test_scanner_flags_a_destination_reused_as_an_address():
    asm = "\n".join([";;#ASMSTART", "ds_read_b32 v141, v150", "ds_read_b32 v134, v141",
                     "s_waitcnt lgkmcnt(0)", ";;#ASMEND"])
    assert len(early_uses(asm)) == 1
    ok = "\n".join([";;#ASMSTART", "ds_read_b32 v141, v150", "ds_read_b32 v134, v142",
                    "s_waitcnt lgkmcnt(0)", ";;#ASMEND", "v_mov_b32_e32 v1, v141"])
    assert early_uses(ok) == []
    # A copy of the destination before the wait, and an AGPR of the same number (no overlap).
    copy = "\n".join([";;#ASMSTART", "ds_read_b128 v[24:27], v1", ";;#ASMEND",
                      "v_mov_b32_e32 v5, v25", "v_accvgpr_write_b32 a24, v9"])
    assert [u[1] for u in early_uses(copy)] == ["v_mov_b32_e32 v5, v25"]


SOURCES_WITH_ASM_READS = ["gqa.hip", "logits_mfma.hip"]


@pytest.mark.parametrize("src", SOURCES_WITH_ASM_READS)
def test_inline_asm_lds_reads_are_waited_for_before_use(src):
    try:
        hipcc = B._hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    path = os.path.join(B.CSRC, src)
    with tempfile.TemporaryDirectory() as tmp:
        out = os.path.join(tmp, "k.s")
        flags = [f for f in B.COMMON if f != "-fPIC"]
        r = subprocess.run([hipcc, *flags, "--cuda-device-only", "-S", "-x", "hip", path,
                            "-o", out], capture_output=True, text=True, timeout=600)
        assert r.returncode == 0, r.stderr[-2000:]
        text = open(out).read()
    assert ";;#ASMSTART" in text
    bad = early_uses(text)
    assert not bad, "\n".join(f"{a}  ...  {b}" for a, b in bad[:10])
