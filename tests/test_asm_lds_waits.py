"""Static check of the gfx950 kernels' hand-issued LDS reads.

Several kernels read LDS with inline asm (so the compiler does not make them
wait for every direct-to-LDS load in flight).  The hardware does not interlock
a VGPR against an LDS read still in flight: until an ``s_waitcnt lgkmcnt``
covers the read, no instruction may read or overwrite the register it loads.
The compiler cannot know this about asm outputs and may copy such a register
right after the asm statement, so the kernels put each wait in the same
statement as its reads.  This test compiles every source to device assembly
and walks each function in layout order, tracking the registers of asm LDS
reads that no wait has covered yet; any other instruction that names one of
them fails the test.  No GPU is needed."""
import os
import re
import subprocess

import pytest

from block_scaled_fp4_histogram_amd import build as B


def _regs(tok):
    tok = tok.strip().rstrip(",")
    m = re.match(r"^v\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"^v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def lds_wait_hazards(asm_text):
    """[(function, instruction)] of uses of registers loaded by in-flight asm LDS reads."""
    out = []
    for name, body in re.findall(r"^(_Z\w+):[^\n]*\n(.*?)^\.Lfunc_end", asm_text, re.S | re.M):
        pending = []   # register sets of LDS-counter operations in issue order (LDS returns in order)
        in_asm = False
        for line in body.split("\n"):
            t = line.strip()
            if ";;#ASMSTART" in t:
                in_asm = True
                continue
            if ";;#ASMEND" in t:
                in_asm = False
                continue
            t = t.split(";")[0].strip()
            if not t or t.startswith(".") or t.endswith(":"):
                continue
            op, _, args = t.partition(" ")
            toks = [x for x in re.split(r",\s*|\s+", args) if x]
            if op == "s_waitcnt":
                m = re.search(r"lgkmcnt\((\d+)\)", t)
                if m:
                    n = int(m.group(1))
                    pending = pending[len(pending) - n:] if 0 < n < len(pending) else ([] if n == 0 else pending)
                continue
            if op.startswith("ds_read") or op.startswith("ds_load"):
                pending.append(_regs(toks[0]) if in_asm else set())
                continue
            if op.startswith("ds_") or op.startswith("s_load") or op.startswith("s_buffer_load"):
                pending.append(set())
                continue
            live = set().union(*pending) if pending else set()
            if live and any(_regs(x) & live for x in toks):
                out.append((name, t))
    return out


def test_checker_finds_a_planted_hazard():
    body = """_Zplanted:
\t;;#ASMSTART
\tds_read_b128 v[4:7], v1
\tds_read_b32 v9, v1 offset:16
\t;;#ASMEND
\tv_mov_b32_e32 v20, v9
\t;;#ASMSTART
\ts_waitcnt lgkmcnt(0)
\t;;#ASMEND
\tv_mov_b32_e32 v21, v5
.Lfunc_end0:
"""
    found = lds_wait_hazards(body)
    assert found == [("_Zplanted", "v_mov_b32_e32 v20, v9")]
    # a partial wait covers the older read only
    partial = body.replace("v_mov_b32_e32 v20, v9", "s_waitcnt lgkmcnt(1)\n\tv_mov_b32_e32 v20, v5")
    assert lds_wait_hazards(partial) == []
    partial2 = body.replace("v_mov_b32_e32 v20, v9", "s_waitcnt lgkmcnt(1)\n\tv_mov_b32_e32 v20, v9")
    assert lds_wait_hazards(partial2) == [("_Zplanted", "v_mov_b32_e32 v20, v9")]


@pytest.mark.parametrize("src", [os.path.basename(s) for s in B.SOURCES if s.endswith(".hip")])
def test_no_use_of_inflight_lds_reads(src, tmp_path):
    path = os.path.join(B.CSRC, src)
    flags = [f for f in B.FLAGS if f not in ("-shared", "-fPIC")]
    out = tmp_path / (src + ".s")
    r = subprocess.run([B.HIPCC] + flags + ["--cuda-device-only", "-S", path, "-o", str(out)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    text = out.read_text()
    assert re.search(r"^_Z\w+:", text, re.M), "no kernels in the assembly"
    found = lds_wait_hazards(text)
    assert not found, "\n".join(f"{n}: {t}" for n, t in found[:10])
