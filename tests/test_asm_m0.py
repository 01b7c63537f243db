"""M0 in the kernels that write LDS by buffer loads.

Those loads take their LDS address from M0 and are issued as inline
assembly that sets M0 itself.  M0 is a register the compiler reserves, so it
neither saves it around the asm nor knows that the asm changes it: that is
only safe while no code the compiler generates keeps a value in M0.  This
test compiles each such source for gfx950 and checks, on the assembly, that
every instruction naming M0 is one of the asm's writes and that each write
feeds the LDS-writing load right after it.
"""
import os
import re
import shutil
import subprocess

import pytest

from drafting_eagle_draft_amd import build as libbuild

SOURCES = ("gemm_tile.hip", "attn_decode.hip")

pytestmark = pytest.mark.skipif(not shutil.which(libbuild.HIPCC), reason="hipcc not available")

M0 = re.compile(r"\bm0\b")


def _instructions(asm):
    for line in asm.splitlines():
        text = line.split(";")[0].strip()
        if not text or text.startswith(".") or text.endswith(":"):
            continue
        yield text


@pytest.mark.parametrize("src", SOURCES)
def test_m0_only_feeds_lds_dma(src, tmp_path):
    out = tmp_path / (src + ".s")
    cmd = [libbuild.HIPCC, *libbuild.DEVICE_FLAGS, "--cuda-device-only", "-S",
           os.path.join(libbuild.CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    ins = list(_instructions(out.read_text()))
    writes = 0
    for i, text in enumerate(ins):
        if not M0.search(text):
            continue
        assert re.match(r"s_mov_b32 m0, s\d+$", text), f"{src}: M0 used by '{text}'"
        nxt = ins[i + 1] if i + 1 < len(ins) else ""
        assert nxt.startswith("buffer_load_dwordx4") and nxt.endswith(" lds"), \
            f"{src}: M0 write followed by '{nxt}'"
        writes += 1
    dma = sum(1 for t in ins if t.startswith("buffer_load_dwordx4") and t.endswith(" lds"))
    assert writes > 0 and writes == dma, (src, writes, dma)
