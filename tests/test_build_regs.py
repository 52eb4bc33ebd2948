"""The HIP kernels build without register spills.

A kernel that runs out of registers spills to scratch memory; in the
scorer's streaming loops every spill reload also waits on the vector-memory
counter that paces the K/V ring, which stalls the pipeline.  This compiles
each HIP source to gfx950 assembly with the library's own flags and checks
that every kernel reports zero scratch.  CPU only (cross-compilation).
"""
import os
import re
import subprocess

import pytest

from long_context_attention_kvevict_amd import build as B


@pytest.mark.parametrize("src", [s for s in B.SOURCES if s.endswith(".hip")])
def test_no_scratch_spills(src, tmp_path):
    out = tmp_path / (src + ".s")
    cmd = [B.HIPCC, "-x", "hip", *B.DEVICE, *B.COMMON, *B.PER_FILE.get(src, []), "--cuda-device-only",
           "-S", os.path.join(B.CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    text = out.read_text()
    kernels = re.findall(r"^(_Z\w+):\s+; @", text, re.M)   # function labels (not data symbols)
    scratch = [int(x) for x in re.findall(r"; ScratchSize: (\d+)", text)]
    assert kernels and len(scratch) >= len(kernels)
    assert all(x == 0 for x in scratch), f"{src}: scratch sizes {scratch}"
