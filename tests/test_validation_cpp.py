"""CPU tier: the host-only planner/validator builds with plain g++ (no HIP)
and passes its error-path driver, also under AddressSanitizer."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("sanitize", [False, True])
def test_validation_driver(tmp_path, sanitize):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = tmp_path / "validate"
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "validation_driver.cpp"),
           os.path.join(ROOT, "long_context_attention_kvevict_amd", "csrc", "plan.cpp"), "-o", str(exe)]
    if sanitize:
        cmd[1:1] = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer"]
    subprocess.run(cmd, check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip() == "ok"
