"""CPU check of the MFMA prefix tile's LDS index maps (csrc/layout.h).

The kernel and the checker include the same header, so this enumerates the
exact lane -> (token, chunk, LDS offset) maps the kernel uses: every copy and
every operand read must stay inside its tile, the copy must write each
(token, chunk) once, and reads must find the chunk the MFMA layout expects.
"""

import os
import shutil
import subprocess

import pytest

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "prefix_shared_decode_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_mfma_lds_layout(tmp_path):
    exe = tmp_path / "layout_check"
    subprocess.run(["g++", "-std=c++17", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    os.path.join(CSRC, "layout_check.cpp"), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ok" in r.stdout
