"""The host-side planner, tree flattening and prefix identification under
AddressSanitizer, LeakSanitizer and UndefinedBehaviorSanitizer.

tests/host_fuzz.cpp is compiled with g++ together with the three plain C++
sources of the library (no HIP code is involved) and run over random valid
batches, trees and prompt sets, each followed by an invalid mutation that
must be rejected with an error status.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "prefix_shared_decode_amd", "csrc")
SOURCES = [os.path.join(ROOT, "tests", "host_fuzz.cpp")] + [
    os.path.join(CSRC, f) for f in ("plan.cpp", "flatten.cpp", "identify.cpp")]


@pytest.fixture(scope="module")
def fuzz_exe(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("needs g++")
    exe = tmp_path_factory.mktemp("host_fuzz") / "host_fuzz"
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", *SOURCES, "-o", str(exe)], check=True)
    return str(exe)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_host_fuzz_sanitized(fuzz_exe, seed):
    r = subprocess.run([fuzz_exe, str(seed), "300"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr[-4000:]
    assert r.stdout.strip().endswith("ok")
    assert "300 of 300 valid batches planned" in r.stdout
