"""Register budget of the fused kernel: no instantiation uses scratch.

The compiler's resource remarks for decode.hip, built with the library's
own flags for gfx950 (host cross-compile, no GPU needed).  A spill or a
kernel argument copied to private memory (e.g. a tile function the compiler
decided not to inline) shows up as a non-zero scratch size.
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not shutil.which(HIPCC) and not os.path.exists(HIPCC), reason="hipcc not installed")
def test_no_instantiation_uses_scratch(tmp_path):
    from prefix_shared_decode_amd.build import ARCH, COMMON

    src = os.path.join(ROOT, "prefix_shared_decode_amd", "csrc", "decode.hip")
    cmd = [HIPCC, f"--offload-arch={ARCH}", *COMMON, "-x", "hip", "-c", src, "-o", str(tmp_path / "d.o"),
           "--offload-device-only", "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    names = re.findall(r"Function Name: (\S+)", r.stderr)
    scratch = [int(x) for x in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", r.stderr)]
    assert len(names) == len(scratch) == 16, (names, scratch)
    usage = dict(zip(names, scratch))
    # decode_kernel<D, R, BF16>: mangled ...ILi<D>ELi<R>ELb<0|1>E...
    assert len([n for n in usage if re.search(r"ELb1E", n)]) == 8
    assert all(s == 0 for s in usage.values()), usage
