"""Build the HIP library ``libpsa.so`` in-tree for gfx950.

Run ``python -m prefix_shared_decode_amd.build`` (or ``__graft_entry__.build()``).
Sources are compiled in parallel, then linked; the result sits next to this
file so it travels with the source tree.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libpsa.so")
OBJ = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from forming packed fp32 VALU ops.
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          f"-I{os.path.join(ROOT, 'include')}"]

SOURCES = ["abi.cpp", "plan.cpp", "flatten.cpp", "identify.cpp", "decode.hip", "merge.hip", "peaks.hip", "noalloc.hip"]


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, src + ".o")
    path = os.path.join(CSRC, src)
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, f"--offload-arch={ARCH}", *COMMON, *lang, "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    noise = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
