"""Build libdgemm.so (gfx950) in-tree with hipcc.

Run as ``python -m dense_gemm_02_amd.build`` or through
``__graft_entry__.build()``.  Always recompiles.
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = [os.path.join(HERE, "csrc", "dgemm.hip")]
OUT = os.path.join(HERE, "libdgemm.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # Packed FP32 VALU forms are kept out of every kernel.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


def build(extra_flags=None, out=OUT, verbose=False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc] + HIPCC_FLAGS + list(extra_flags or []) + SRC + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libdgemm.so")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(sys.argv[1:], verbose=True))
