"""Build libdgemm.so (gfx950) in-tree with hipcc.

Run as ``python -m dense_gemm_02_amd.build`` or through
``__graft_entry__.build()``.  Always recompiles.

The library is one host/dispatch translation unit (csrc/dgemm.hip) plus the
four-wave kernel instantiated once per input format and layout
(csrc/four_wave.hip compiled with -D selectors); the objects are compiled
in parallel under _build/ and linked into one shared library.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libdgemm.so")
OBJDIR = os.path.join(HERE, "_build")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # Packed FP32 VALU forms are kept out of every kernel.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]

# (object tag, Op, NN with transposing reads?, kernel-name prefix)
FOUR_WAVE = [
    ("f16_tn", "OpF16", 0), ("f16_nn", "OpF16", 1),
    ("bf16_tn", "OpBF16", 0), ("bf16_nn", "OpBF16", 1),
    ("fp8_tn", "OpFP8", 0), ("fp8_nn", "OpFP8", 1),
    ("fp8s_tn", "OpFP8S", 0), ("fp8s_nn", "OpFP8S", 1),
    ("mx8_tn", "OpMX8", 0), ("mx8_nn", "OpMX8", 1),
]


def units():
    """(source, object, extra flags) of every translation unit."""
    out = [(os.path.join(CSRC, "dgemm.hip"), os.path.join(OBJDIR, "dgemm.o"), []),
           (os.path.join(CSRC, "pp.hip"), os.path.join(OBJDIR, "pp.o"), [])]
    for tag, op, nn in FOUR_WAVE:
        out.append((os.path.join(CSRC, "four_wave.hip"), os.path.join(OBJDIR, f"four_wave_{tag}.o"),
                    [f"-DDG_OP={op}", f"-DDG_PKM={nn}", f"-DDG_TAG={tag}", f"-DDG_FN=four_wave_{tag}"]))
    return out


def _compile(hipcc, src, obj, flags, extra, verbose):
    cmd = [hipcc] + HIPCC_FLAGS + list(extra or []) + flags + ["-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed on {os.path.basename(obj)}")
    return obj


def build(extra_flags=None, out=OUT, verbose=False, jobs=None) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(OBJDIR, exist_ok=True)
    jobs = jobs or min(16, len(os.sched_getaffinity(0)))
    us = units()
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda u: _compile(hipcc, u[0], u[1], u[2], extra_flags, verbose), us))
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed linking libdgemm.so")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(sys.argv[1:], verbose=True))
