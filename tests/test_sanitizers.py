"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

* The oracle (oracle/oracle.cpp, g++) driven by tests/sanitize/oracle_harness.cpp
  over edge shapes, padded leading dimensions and row subsets.
* The library's host side (argument checks, kernel and tile choice, split
  planning, tile map, sizing helpers) driven by tests/sanitize/abi_harness.cpp
  through the C ABI with arguments that are refused before any launch and
  with the host-only planning helpers.  Only host code is instrumented (the
  sanitizer flags go to the host compilation); the kernels are compiled as
  usual and never launched.
"""

import concurrent.futures as cf
import os
import subprocess

import pytest

from dense_gemm_02_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, (" ".join(cmd[:3]), res.stdout[-3000:], res.stderr[-3000:])
    return res


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["g++", "-O1", "-g", "-std=c++17", "-fopenmp", "-ffp-contract=off", "-fno-omit-frame-pointer",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          os.path.join(ROOT, "oracle", "oracle.cpp"), os.path.join(HERE, "oracle_harness.cpp"), "-o", exe])
    res = _run([exe], env=SAN_ENV)
    assert "0 failures" in res.stdout


def test_abi_host_code_under_sanitizers(tmp_path):
    hipcc = "/opt/rocm/bin/hipcc"
    san = ["-O1", "-g", "-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=all"]
    flags = [f for f in B.HIPCC_FLAGS if f != "-O3"] + san

    def compile_unit(u):
        src, obj, extra = u
        out = str(tmp_path / os.path.basename(obj))
        _run([hipcc] + flags + extra + ["-c", src, "-o", out])
        return out

    jobs = min(16, len(os.sched_getaffinity(0)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_unit, B.units()))
    harness = str(tmp_path / "abi_harness.o")
    _run(["/opt/rocm/llvm/bin/clang++", "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"), "-c",
          os.path.join(HERE, "abi_harness.cpp"), "-o", harness])
    exe = str(tmp_path / "abi_san")
    _run([hipcc, "-Xarch_host", "-fsanitize=address,undefined", harness] + objs + ["-o", exe])
    res = _run([exe], env=SAN_ENV)
    assert " 0 failures" in res.stdout, res.stdout
