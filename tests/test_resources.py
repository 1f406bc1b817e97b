"""Register, LDS and private-memory use of every kernel in the library, from
the compiler's resource-usage remarks (-Rpass-analysis=kernel-resource-usage),
compiled here on the CPU from the same sources and flags as the library.

* No kernel may use private (scratch) memory: spilled registers go through
  it and cost memory traffic inside the loop ("Optimizing GEMM in HIP", Step
  6, register pressure and occupancy: the scratch size must remain zero;
  "FP16 GEMM Optimization on AMD RDNA 3 and RDNA 4", Step 1, measuring
  resources).
* The LDS a four-wave kernel declares equals the size the host dispatch
  reports for it, and fits gfx950's 160 KiB.
* The figures of the kernels in a committed kernel trace
  (profiles/kernel_resources.md: rocprofv3 --kernel-trace, same sources) match
  the compiler's: VGPRs (allocation granularity 8), AGPRs, LDS and scratch.
"""

import concurrent.futures as cf
import os
import re
import subprocess

import pytest

from dense_gemm_02_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

_REMARK = re.compile(r"remark:\s+(Function Name|TotalSGPRs|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|"
                     r"LDS Size \[bytes/block\]|Occupancy \[waves/SIMD\]|VGPRs Spill|SGPRs Spill):\s+(\S+)")


def _remarks(unit, outdir):
    src, obj, flags = unit
    cmd = (["/opt/rocm/bin/hipcc"] + B.HIPCC_FLAGS + flags +
           ["-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", os.path.join(outdir, os.path.basename(obj))])
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    kernels, cur = {}, None
    for m in _REMARK.finditer(res.stderr):
        key, val = m.group(1), m.group(2)
        if key == "Function Name":
            cur = kernels.setdefault(val, {})
        elif cur is not None:
            cur[key.split(" [")[0]] = int(val) if val.lstrip("-").isdigit() else val
    return kernels


@pytest.fixture(scope="module")
def usage(tmp_path_factory):
    out = tmp_path_factory.mktemp("res")
    jobs = min(16, len(os.sched_getaffinity(0)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        parts = list(ex.map(lambda u: _remarks(u, str(out)), B.units()))
    allk = {}
    for p in parts:
        allk.update(p)
    return allk


def test_every_kernel_is_reported(usage):
    names = list(usage)
    assert sum("gemm_tn_kernel" in n for n in names) >= 80
    assert any("gemm_f32_kernel" in n for n in names)
    assert any("gemm_skinny_kernel" in n for n in names)
    assert any("gemm_mfma_kernel" in n for n in names)


def test_no_kernel_spills_to_scratch(usage):
    bad = {n: (u.get("ScratchSize"), u.get("VGPRs Spill"), u.get("SGPRs Spill")) for n, u in usage.items()
           if u.get("ScratchSize", 0) != 0 or u.get("VGPRs Spill", 0) != 0 or u.get("SGPRs Spill", 0) != 0}
    assert not bad, f"kernels using scratch (bytes/lane, VGPR spills, SGPR spills): {bad}"


_TN = re.compile(r"gemm_tn_kernelINS_\d+(Op\w+?)ELb([01])ELi(\d+)ELi(\d+)ELi(\d+)ELb([01])E")


def _tn_lds(op, bp, bq, ns):
    # (BP + BQ) rows of 128 bytes per stage, NS stages, plus the MX scale ring
    # (two groups of 16 bytes per row).
    lds = (bp + bq) * 128 * ns
    if op == "OpMX8":
        lds += 2 * 16 * (bp + bq)
    return lds


def test_four_wave_lds_matches_its_layout(usage):
    seen = 0
    for name, u in usage.items():
        m = _TN.search(name)
        if not m:
            continue
        op, _, bp, bq, ns, _ = m.groups()
        assert u["LDS Size"] == _tn_lds(op, int(bp), int(bq), int(ns)), name
        assert u["LDS Size"] <= 160 * 1024, name
        seen += 1
    assert seen >= 80


def _trace_table():
    path = os.path.join(ROOT, "profiles", "kernel_resources.md")
    if not os.path.exists(path):
        return []
    rows = []
    for line in open(path):
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) == 6 and cells[0].startswith("_Z"):
            rows.append((cells[0], *[int(c) for c in cells[1:]]))
    return rows


def test_kernel_trace_matches_the_compiler(usage):
    rows = _trace_table()
    if not rows:
        pytest.skip("no kernel trace summary committed")
    for name, vgpr, agpr, lds, scratch, _sgpr in rows:
        assert name in usage, name
        u = usage[name]
        assert scratch == u["ScratchSize"] == 0, name
        assert lds == u["LDS Size"], name
        assert agpr == u["AGPRs"], name
        assert vgpr == -(-u["VGPRs"] // 8) * 8, (name, vgpr, u["VGPRs"])
