"""Register, LDS and private-memory use of every kernel in the library, from
the compiler's resource-usage remarks (-Rpass-analysis=kernel-resource-usage),
compiled here on the CPU from the same sources and flags as the library.

* No kernel may use private (scratch) memory: spilled registers go through
  it and cost memory traffic ("Optimizing GEMM in HIP", Step 6, register
  pressure and occupancy: the scratch size must remain zero; "FP16 GEMM
  Optimization on AMD RDNA 3 and RDNA 4", Step 1, measuring resources).  One
  named kernel pair keeps a single dword outside its stage loop; the
  ping-pong and FP8 TN kernels spill nothing at all, and SGPRs parked in
  VGPR lanes stay few.
* The LDS a four-wave kernel declares equals the size the host dispatch
  reports for it, and fits gfx950's 160 KiB.
* The figures of the kernels in a committed kernel trace
  (profiles/kernel_resources.md: rocprofv3 --kernel-trace, same sources) match
  the compiler's: LDS, scratch, and the VGPR field of the kernel
  descriptor.  gfx950 allocates the unified VGPR/AGPR file of a wave64 in
  granules of 8 registers and the descriptor stores the granule count; the
  trace prints that count times 4, half the registers actually allocated.
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


_DESC = re.compile(r"^\s*\.amdhsa_kernel\s+(\S+)(.*?)^\s*\.end_amdhsa_kernel", re.S | re.M)
_NEXT_VGPR = re.compile(r"\.amdhsa_next_free_vgpr\s+(\d+)")


def _remarks(unit, outdir):
    # Device-only compile to assembly: the remarks on stderr, the kernel
    # descriptors (.amdhsa_kernel blocks) in the output.
    src, obj, flags = unit
    out = os.path.join(outdir, os.path.basename(obj)[:-2] + ".s")
    cmd = (["/opt/rocm/bin/hipcc"] + B.HIPCC_FLAGS + flags +
           ["-Rpass-analysis=kernel-resource-usage", "--offload-device-only", "-S", src, "-o", out])
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    kernels, cur = {}, None
    for m in _REMARK.finditer(res.stderr):
        key, val = m.group(1), m.group(2)
        if key == "Function Name":
            cur = kernels.setdefault(val, {})
        elif cur is not None:
            cur[key.split(" [")[0]] = int(val) if val.lstrip("-").isdigit() else val
    with open(out) as f:
        for m in _DESC.finditer(f.read()):
            if m.group(1) in kernels:
                kernels[m.group(1)]["next_free_vgpr"] = int(_NEXT_VGPR.search(m.group(2)).group(1))
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
    assert all("next_free_vgpr" in u for u in usage.values())
    assert sum("gemm_tn_kernel" in n for n in names) >= 80
    assert any("gemm_f32_kernel" in n for n in names)
    assert any("gemm_skinny_kernel" in n for n in names)
    assert any("gemm_mfma_kernel" in n for n in names)


# The one kernel pair that still keeps a dword in private memory: the NN
# 16-bit 256 x 256 four-wave tile built with K-tail masks (its accumulators
# at the loop exit); the spill code sits outside the stage loop.  Any other
# kernel, or a larger spill here, fails.
_SCRATCH_ALLOWED = {
    "_ZN2dg14gemm_tn_kernelINS_5OpF16ELb1ELi256ELi256ELi2ELb1EEEvNS_8GemmArgsE": 8,
    "_ZN2dg14gemm_tn_kernelINS_6OpBF16ELb1ELi256ELi256ELi2ELb1EEEvNS_8GemmArgsE": 8,
}


def test_no_kernel_spills_to_scratch(usage):
    bad = {}
    for n, u in usage.items():
        allowed = _SCRATCH_ALLOWED.get(n, 0)
        if u.get("ScratchSize", 0) > allowed or (allowed == 0 and u.get("VGPRs Spill", 0) != 0):
            bad[n] = (u.get("ScratchSize"), u.get("VGPRs Spill"))
    assert not bad, f"kernels using scratch (bytes/lane, VGPR spills): {bad}"


def test_headline_kernels_spill_nothing(usage):
    # The eight-wave ping-pong kernels (TN 256 x 256) and the FP8 four-wave
    # TN 256 x 256 kernels: no scratch, no VGPR spills, no SGPRs parked in
    # VGPR lanes.
    heads = [n for n in usage if "gemm_pp_kernel" in n or
             re.search(r"gemm_tn_kernelINS_\d+Op(FP8|FP8S|MX8)ELb0ELi256ELi256", n)]
    assert len(heads) == 8 + 6
    for n in heads:
        u = usage[n]
        assert (u["ScratchSize"], u["VGPRs Spill"], u["SGPRs Spill"]) == (0, 0, 0), n


def test_sgpr_spills_stay_few(usage):
    # SGPRs parked in VGPR lanes (v_writelane / v_readlane, no memory) when a
    # kernel needs more than 102: a few, at the kernel's start and end.
    many = {n: u.get("SGPRs Spill") for n, u in usage.items() if u.get("SGPRs Spill", 0) > 16}
    assert not many, many


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
    """Rows of the committed trace summary, if it was taken on the current
    kernel sources (its "Sources hash"); otherwise none."""
    path = os.path.join(ROOT, "profiles", "kernel_resources.md")
    if not os.path.exists(path):
        return []
    import bench
    text = open(path).read()
    m = re.search(r"Sources hash: `([0-9a-f]+)`", text)
    if not m or m.group(1) != bench.kernel_source_hash():
        return []
    rows = []
    for line in text.splitlines():
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) == 6 and cells[0].startswith("_Z"):
            rows.append((cells[0], *[int(c) for c in cells[1:]]))
    return rows


def test_kernel_trace_matches_the_compiler(usage):
    rows = _trace_table()
    if not rows:
        pytest.skip("no kernel trace summary of the current kernel sources")
    for name, vgpr, agpr, lds, scratch, _sgpr in rows:
        assert name in usage, name
        u = usage[name]
        assert scratch == u["ScratchSize"] == 0, name
        assert lds == u["LDS Size"], name
        # gfx950 has one unified VGPR/AGPR file: the trace's accumulation
        # count stays 0 and the AGPRs are inside the VGPR granules.
        assert agpr == 0, name
        nfv = u["next_free_vgpr"]
        # The descriptor covers every VGPR and AGPR the compiler reports
        # (AGPRs start at a 4-aligned offset after the VGPRs).
        assert nfv >= (-(-u["VGPRs"] // 4) * 4 if u["AGPRs"] else u["VGPRs"]) + u["AGPRs"], name
        assert vgpr == -(-nfv // 8) * 4, (name, vgpr, nfv)


def test_bench_reads_power_and_clocks_from_amd_smi_text():
    """bench.py --sustain reads socket power and the per-XCD engine clocks
    from amd-smi's text; a layout it does not know gives None and []."""
    import bench
    txt = ("GPU: 0\n    POWER:\n        SOCKET_POWER: 1398 W\n        GFX_VOLTAGE: N/A\n    CLOCK:\n"
           "        GFX_0:\n            CLK: 1795 MHz\n            MIN_CLK: 500 MHz\n"
           "        GFX_1:\n            CLK: 1713 MHz\n            MIN_CLK: 500 MHz\n"
           "        MEM_0:\n            CLK: 2000 MHz\n")
    assert bench.parse_smi(txt) == (1398.0, [1795, 1713])
    assert bench.parse_smi("") == (None, [])


def test_fp8_kernels_use_the_unscaled_mfma():
    """The FP8 ping-pong kernels issue v_mfma_f32_16x16x128_f8f6f4 (the scale
    builtin with zero scale operands compiles to it) and no scaled MFMA."""
    u = [x for x in B.units() if os.path.basename(x[0]) == "pp.hip"][0]
    out = subprocess.run(["/opt/rocm/bin/hipcc"] + B.HIPCC_FLAGS + u[2] +
                         ["--offload-device-only", "-S", "-o", "-", "-c", u[0]],
                         capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stderr[-2000:]
    asm = out.stdout
    assert asm.count("v_mfma_f32_16x16x128_f8f6f4") > 0
    assert "v_mfma_scale_" not in asm
