"""Benchmark of the dense GEMM hot path on one MI355X.

One step = one C = A x B through the C ABI (host dispatch, tile scheduler,
buffer loads, swizzled LDS, MFMA pipeline, converting epilogue) on inputs
already resident in HBM.  Default workload: FP16 TN, M = N = K = 8192,
A and B i.i.d. N(0,1)/sqrt(K) rounded to FP16 (seed 3), FP32 accumulation,
FP16 output.  BF16 TN and FP8 E4M3 TN at the same size are timed in the
same run and reported under "per_dtype".

Timing: the workload back to back for --settle-ms of wall time (the chip's
power controller dips after an idle spell and recovers over 50-100
launches), W untimed warm-up steps, then exactly K steps between two
synchronisations, with HIP events recorded on the stream the kernels run on
(one before each launch, so the mean, min and median per launch are
known).  TFLOP/s = 2*M*N*K / t.  After the timed region one more launch runs
with the library's clock trace on, which gives the engine clock the kernel
ran at (per workgroup, median); each throughput is also given as a fraction
of the MFMA peak at that clock.  Prints one JSON line.

cpu_baseline: the CPU oracle (test infrastructure, never tuned) timed on
whole output rows of the same workload, as many as fit about 25 s (all of
them when the host is fast enough), on every core the process may use; its
rate is scaled to TFLOP/s of useful work.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GEMM TFLOP/s + % of dense MFMA peak (FP16/BF16/FP8, M=N=K=8192)"
# MI355X published dense peaks (TFLOP/s) and HBM bandwidth (GB/s).
PEAK_TFLOPS = {"f16": 2516.6, "bf16": 2516.6, "fp8": 5033.2, "f32": 157.3}
HBM_GBS = 8000.0
# Engine clock the published MFMA peaks assume (MHz).
PEAK_CLOCK_MHZ = 2400.0
WORKLOADS = {
    "f16": ("f16", "tn", 8192, 8192, 8192, 3, "normal"),
    "bf16": ("bf16", "tn", 8192, 8192, 8192, 4, "normal"),
    "fp8": ("fp8", "tn", 8192, 8192, 8192, 5, "uniform4"),
}
# Other workload configurations, timed with --workload (not part of the
# default line).  The skinny BF16 case is HBM-bound: B is rotated over
# ROTATE copies (> 256 MB Infinity Cache + L2) so each launch reads it from HBM.
# An eighth field selects a variant of the FP8 call: "scaled" (per-row FP32
# factors for A and B, gemm_fp8_scaled) or "mx" (E8M0 block scales,
# gemm_mxfp8).
EXTRA = {
    "bf16_tn_16x8192x8192": ("bf16", "tn", 16, 8192, 8192, 4, "normal"),
    "bf16_tn_4096x14336x4096": ("bf16", "tn", 4096, 14336, 4096, 4, "normal"),
    "bf16_tn_4096x4096x14336": ("bf16", "tn", 4096, 4096, 14336, 4, "normal"),
    "bf16_tn_8191x8190x8200": ("bf16", "tn", 8191, 8190, 8200, 4, "normal"),
    "fp8_tn_4096x14336x4096": ("fp8", "tn", 4096, 14336, 4096, 5, "uniform4"),
    "fp8_tn_4096x4096x14336": ("fp8", "tn", 4096, 4096, 14336, 5, "uniform4"),
    "fp8_tn_8192x28672x8192": ("fp8", "tn", 8192, 28672, 8192, 5, "uniform4"),
    "f32_nn_4096x4096x4096": ("f32", "nn", 4096, 4096, 4096, 1, "uniform"),
    "f32_nn_256x256x256": ("f32", "nn", 256, 256, 256, 0, "uniform"),
    "bf16_nn_8192x8192x8192": ("bf16", "nn", 8192, 8192, 8192, 4, "normal"),
    "fp8_nn_8192x8192x8192": ("fp8", "nn", 8192, 8192, 8192, 5, "uniform4"),
    "fp8_tn_8192x8192x8192_scaled": ("fp8", "tn", 8192, 8192, 8192, 5, "uniform4", "scaled"),
    "fp8_tn_8192x8192x8192_mx": ("fp8", "tn", 8192, 8192, 8192, 5, "uniform4", "mx"),
    "bf16_tn_2048x2048x2048": ("bf16", "tn", 2048, 2048, 2048, 4, "normal"),
    "bf16_tn_3072x4096x8192": ("bf16", "tn", 3072, 4096, 8192, 4, "normal"),
    "bf16_tn_8192x10240x8192": ("bf16", "tn", 8192, 10240, 8192, 4, "normal"),
}
ROTATE = 4
DTYPE_NAME = {"f16": "f16", "bf16": "bf16", "fp8": "fp8 (e4m3) x fp8 -> f32", "f32": "f32"}


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "dense_gemm_02_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".hpp", ".h")):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str):
    """HBM bytes per launch measured with rocprofv3 counters, if they were
    taken on the current kernel sources; otherwise None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    w = t.get("workloads", {}).get(workload)
    return None if w is None else float(w["hbm_bytes_per_launch"])


def make_inputs(dtype, spec=None):
    import torch
    from dense_gemm_02_amd import inputs
    dt, layout, M, N, K, seed, dist = (spec or WORKLOADS[dtype])[:7]
    p = inputs.make(dt, layout, M, N, K, seed, dist)

    def dev(x):
        x = np.ascontiguousarray(x)
        v = {np.dtype(np.uint32): np.int32, np.dtype(np.uint16): np.int16, np.dtype(np.uint8): np.uint8}[x.dtype]
        return torch.from_numpy(x.view(v)).cuda()

    A, B = dev(p.A), dev(p.B)
    out32 = dt in ("f32", "fp8")
    C = torch.empty((N, p.ldc) if layout == "tn" else (M, p.ldc),
                    dtype=torch.int32 if out32 else torch.int16, device="cuda")
    return p, A, B, C


def time_gemm(dtype, steps, warmup, spec=None, rotate=1, made=None, settle_ms=0.0):
    import torch
    from dense_gemm_02_amd import binding
    p, A, B, C = made if made is not None else make_inputs(dtype, spec)
    print(f"[bench] {p.dtype} {p.layout} {p.M}x{p.N}x{p.K}: operands on the device, launching", file=sys.stderr,
          flush=True)
    Bs = [B] + [B.clone() for _ in range(rotate - 1)]
    stream = torch.cuda.current_stream()
    it = [0]
    variant = spec[7] if spec is not None and len(spec) > 7 else None
    rng = np.random.default_rng(11)
    if variant == "scaled":
        # per-row factors in [0.5, 2)
        sa = torch.from_numpy(rng.uniform(0.5, 2.0, p.M).astype(np.float32)).cuda()
        sb = torch.from_numpy(rng.uniform(0.5, 2.0, p.N).astype(np.float32)).cuda()
    elif variant == "mx":
        # E8M0 codes 2^-7 .. 2^7, K/32 per row
        ld = ((p.K // 32 + 15) // 16) * 16
        sa = torch.from_numpy(rng.integers(120, 135, (p.M, ld)).astype(np.uint8)).cuda()
        sb = torch.from_numpy(rng.integers(120, 135, (p.N, ld)).astype(np.uint8)).cuda()

    def step():
        b = Bs[it[0] % len(Bs)]
        it[0] += 1
        if variant == "scaled":
            binding.gemm_scaled(p.layout, p.M, p.N, p.K, A, p.lda, b, p.ldb, C, p.ldc, sa, sb, stream=stream)
        elif variant == "mx":
            binding.gemm_mx(p.layout, p.M, p.N, p.K, A, p.lda, b, p.ldb, C, p.ldc, sa, ld, sb, ld, stream=stream)
        else:
            binding.gemm(p.dtype, p.layout, p.M, p.N, p.K, A, p.lda, b, p.ldb, C, p.ldc, stream=stream)

    # Settle: the workload back to back for settle_ms of wall time before the
    # warm-up steps.  After an idle spell the chip's power controller first
    # lets the clock run high, then pulls it below its steady value and only
    # recovers over the next 50-100 launches (launches 3-10 of a cold start
    # run up to 35% slower than steady state, profiles/warmup_transient_8192.md);
    # the timed region is meant to see the steady state.
    settle_n, t_s = 0, time.perf_counter()
    while settle_ms > 0 and (time.perf_counter() - t_s) * 1e3 < settle_ms:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
        settle_n += 10
    settle_wall = (time.perf_counter() - t_s) * 1e3
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # The timed region: K launches back to back between two events (mean =
    # its length / K).  An event recorded between launches costs the stream
    # a few microseconds, so the per-launch spread (min, median, max) comes
    # from a second pass of K launches with an event before each one; those
    # figures include that cost.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    for i in range(steps):
        ev[i].record(stream)
        step()
    ev[steps].record(stream)
    torch.cuda.synchronize()
    each = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    flops = p.flops
    res = {"ms_per_launch": ms, "tflops": flops / (ms * 1e-3) / 1e12, "wall_s": wall,
           "settle_launches": settle_n, "settle_ms": round(settle_wall, 1),
           "min_ms": each[0], "median_ms": each[len(each) // 2] if steps % 2 else
           0.5 * (each[steps // 2 - 1] + each[steps // 2]), "max_ms": each[-1]}
    res["clock_mhz"] = engine_clock(step, stream, kernel_grid(p))
    return p, res


def kernel_grid(p):
    """Workgroups of the main launch of this workload (from the library's
    own description of the launch)."""
    import ctypes
    import re
    from dense_gemm_02_amd import binding
    code = {"f32": 0, "f16": 1, "bf16": 2, "fp8": 3}[p.dtype]
    buf = ctypes.create_string_buffer(512)
    binding.load_library().dgemm_kernel_config(code, 1 if p.layout == "tn" else 0, p.M, p.N, p.K, buf, 512)
    m = re.search(r"grid=(\d+)", buf.value.decode())
    return int(m.group(1)) if m else 1


def engine_clock(step, stream, grid):
    """Engine clock (MHz) the GEMM itself ran at: one more launch of the timed
    workload (after the timed region) with the library's clock trace on;
    each workgroup's core-clock ticks over its real-time ticks (100 MHz),
    median over the workgroups."""
    import numpy as np
    import torch
    from dense_gemm_02_amd import binding
    buf = torch.zeros(4 * grid, dtype=torch.int64, device="cuda")
    torch.cuda.synchronize()
    binding.trace_clock(buf)
    try:
        step()
        torch.cuda.synchronize()
    finally:
        binding.trace_clock(None)
    mhz = binding.traced_clock_mhz(buf, grid)
    mhz = mhz[np.isfinite(mhz)]
    return float(np.median(mhz)) if mhz.size else None


def cpu_baseline(dtype, target_s=25.0, full_s=60.0):
    """The oracle (never tuned) on the headline workload, timed wall-clock on
    every core this process may run on.  A short run on 256 rows measures its
    rate; if the whole product is estimated at full_s seconds or less it is
    computed in one timed call, otherwise as many whole output rows as fit
    about target_s seconds, so the default bench stays within minutes on
    hosts where the full product would take longer."""
    import oracle
    from dense_gemm_02_amd import inputs
    dt, layout, M, N, K, seed, dist = WORKLOADS[dtype]
    p = inputs.make(dt, layout, M, N, K, seed, dist)
    fmt = {"f32": oracle.F32, "f16": oracle.F16, "bf16": oracle.BF16, "fp8": oracle.E4M3}[dt]
    lay = oracle.TN if layout == "tn" else oracle.NN
    cores = len(os.sched_getaffinity(0))
    rng = np.random.default_rng(0)
    probe = np.sort(rng.choice(M, min(M, 256), replace=False))
    t0 = time.perf_counter()
    oracle.gemm(fmt, lay, M, N, K, p.A, p.lda, p.B, p.ldb, rows=probe, threads=cores)
    per_row = (time.perf_counter() - t0) / len(probe)
    nrows = M if per_row * M <= full_s else int(min(M, max(64, target_s / max(per_row, 1e-6))))
    rows = None if nrows >= M else np.sort(rng.choice(M, nrows, replace=False))
    t0 = time.perf_counter()
    oracle.gemm(fmt, lay, M, N, K, p.A, p.lda, p.B, p.ldb, rows=rows, threads=cores)
    dt_s = time.perf_counter() - t0
    nrows = M if rows is None else nrows
    flops = 2.0 * nrows * N * K
    what = ("the full product" if rows is None else
            f"{nrows} of {M} output rows (all {N} columns, K={K}; the full product would take "
            f"~{per_row * M:.0f} s)")
    return {"value": flops / dt_s / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{what} of {dtype} {layout} {M}x{N}x{K}, {dt_s:.1f} s wall on {cores} threads"}


def run_tool(name, *args):
    """stdout of a ROCm command-line tool (PATH, then /opt/rocm/bin), or ""."""
    import shutil
    import subprocess
    exe = shutil.which(name) or os.path.join("/opt/rocm/bin", name)
    try:
        return subprocess.run([exe, *args], capture_output=True, text=True, timeout=20).stdout
    except (OSError, subprocess.SubprocessError):
        return ""


def parse_smi(txt):
    """Socket power (W) and per-XCD engine clocks (MHz) from the text of
    `amd-smi metric -p -c`; None / [] where a field is missing."""
    import re
    m = re.search(r"SOCKET_POWER:\s*(\d+(?:\.\d+)?)\s*W", txt)
    clocks = [int(c) for _, c in re.findall(r"GFX_(\d+):\s*\n\s*CLK:\s*(\d+)\s*MHz", txt)]
    return (float(m.group(1)) if m else None), clocks


def smi_sample():
    return parse_smi(run_tool("amd-smi", "metric", "-p", "-c"))


def power_cap_w():
    import re
    txt = run_tool("rocm-smi", "-M")
    m = re.search(r"Max Graphics Package Power \(W\):\s*([\d.]+)", txt)
    return float(m.group(1)) if m else None


def sustain(dtype, seconds, made):
    """One workload launched back to back for `seconds` of wall time; over the
    second half, a few samples of socket power and per-XCD engine clocks.
    Shows whether the chip runs at its power cap while the GEMM runs."""
    import threading
    import torch
    from dense_gemm_02_amd import binding
    p, A, B, C = made
    stream = torch.cuda.current_stream()
    samples = []
    stop = threading.Event()

    def sampler():
        if stop.wait(seconds / 2):
            return
        while not stop.is_set():
            samples.append(smi_sample())
            stop.wait(1.0)

    th = threading.Thread(target=sampler, daemon=True)
    for _ in range(20):
        binding.gemm(p.dtype, p.layout, p.M, p.N, p.K, A, p.lda, B, p.ldb, C, p.ldc, stream=stream)
    torch.cuda.synchronize()
    th.start()
    t0 = time.perf_counter()
    n = 0
    last = t0
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            binding.gemm(p.dtype, p.layout, p.M, p.N, p.K, A, p.lda, B, p.ldb, C, p.ldc, stream=stream)
        torch.cuda.synchronize()
        n += 20
        if time.perf_counter() - last > 2.0:
            last = time.perf_counter()
            print(f"[bench] sustain {dtype}: {last - t0:.0f} s, {n} launches", file=sys.stderr, flush=True)
    el = time.perf_counter() - t0
    stop.set()
    th.join()
    tf = p.flops * n / el / 1e12
    pw = [s[0] for s in samples if s[0] is not None]
    return {"sustain": f"{p.dtype}_{p.layout}_{p.M}x{p.N}x{p.K}", "seconds": round(el, 2), "launches": n,
            "tflops": round(tf, 1), "frac_of_peak": round(tf / PEAK_TFLOPS[dtype], 4),
            "socket_power_w": pw, "power_cap_w": power_cap_w(),
            "xcd_clock_mhz": [s[1] for s in samples if s[1]]}


def transient(dtype, n, made):
    """Per-launch durations (us) of the first n launches of one workload after
    3 s of idle, one event before each launch."""
    import torch
    from dense_gemm_02_amd import binding
    p, A, B, C = made
    stream = torch.cuda.current_stream()
    f = lambda: binding.gemm(p.dtype, p.layout, p.M, p.N, p.K, A, p.lda, B, p.ldb, C, p.ldc, stream=stream)
    f()
    torch.cuda.synchronize()
    time.sleep(3.0)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    for i in range(n):
        ev[i].record(stream)
        f()
    ev[n].record(stream)
    torch.cuda.synchronize()
    us = [round(ev[i].elapsed_time(ev[i + 1]) * 1e3, 1) for i in range(n)]
    return {"transient": f"{p.dtype}_{p.layout}_{p.M}x{p.N}x{p.K}", "launch_us": us}


def timing_fields(r, peak=None):
    """Per-launch statistics and the measured engine clock; with a peak, the
    throughput as a fraction of the peak at that clock (the published peak
    scaled by measured clock / 2400 MHz)."""
    out = {"mean_ms": round(r["ms_per_launch"], 5), "min_ms": round(r["min_ms"], 5),
           "median_ms": round(r["median_ms"], 5), "max_ms": round(r["max_ms"], 5),
           "settle_launches": r["settle_launches"], "settle_ms": r["settle_ms"],
           "clock_mhz": None if r["clock_mhz"] is None else round(r["clock_mhz"], 1)}
    if peak is not None and r["clock_mhz"]:
        at = peak * r["clock_mhz"] / PEAK_CLOCK_MHZ
        out["peak_at_clock"] = round(at, 1)
        out["frac_at_clock"] = round(r["tflops"] / at, 4)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--dtype", default="f16", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", action="store_true", help="time only --dtype")
    ap.add_argument("--workload", default=None, choices=sorted(EXTRA),
                    help="time one other workload configuration instead (prints its own line)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="instead of the GEMM, run a plain device copy of MIB MiB three times "
                         "(reference dispatch for the HBM byte counters)")
    ap.add_argument("--settle-ms", type=float, default=150.0, metavar="MS",
                    help="before each format's warm-up steps, run its workload back to back for MS of wall time "
                         "(the power controller's transient after idle; 0: none)")
    ap.add_argument("--transient", type=int, default=0, metavar="N",
                    help="instead of the timed region, time each of the first N launches of each format after "
                         "3 s of idle (no settle, no warm-up)")
    ap.add_argument("--sustain", type=float, default=0, metavar="SECONDS",
                    help="instead of the timed region, launch each format's workload back to back for SECONDS "
                         "and sample socket power and engine clocks (amd-smi) over the second half")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(see the sharding note in DESIGN.md); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from dense_gemm_02_amd import binding
    binding.load_library()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU: torch sees none", file=sys.stderr, flush=True)
        sys.exit(3)
    print(f"[bench] device: {torch.cuda.get_device_name(0)}", file=sys.stderr, flush=True)
    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n}), flush=True)
        return

    if args.workload and args.sustain:
        spec = EXTRA[args.workload]
        print(json.dumps(sustain(spec[0], args.sustain, make_inputs(spec[0], spec))), flush=True)
        return
    if args.workload:
        spec = EXTRA[args.workload]
        skinny = spec[2] <= 32
        p, r = time_gemm(spec[0], args.steps, args.warmup, spec=spec, rotate=ROTATE if skinny else 1,
                         settle_ms=args.settle_ms)
        out_b = 4 if spec[0] in ("f32", "fp8") else 2
        in_b = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1}[spec[0]]
        nbytes = (p.M * p.K + p.N * p.K) * in_b + p.M * p.N * out_b
        gbs = nbytes / (r["ms_per_launch"] * 1e-3) / 1e9
        roof = ({"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_GBS, "unit": "GB/s",
                 "frac": round(gbs / HBM_GBS, 4), "traffic": load_traffic(args.workload)} if skinny else
                {"bound": "mfma", "achieved": round(r["tflops"], 2), "peak": PEAK_TFLOPS[spec[0]], "unit": "TFLOP/s",
                 "frac": round(r["tflops"] / PEAK_TFLOPS[spec[0]], 4), "traffic": load_traffic(args.workload)})
        print(json.dumps({"workload": args.workload, "value": round(r["tflops"], 2), "unit": "TFLOP/s",
                          "ms_per_launch": round(r["ms_per_launch"], 5), "steps": args.steps,
                          "timing": timing_fields(r, None if skinny else PEAK_TFLOPS[spec[0]]),
                          "warmup": args.warmup, "rotated_B_copies": ROTATE if skinny else 1,
                          "roofline": roof}), flush=True)
        return

    # Every format's operands are made and resident on the device before the
    # first timed launch, so no host-side input generation separates the
    # timed regions.
    order = [args.dtype] + ([] if args.only else [d for d in WORKLOADS if d != args.dtype])
    if args.sustain:
        for d in order:
            print(json.dumps(sustain(d, args.sustain, make_inputs(d))), flush=True)
            torch.cuda.empty_cache()
        return
    if args.transient:
        for d in order:
            print(json.dumps(transient(d, args.transient, make_inputs(d))), flush=True)
            torch.cuda.empty_cache()
        return
    made = {d: make_inputs(d) for d in order}
    p, head = time_gemm(args.dtype, args.steps, args.warmup, made=made[args.dtype], settle_ms=args.settle_ms)
    print(f"[bench] {args.dtype}: {head['ms_per_launch']:.4f} ms/launch, {head['tflops']:.1f} TFLOP/s, "
          f"min {head['min_ms']:.4f} median {head['median_ms']:.4f} ms, clock {head['clock_mhz']} MHz",
          file=sys.stderr, flush=True)
    per = {}
    if not args.only:
        for d in WORKLOADS:
            if d == args.dtype:
                continue
            _, r = time_gemm(d, args.steps, args.warmup, made=made.pop(d), settle_ms=args.settle_ms)
            per[d] = {"tflops": round(r["tflops"], 1), "ms_per_launch": round(r["ms_per_launch"], 4),
                      "frac_of_peak": round(r["tflops"] / PEAK_TFLOPS[d], 4), **timing_fields(r, PEAK_TFLOPS[d])}
            print(f"[bench] {d}: {r['ms_per_launch']:.4f} ms/launch, {r['tflops']:.1f} TFLOP/s, "
                  f"min {r['min_ms']:.4f} median {r['median_ms']:.4f} ms, clock {r['clock_mhz']} MHz",
                  file=sys.stderr, flush=True)

    workload = f"{p.dtype}_{p.layout}_{p.M}x{p.N}x{p.K}"
    traffic = load_traffic(workload)
    roof = {"bound": "mfma", "achieved": round(head["tflops"], 2), "peak": PEAK_TFLOPS[args.dtype],
            "unit": "TFLOP/s", "frac": round(head["tflops"] / PEAK_TFLOPS[args.dtype], 4),
            "traffic": traffic}
    cpu = None if args.no_cpu_baseline else cpu_baseline(args.dtype)
    line = {
        "metric": METRIC,
        "value": round(head["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_launch"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic",
        "config": {"workload": workload, "M": p.M, "N": p.N, "K": p.K, "layout": p.layout,
                   "inputs": f"{p.meta['dist']} seed {p.meta['seed']}", "accumulate": "f32",
                   "kernel_sources": kernel_source_hash()},
        "roofline": roof,
        "timing": timing_fields(head, PEAK_TFLOPS[args.dtype]),
        "cpu_baseline": cpu,
        "per_dtype": per,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
