"""GPU parity at sizes the oracle checks completely: every element of C from
the HIP path against the CPU oracle, through the C ABI.

Bars (per output format): bit-exact on +-1 and identity inputs; otherwise
max |c - c_ref| / sum_k |a b| <= 1e-6 (FP32), 2^-10 (FP16), 2^-7 (BF16, FP8
with FP32 output)."""

import numpy as np
import pytest

from dense_gemm_02_amd import inputs
from gpu_util import alloc_c, c_host, compare, pad_untouched, run_gpu, say, to_dev

pytestmark = pytest.mark.gpu

DIST = {"f32": "uniform", "f16": "normal", "bf16": "normal", "fp8": "uniform4"}
COMBOS = [("f32", "nn"), ("f32", "tn"), ("f16", "tn"), ("f16", "nn"), ("bf16", "tn"), ("bf16", "nn"),
          ("fp8", "tn"), ("fp8", "nn")]

# Edges of the block tiles (256 for 16/8-bit, 128 for FP32), the 32-wide MFMA
# tiles, the K stage (64 / 128 / 32 elements) and the 16-byte chunk.
EDGE = [1, 2, 3, 7, 8, 9, 15, 16, 17, 31, 32, 33, 63, 64, 65, 70, 127, 128, 129, 255, 256, 257]


def shapes_for(dtype, layout, n=28, seed=0):
    rng = np.random.default_rng(seed + 7 * len(dtype) + (layout == "nn"))
    out = [(1, 1, 1), (1, 1, 70), (70, 1, 1), (1, 70, 1), (257, 255, 129), (33, 65, 300)]
    for _ in range(n):
        out.append(tuple(int(rng.choice(EDGE)) for _ in range(3)))
    return out


def aligned_ld(n, dtype, extra=0):
    al = {"f32": 4, "f16": 8, "bf16": 8, "fp8": 16}[dtype]
    return ((max(n, 1) + al - 1) // al) * al + extra * al


def make_problem(dtype, layout, M, N, K, seed, dist=None, pad=0):
    la, lb, lc = inputs.min_ld(layout, M, N, K)
    lda = aligned_ld(la, dtype, pad)
    ldb = aligned_ld(lb, dtype, pad)
    return inputs.make(dtype, layout, M, N, K, seed, dist or DIST[dtype], lda=lda, ldb=ldb, ldc=lc + pad)


@pytest.mark.parametrize("dtype,layout", COMBOS)
def test_small_shapes_against_oracle(dtype, layout):
    for idx, (M, N, K) in enumerate(shapes_for(dtype, layout)):
        p = make_problem(dtype, layout, M, N, K, seed=1000 + idx, pad=idx % 3)
        say(f"case {dtype} {layout} M={M} N={N} K={K} lda={p.lda} ldb={p.ldb} ldc={p.ldc}")
        C = run_gpu(p)
        cij, pad = c_host(p, C)
        assert pad_untouched(pad, dtype), "kernel wrote outside the C matrix"
        ok, err, nbad = compare(p, cij)
        assert ok, f"{dtype} {layout} {(M, N, K)}: max err {err:.3e}, {nbad} bad"


@pytest.mark.parametrize("dtype,layout", COMBOS)
def test_multi_tile_ragged(dtype, layout):
    for idx, (M, N, K) in enumerate([(600, 520, 333), (515, 777, 1029), (1024, 256, 64)]):
        p = make_problem(dtype, layout, M, N, K, seed=2000 + idx, pad=1)
        say(f"case {dtype} {layout} M={M} N={N} K={K}")
        cij, pad = c_host(p, run_gpu(p))
        assert pad_untouched(pad, dtype)
        ok, err, nbad = compare(p, cij)
        assert ok, f"{dtype} {layout} {(M, N, K)}: max err {err:.3e}, {nbad} bad"


def kernel_name(dtype, layout, M, N, K):
    import ctypes
    from dense_gemm_02_amd import binding
    buf = ctypes.create_string_buffer(256)
    code = {"f32": 0, "f16": 1, "bf16": 2, "fp8": 3, "fp8s": 4, "mx8": 5}[dtype]
    assert binding.load_library().dgemm_kernel_config(code, 1 if layout == "tn" else 0, M, N, K, buf, 256) == 0
    return buf.value.decode()


# The four-wave kernel (K a multiple of the 16-byte chunk, at least two
# 128-byte stages; NN reads B through transposing LDS reads), with each block
# tile the shape table picks (and 128 x 128 with two and with four LDS
# stages, the latter also with fewer stages than buffers): exactly two stages, an odd stage count with edge
# tiles (N not a multiple of 8 in NN, so B's rows are padded and the last p
# tile reads past the row end), a partial last stage, and 400 tiles of
# 256 x 256, more than the CUs, also with a partial last stage
# (the kernels built with tail masks); then the one-round 192 tiles (TN
# 192 x 256 and 256 x 192, NN 256 x 192), a whole round and ragged ones with
# a partial last stage.
@pytest.mark.parametrize("dtype,layout", [(d, l) for d in ("f16", "bf16", "fp8") for l in ("tn", "nn")])
def test_four_wave_kernel(dtype, layout):
    bk = {"f16": 64, "bf16": 64, "fp8": 128}[dtype]
    fp8nn = (dtype, layout) == ("fp8", "nn")
    small = "256x128_w4" if fp8nn else "128x128_w4_s4"
    mid = "256x128_w4" if fp8nn else "128x128_w4"
    # the last two split into whole 256 x 256 rounds plus a second launch
    # (along q, then along p; TN splits only a last round under half full)
    psplit = (20480, 2560) if layout == "tn" else (4096, 14336)
    shapes = [(512, 512, 2 * bk, small), (300, 521, 3 * bk, small), (5120, 5120, 3 * bk, "256x256_w4"),
              (1000, 1100, 9 * bk + 16, small), (2048, 1800, 2 * bk + 16, small), (2560, 2304, 3 * bk, mid),
              (129, 77, 5 * bk + 16, small), (5120, 5120, 3 * bk + 16, "256x256_w4"),
              (4352, 4352, 3 * bk, "256x256_w4"), (psplit[0], psplit[1], 3 * bk + 16, "256x256_w4")]
    # NN runs p along N: the same shapes take 256 x 192 there (and the third
    # one 256 x 256).
    t192 = "192x256_w4" if layout == "tn" else "256x192_w4"
    q192 = "256x192_w4" if layout == "tn" else "256x256_w4"
    # TN takes the eight-wave ping-pong kernel where the table picks 256 x 256
    big = "256x256_pp" if layout == "tn" else "256x256_w4"
    shapes = [(M, N, K, big if t == "256x256_w4" else t) for M, N, K, t in shapes]
    shapes += [(1536, 8192, 4096, t192), (1500, 8000, 4096 + 16, t192), (8192, 1500, 4096 + 16, q192)]
    for idx, (M, N, K, tile) in enumerate(shapes):
        name = kernel_name(dtype, layout, M, N, K)
        k = name.split()[0]
        assert k.endswith(tile), name
        assert (" + " in name) == (idx in (8, 9)), name
        p = make_problem(dtype, layout, M, N, K, seed=5000 + idx, pad=idx % 2)
        say(f"case w4 {name} M={M} N={N} K={K}")
        cij, pad = c_host(p, run_gpu(p))
        assert pad_untouched(pad, dtype)
        ok, err, nbad = compare(p, cij)
        assert ok, f"{dtype} {layout} {(M, N, K)}: max err {err:.3e}, {nbad} bad"
    for idx, (M, N) in enumerate([(260, 300), (4096, 4096)]):
        p = make_problem(dtype, layout, M, N, 16 * bk, seed=5100 + idx, dist="pm1")
        say(f"case w4 pm1 {kernel_name(dtype, layout, M, N, 16 * bk)} M={M} N={N}")
        cij, _ = c_host(p, run_gpu(p))
        ok, _, nbad = compare(p, cij, exact=True)
        assert ok, f"pm1 {(M, N)}: {nbad} elements differ"


@pytest.mark.parametrize("dtype,layout", COMBOS)
def test_pm1_bit_exact(dtype, layout):
    for idx, (M, N, K) in enumerate([(300, 260, 1000), (64, 64, 4096), (257, 129, 77)]):
        p = make_problem(dtype, layout, M, N, K, seed=3000 + idx, dist="pm1")
        say(f"case pm1 {dtype} {layout} M={M} N={N} K={K}")
        cij, _ = c_host(p, run_gpu(p))
        ok, _, nbad = compare(p, cij, exact=True)
        assert ok, f"{nbad} elements differ"


# +-1 operands on the paths the cases above reach only with random data:
# every partial sum is an integer below 2^24, so FP32 accumulation is exact
# in any order and the output must equal the oracle bit for bit ("FP16 GEMM
# Optimization on AMD RDNA 3 and RDNA 4", What We Are Computing).  A dropped,
# doubled or misplaced stage, chunk or tile shows here even where the
# tolerance would hide it.  The kernel each case must reach is asserted.
PM1_PATHS = [
    # four-wave FP8 with the K-tail instantiation (K = 3 * 128 + 16)
    ("fp8", "tn", 5120, 5120, 400, "fp8_tn_256x256_pp", None),
    ("fp8", "nn", 5120, 5120, 400, "fp8_nn_256x256_w4", None),
    ("fp8", "tn", 600, 520, 400, "fp8_tn_128x128_w4_s4", None),
    ("fp8", "nn", 600, 520, 400, "fp8_nn_256x128_w4", None),
    # the one-round 192 tiles (K >= 4096), with and without a K tail
    ("bf16", "tn", 1536, 8192, 4096, "bf16_tn_192x256_w4", None),
    ("f16", "nn", 1536, 8192, 4096, "f16_nn_256x192_w4", None),
    ("fp8", "tn", 1536, 8192, 4096, "fp8_tn_192x256_w4", None),
    ("fp8", "tn", 8192, 1500, 4112, "fp8_tn_256x192_w4", None),
    ("bf16", "tn", 8192, 1500, 4104, "bf16_tn_256x192_w4", None),
    # split launches: whole 256 x 256 rounds plus a second launch along q / p
    ("bf16", "tn", 4352, 4352, 192, "bf16_tn_256x256_pp", "q"),
    ("bf16", "tn", 20480, 2560, 192, "bf16_tn_256x256_pp", "p"),
    ("fp8", "tn", 4352, 4352, 384, "fp8_tn_256x256_pp", "q"),
    ("fp8", "nn", 4096, 14336, 384, "fp8_nn_256x256_w4", "p"),
]


@pytest.mark.parametrize("dtype,layout,M,N,K,kern,split", PM1_PATHS,
                         ids=lambda v: str(v) if not isinstance(v, str) or len(v) < 12 else v.split("_", 2)[-1])
def test_pm1_bit_exact_paths(dtype, layout, M, N, K, kern, split):
    name = kernel_name(dtype, layout, M, N, K)
    assert name.split()[0] == kern, name
    assert (f" from {split}=" in name) if split else (" + " not in name), name
    p = make_problem(dtype, layout, M, N, K, seed=3100 + M % 97 + K, dist="pm1", pad=1)
    say(f"case pm1 path {name} M={M} N={N} K={K}")
    cij, pad = c_host(p, run_gpu(p))
    assert pad_untouched(pad, dtype)
    ok, _, nbad = compare(p, cij, exact=True)
    assert ok, f"{name}: {nbad} elements differ"


# Bit-for-bit repeatability, one case per kernel family, on random data and a
# side stream: an LDS race (a read before a copy lands, a copy over a buffer
# still being read) shows as two runs that differ.
DETERMINISM = [
    ("bf16", "tn", 5120, 5120, 512, None),       # 16-bit two-k-step stage, staged epilogue
    ("f16", "nn", 5120, 5120, 512, None),        # transposing reads of B
    ("fp8", "tn", 5120, 5120, 384, None),        # rolling FP8 stage
    ("fp8", "nn", 5120, 5120, 400, None),        # rolling stage, transposing reads, K tail
    ("fp8", "tn", 5120, 5120, 384, "scaled"),    # factors in the epilogue
    ("fp8", "tn", 3000, 3000, 4096, "mx"),       # MX scale ring, 192 x 256
    ("fp8", "nn", 5120, 5120, 1184, "mx"),       # MX scale ring, partial scale group
    ("bf16", "tn", 1536, 8192, 4096, None),      # 192 x 256, direct epilogue
    ("bf16", "tn", 1000, 1000, 2048, None),      # 128 x 128, four LDS stages
    ("bf16", "tn", 20480, 2560, 192, None),      # split launch along p
    ("bf16", "tn", 1000, 1000, 1001, None),      # eight-wave kernel, ragged K
    ("bf16", "tn", 16, 3000, 4096, None),        # skinny split-K, LDS reduction
    ("f32", "nn", 1000, 1000, 1000, None),       # FP32 MFMA kernel
]


@pytest.mark.parametrize("dtype,layout,M,N,K,variant", DETERMINISM)
def test_deterministic_per_kernel_family(dtype, layout, M, N, K, variant):
    import torch
    from dense_gemm_02_amd import binding
    p = make_problem(dtype, layout, M, N, K, seed=9100 + K)
    A, B = to_dev(p.A), to_dev(p.B)
    rng = np.random.default_rng(9)
    if variant == "scaled":
        sa = torch.from_numpy(_factors(rng, M)).cuda()
        sb = torch.from_numpy(_factors(rng, N)).cuda()
    elif variant == "mx":
        ld = ((K // 32 + 15) // 16) * 16
        sa = torch.from_numpy(mx_scales(rng, M, K // 32, ld).reshape(-1)).cuda()
        sb = torch.from_numpy(mx_scales(rng, N, K // 32, ld).reshape(-1)).cuda()
    kern = kernel_name({"scaled": "fp8s", "mx": "mx8"}.get(variant, dtype), layout, M, N, K)
    say(f"case determinism {kern} M={M} N={N} K={K}")
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    outs = []
    with torch.cuda.stream(s):
        for _ in range(2):
            C = alloc_c(p)
            if variant == "scaled":
                binding.gemm_scaled(layout, M, N, K, A, p.lda, B, p.ldb, C, p.ldc, sa, sb, stream=s)
            elif variant == "mx":
                binding.gemm_mx(layout, M, N, K, A, p.lda, B, p.ldb, C, p.ldc, sa, ld, sb, ld, stream=s)
            else:
                binding.gemm(dtype, layout, M, N, K, A, p.lda, B, p.ldb, C, p.ldc, stream=s)
            outs.append(C)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]), f"{kern}: two runs differ"


@pytest.mark.parametrize("dtype,layout", COMBOS)
def test_identity_bit_exact(dtype, layout):
    for n, M in ((256, 300), (100, 77)):
        p0 = make_problem(dtype, layout, M, n, n, seed=4000 + n)
        p = inputs.identity(dtype, layout, n, p0.A, p0.lda, ldb=aligned_ld(n, dtype))
        say(f"case identity {dtype} {layout} M={M} n={n}")
        cij, _ = c_host(p, run_gpu(p))
        a = p0.A[:, :n]
        if dtype == "fp8":
            from gpu_util import oracle
            assert np.array_equal(oracle.decode(oracle.F32, cij), oracle.decode(oracle.E4M3, a))
        else:
            from gpu_util import oracle
            assert oracle.bits_equal(cij, a, {"f32": oracle.F32, "f16": oracle.F16, "bf16": oracle.BF16}[dtype])


def _midpoint_problem(dtype, layout, seed):
    """Columns whose exact (and FP32) sums land on, or just beside, rounding
    midpoints of the output format: a = (1, 1, 1), b = (v, d, e) with v an
    output value, d a half or one-and-a-half output ulp of v, e tiny or 0."""
    import torch
    rng = np.random.default_rng(seed)
    N, K, M = 512, 3, 4
    frac = 10 if dtype == "f16" else 7
    e = rng.integers(-3, 6, N).astype(np.float64)     # keeps every term a normal number
    mant = rng.integers(0, 1 << frac, N).astype(np.float64)
    v = (1.0 + mant / 2.0 ** frac) * 2.0 ** e * rng.choice([-1.0, 1.0], N)
    ulp = 2.0 ** (e - frac)
    d = np.sign(v) * ulp * rng.choice([0.5, 1.5, -0.5], N)
    tiny = np.where(rng.random(N) < 0.3, np.sign(v) * ulp * 2.0 ** -6 * rng.choice([-1.0, 1.0], N), 0.0)
    bt = np.stack([v, d, tiny], axis=1)         # [N][K]
    def enc(x):
        if dtype == "f16":
            return x.astype(np.float16).view(np.uint16)
        return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    A = enc(np.ones((M, K)))
    if layout == "tn":
        B = enc(bt)
    else:
        B = enc(np.ascontiguousarray(bt.T))
    la, lb, lc = inputs.min_ld(layout, M, N, K)
    lda, ldb = aligned_ld(la, dtype), aligned_ld(lb, dtype)
    Ap = np.zeros((M, lda), np.uint16); Ap[:, :K] = A
    Bp = np.zeros((B.shape[0], ldb), np.uint16); Bp[:, :B.shape[1]] = B
    return inputs.Problem(dtype, layout, M, N, K, Ap, Bp, lda, ldb, lc)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("layout", ["tn", "nn"])
def test_epilogue_rounds_to_nearest_even(dtype, layout):
    p = _midpoint_problem(dtype, layout, seed=5 + len(dtype))
    cij, _ = c_host(p, run_gpu(p))
    ok, _, nbad = compare(p, cij, exact=True)
    assert ok, f"{nbad} outputs not rounded to nearest even"


def test_k_zero_writes_zeros_and_empty_is_noop():
    for dtype, layout in COMBOS:
        p = make_problem(dtype, layout, 70, 90, 0, seed=1)
        cij, pad = c_host(p, run_gpu(p))
        assert np.all(cij == 0) and pad_untouched(pad, dtype)
    # M = 0 / N = 0: nothing to write, the call must still succeed and touch nothing
    import torch
    from dense_gemm_02_amd import binding
    p = make_problem("bf16", "tn", 16, 16, 16, seed=1)
    A, B, C = to_dev(p.A), to_dev(p.B), alloc_c(p)
    binding.gemm("bf16", "tn", 0, 16, 16, A, 16, B, 16, C, 16)
    binding.gemm("bf16", "tn", 16, 0, 16, A, 16, B, 16, C, 16)
    torch.cuda.synchronize()
    assert bool((C == -1).all())


def test_deterministic_and_stream_ordered():
    import torch
    p = make_problem("bf16", "tn", 1000, 1000, 2000, seed=9)
    A, B = to_dev(p.A), to_dev(p.B)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        C1 = run_gpu(p, A=A, B=B, stream=s, sync=False)
        C2 = run_gpu(p, A=A, B=B, stream=s, sync=False)
    torch.cuda.synchronize()
    assert torch.equal(C1, C2)
    ok, err, _ = compare(p, c_host(p, C1)[0])
    assert ok, err


def test_concurrent_calls_from_threads_and_streams():
    # Host threads calling the library at once, each on its own stream (the
    # binding drops the interpreter lock inside the C calls): every result
    # must match the oracle, as the planning state is per call and the
    # diagnostics per thread.
    import threading
    import torch
    cases = [("bf16", "tn", 1000, 900, 700), ("fp8", "tn", 600, 1300, 512), ("f16", "nn", 800, 700, 300),
             ("f32", "nn", 700, 500, 260), ("bf16", "nn", 16, 3000, 4096), ("fp8", "nn", 5120, 2048, 256)]
    probs = [make_problem(d, l, M, N, K, seed=14000 + i) for i, (d, l, M, N, K) in enumerate(cases)]
    devs = [(to_dev(p.A), to_dev(p.B), alloc_c(p)) for p in probs]
    streams = [torch.cuda.Stream() for _ in probs]
    torch.cuda.synchronize()
    errors = []

    def work(i):
        try:
            p, (A, B, C), st = probs[i], devs[i], streams[i]
            for _ in range(3):
                run_gpu(p, A=A, B=B, C=C, stream=st, sync=False)
        except Exception as e:  # noqa: BLE001 -- reported below
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(probs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for p, (_, _, C) in zip(probs, devs):
        cij, pad = c_host(p, C)
        assert pad_untouched(pad, p.dtype)
        ok, err, nbad = compare(p, cij)
        assert ok, f"{p.dtype} {p.layout} {(p.M, p.N, p.K)}: max err {err:.3e}, {nbad} bad"


def test_calls_captured_in_a_hip_graph():
    # The library allocates nothing and issues only kernel launches on the
    # caller's stream, so its calls can be captured: a graph holding a split
    # launch (BF16 TN 4352 x 4352, two kernels), an FP8 call and a skinny call
    # is replayed three times with new operands copied in eagerly between the
    # replays; every replay must equal an eager run on the same operands bit
    # for bit.
    import torch
    from dense_gemm_02_amd import binding
    cases = [("bf16", "tn", 4352, 4352, 192), ("fp8", "tn", 1000, 1100, 640), ("bf16", "tn", 16, 3000, 4096)]
    assert " + " in kernel_name("bf16", "tn", 4352, 4352, 192)
    probs = [[make_problem(d, l, M, N, K, seed=15000 + 10 * i + r) for r in range(3)]
             for i, (d, l, M, N, K) in enumerate(cases)]
    bufs = [(to_dev(ps[0].A), to_dev(ps[0].B), alloc_c(ps[0])) for ps in probs]

    def calls():
        for ps, (A, B, C) in zip(probs, bufs):
            p = ps[0]
            binding.gemm(p.dtype, p.layout, p.M, p.N, p.K, A, p.lda, B, p.ldb, C, p.ldc)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()                      # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    torch.cuda.synchronize()
    for r in range(3):
        for ps, (A, B, C) in zip(probs, bufs):
            A.copy_(to_dev(ps[r].A))
            B.copy_(to_dev(ps[r].B))
            C.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for ps, (A, B, C) in zip(probs, bufs):
            eager = run_gpu(ps[r], A=A, B=B)
            assert torch.equal(C, eager), (ps[r].dtype, ps[r].M, ps[r].N, ps[r].K, r)
            cij, pad = c_host(ps[r], C)
            ok, err, nbad = compare(ps[r], cij)
            assert ok, f"replay {r} {(ps[r].M, ps[r].N, ps[r].K)}: max err {err:.3e}, {nbad} bad"


def test_odd_ldc_scalar_store_path():
    for dtype in ("bf16", "f16", "fp8", "f32"):
        p = make_problem(dtype, "tn", 301, 133, 200, seed=11)
        p.ldc = 303        # odd: columns start at every alignment
        cij, pad = c_host(p, run_gpu(p))
        assert pad_untouched(pad, dtype)
        ok, err, nbad = compare(p, cij)
        assert ok, (dtype, err, nbad)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_skinny_split_k_path(dtype):
    # TN with at most 32 rows of A runs the split-K skinny kernel: K is cut
    # into 8 slices of whole 128-k steps whose boundaries and tail chunks
    # must all line up.
    idx = 0
    for M in (1, 5, 16, 17, 31, 32):
        for N in (1, 33, 300):
            for K in (1, 7, 8, 31, 33, 127, 128, 129, 255, 1000, 1032, 2049):
                p = make_problem(dtype, "tn", M, N, K, seed=6000 + idx, pad=idx % 2)
                idx += 1
                cij, pad = c_host(p, run_gpu(p))
                assert pad_untouched(pad, dtype)
                ok, err, nbad = compare(p, cij)
                assert ok, f"{dtype} {(M, N, K)}: max err {err:.3e}, {nbad} bad"
    p = make_problem(dtype, "tn", 16, 700, 4096, seed=7, dist="pm1")
    cij, _ = c_host(p, run_gpu(p))
    assert compare(p, cij, exact=True)[0]


# ---- FP8 with scale factors (gemm_fp8_scaled) --------------------------------

def _factors(rng, n, pow2=False):
    e = rng.integers(-8, 9, n)
    m = np.ones(n) if pow2 else rng.uniform(1.0, 2.0, n)
    return (m * 2.0 ** e * rng.choice([-1.0, 1.0], n)).astype(np.float32)


def run_scaled(p, sa, sb):
    import torch
    from dense_gemm_02_amd import binding
    C = alloc_c(p)
    binding.gemm_scaled(p.layout, p.M, p.N, p.K, to_dev(p.A), p.lda, to_dev(p.B), p.ldb, C, p.ldc,
                        torch.from_numpy(sa).cuda(), torch.from_numpy(sb).cuda())
    torch.cuda.synchronize()
    return C


def compare_scaled(p, cij, sa, sb, rows=None, exact=False):
    from gpu_util import oracle
    c_ref, sab = oracle.gemm_fp8_scaled(oracle.NN if p.layout == "nn" else oracle.TN, p.M, p.N, p.K, p.A, p.lda,
                                        p.B, p.ldb, sa, sb, rows=rows)
    got = cij if rows is None else cij[np.asarray(rows)]
    if exact:
        return oracle.bits_equal(got, c_ref, oracle.F32), 0.0
    ok, err, _ = oracle.check(got, c_ref, sab, oracle.F32, oracle.TOL["fp8"])
    return ok, err


# Every kernel the FP8 path can pick (the eight-wave kernel for ragged K, the
# four-wave tiles, 256 x 256 with 400 tiles, 192 x 256 in TN), per-tensor
# and per-row factors, K = 0 (C = 0 * factors).  Tolerance relative to
# |sa_i sb_j| * sum_k |a b|.
@pytest.mark.parametrize("layout", ["tn", "nn"])
@pytest.mark.parametrize("mode", ["tensor", "row"])
def test_fp8_scaled_against_oracle(layout, mode):
    rng = np.random.default_rng(6000 + (layout == "nn") + 2 * (mode == "row"))
    shapes = [(1, 1, 1), (257, 129, 77), (33, 65, 300), (300, 521, 384), (512, 512, 256), (1000, 1100, 1168),
              (5120, 5120, 384), (5120, 5120, 400), (70, 90, 0), (4352, 4352, 384), (20480, 2560, 384)
              if layout == "tn" else (4096, 14336, 384), (1500, 8000, 4096 + 16)]
    for idx, (M, N, K) in enumerate(shapes):
        p = make_problem("fp8", layout, M, N, K, seed=6100 + idx, pad=idx % 2)
        sa = _factors(rng, M if mode == "row" else 1)
        sb = _factors(rng, N if mode == "row" else 1)
        say(f"case scaled {kernel_name('fp8s', layout, M, N, K)} mode={mode} M={M} N={N} K={K}")
        cij, pad = c_host(p, run_scaled(p, sa, sb))
        assert pad_untouched(pad, "fp8")
        ok, err = compare_scaled(p, cij, sa, sb)
        assert ok, f"{layout} {mode} {(M, N, K)}: max err {err:.3e}"


# +-1 operands and power-of-two factors: every result is exact, so the
# output must match the oracle bit for bit; unit factors must reproduce
# gemm_fp8's own output.
@pytest.mark.parametrize("layout", ["tn", "nn"])
def test_fp8_scaled_bit_exact(layout):
    rng = np.random.default_rng(6200 + (layout == "nn"))
    for idx, (M, N, K) in enumerate([(260, 300, 2048), (4096, 4096, 512), (77, 50, 100)]):
        p = make_problem("fp8", layout, M, N, K, seed=6300 + idx, dist="pm1")
        sa, sb = _factors(rng, M, pow2=True), _factors(rng, N, pow2=True)
        say(f"case scaled pm1 {layout} M={M} N={N} K={K}")
        cij, _ = c_host(p, run_scaled(p, sa, sb))
        ok, _ = compare_scaled(p, cij, sa, sb, exact=True)
        assert ok, f"{(M, N, K)}: not bit-exact"
        one = np.float32([1.0])
        c1, _ = c_host(p, run_scaled(p, one, one))
        c0, _ = c_host(p, run_gpu(p))
        assert np.array_equal(c1, c0)


# The binding must leave one HIP runtime in the process whichever is touched
# first: a fresh interpreter loads the library before using torch, then runs
# a small GEMM through it.
def test_library_loaded_before_torch_use():
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = (
        "from dense_gemm_02_amd import binding\n"
        "binding.load_library()\n"
        "import torch\n"
        "a = torch.ones(64, 64, dtype=torch.float32, device='cuda')\n"
        "c = torch.empty(64, 64, dtype=torch.float32, device='cuda')\n"
        "binding.gemm('f32', 'nn', 64, 64, 64, a, 64, a, 64, c, 64)\n"
        "torch.cuda.synchronize()\n"
        "assert bool((c == 64).all())\n"
        "print('ok', flush=True)\n")
    say("case fresh process: library loaded before torch use")
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=180)
    assert r.returncode == 0 and "ok" in r.stdout, r.stdout + r.stderr


# ---- MXFP8 with E8M0 block scales (gemm_mxfp8) -------------------------------

def mx_scales(rng, rows, nb, ld, lo=112, hi=143):
    """rows x ld scale bytes: nb random E8M0 codes per row, the padding 255
    (the format's NaN), which no call may read."""
    s = np.full((max(rows, 1), ld), 255, np.uint8)
    s[:, :nb] = rng.integers(lo, hi, (max(rows, 1), nb))
    return s


def run_mx(p, SA, ldsa, SB, ldsb):
    import torch
    from dense_gemm_02_amd import binding
    C = alloc_c(p)
    binding.gemm_mx(p.layout, p.M, p.N, p.K, to_dev(p.A), p.lda, to_dev(p.B), p.ldb, C, p.ldc,
                    torch.from_numpy(SA.reshape(-1)).cuda(), ldsa, torch.from_numpy(SB.reshape(-1)).cuda(), ldsb)
    torch.cuda.synchronize()
    return C


def compare_mx(p, cij, SA, ldsa, SB, ldsb, rows=None, exact=False):
    from gpu_util import oracle
    c_ref, sab = oracle.gemm_mxfp8(oracle.NN if p.layout == "nn" else oracle.TN, p.M, p.N, p.K, p.A, p.lda, p.B,
                                   p.ldb, SA.reshape(-1), ldsa, SB.reshape(-1), ldsb, rows=rows)
    got = cij if rows is None else cij[np.asarray(rows)]
    if exact:
        return oracle.bits_equal(got, c_ref, oracle.F32), 0.0
    ok, err, _ = oracle.check(got, c_ref, sab, oracle.F32, oracle.TOL["fp8"])
    return ok, err


# Every tile the MXFP8 path picks: one or two stages (K < 256), a partial
# last stage whose scale dword reaches past K/32, 256 x 256 with 400 tiles
# (and with tiles of one scale group, K = 384), K = 0, padded scale rows full
# of NaN codes, launches split along q and p.
# Scales 2^-15 .. 2^15.
@pytest.mark.parametrize("layout", ["tn", "nn"])
def test_mxfp8_against_oracle(layout):
    rng = np.random.default_rng(7000 + (layout == "nn"))
    shapes = [(1, 1, 32), (33, 65, 96), (257, 129, 224), (300, 521, 384), (512, 512, 256), (1000, 1100, 1184),
              (5120, 5120, 384), (70, 90, 0), (4352, 4352, 384), (14336, 4096, 384) if layout == "tn" else
              (4096, 14336, 384), (5120, 5120, 1184), (1500, 8000, 4096 + 32), (8192, 1500, 4096)]
    for idx, (M, N, K) in enumerate(shapes):
        p = make_problem("fp8", layout, M, N, K, seed=7100 + idx, pad=idx % 2)
        nb = K // 32
        ld = ((nb + 15) // 16) * 16 + 16 * (idx % 2)
        SA, SB = mx_scales(rng, M, nb, ld), mx_scales(rng, N, nb, ld)
        say(f"case mx {kernel_name('mx8', layout, M, N, K)} M={M} N={N} K={K} ld={ld}")
        cij, pad = c_host(p, run_mx(p, SA, ld, SB, ld))
        assert pad_untouched(pad, "fp8")
        ok, err = compare_mx(p, cij, SA, ld, SB, ld)
        assert ok, f"{layout} {(M, N, K)}: max err {err:.3e}"


# +-1 operands with scales 2^-3 .. 2^3: every partial sum is exact in FP32,
# so the output matches the oracle bit for bit; unit scales reproduce
# gemm_fp8 where both take the same four-wave tile.
@pytest.mark.parametrize("layout", ["tn", "nn"])
def test_mxfp8_bit_exact(layout):
    rng = np.random.default_rng(7200 + (layout == "nn"))
    for idx, (M, N, K) in enumerate([(260, 300, 2048), (4096, 4096, 512), (77, 50, 160)]):
        p = make_problem("fp8", layout, M, N, K, seed=7300 + idx, dist="pm1")
        nb = K // 32
        ld = ((nb + 15) // 16) * 16
        SA, SB = mx_scales(rng, M, nb, ld, 124, 131), mx_scales(rng, N, nb, ld, 124, 131)
        say(f"case mx pm1 {layout} M={M} N={N} K={K}")
        cij, _ = c_host(p, run_mx(p, SA, ld, SB, ld))
        ok, _ = compare_mx(p, cij, SA, ld, SB, ld, exact=True)
        assert ok, f"{(M, N, K)}: not bit-exact"
        if K >= 256:
            one = np.full((max(M, N), ld), 127, np.uint8)
            c1, _ = c_host(p, run_mx(p, one[:M], ld, one[:N], ld))
            c0, _ = c_host(p, run_gpu(p))
            assert np.array_equal(c1, c0)


# The tensor-level face: layouts read from strides, against the oracle.
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "fp8"])
def test_matmul_tensor_api(dtype):
    import torch
    from dense_gemm_02_amd import matmul
    from gpu_util import oracle
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}[dtype]
    for layout in ("nn", "tn"):
        M, N, K = 200, 136, 320
        p = make_problem(dtype, layout, M, N, K, seed=8000 + (layout == "tn"))
        A = to_dev(p.A).view(tdt) if dtype != "fp8" else to_dev(p.A).view(tdt)
        B = to_dev(p.B).view(tdt)
        a = A.view(-1)[: M * p.lda].view(M, p.lda)[:, :K]
        if layout == "nn":
            b = B.view(-1)[: K * p.ldb].view(K, p.ldb)[:, :N]
        else:
            b = B.view(-1)[: N * p.ldb].view(N, p.ldb)[:, :K].t()
        say(f"case matmul {dtype} {layout}")
        c = matmul(a, b)
        torch.cuda.synchronize()
        assert c.shape == (M, N)
        bits = c.contiguous().view(torch.int32 if c.element_size() == 4 else torch.int16).cpu().numpy()
        cij = bits.view(np.uint32) if c.element_size() == 4 else bits.view(np.uint16)
        ok, err, nbad = compare(p, np.ascontiguousarray(cij))
        assert ok, f"{dtype} {layout}: max err {err:.3e}"
    # scale factors through the same face
    if dtype == "fp8":
        sa = torch.full((M,), 0.5, device="cuda")
        sb = torch.full((N,), 4.0, device="cuda")
        c2 = matmul(a, b, scale_a=sa, scale_b=sb)
        torch.cuda.synchronize()
        assert torch.equal(c2, 2.0 * matmul(a, b))


# Maximum sizes: leading dimensions at the 32-bit descriptor limit (the bytes
# one block tile spans stay below 2^31), operands placed in the first K (NN B:
# N) columns of huge device rows; the oracle sees the compact problem.
@pytest.mark.parametrize("dtype,layout", [("bf16", "tn"), ("fp8", "tn"), ("bf16", "nn"), ("fp8", "nn")])
def test_leading_dimensions_at_the_descriptor_limit(dtype, layout):
    import torch
    from dense_gemm_02_amd import binding
    e = {"bf16": 2, "fp8": 1}[dtype]
    bk = 128 // e
    M, N, K = 300, 280, 3 * bk
    p = make_problem(dtype, layout, M, N, K, seed=8100)
    limit = (1 << 31) - 64
    al = 16 // e
    big_q = ((limit // (256 * e)) // al) * al               # K-contiguous operand: 256 rows per block
    lda = big_q
    ldb = big_q if layout == "tn" else ((limit // (K * e)) // al) * al   # NN B: K rows per block
    assert 256 * lda * e <= limit and (256 * ldb * e <= limit if layout == "tn" else K * ldb * e <= limit)
    tdt = torch.uint8 if e == 1 else torch.int16
    A = torch.zeros((M, lda), dtype=tdt, device="cuda")
    A[:, :K] = to_dev(p.A).view(M, p.lda)[:, :K]
    if layout == "tn":
        B = torch.zeros((N, ldb), dtype=tdt, device="cuda")
        B[:, :K] = to_dev(p.B).view(N, p.ldb)[:, :K]
    else:
        B = torch.zeros((K, ldb), dtype=tdt, device="cuda")
        B[:, :N] = to_dev(p.B).view(K, p.ldb)[:, :N]
    C = alloc_c(p)
    say(f"case limit {dtype} {layout} lda={lda} ldb={ldb}")
    binding.gemm(dtype, layout, M, N, K, A, lda, B, ldb, C, p.ldc)
    torch.cuda.synchronize()
    cij, pad = c_host(p, C)
    assert pad_untouched(pad, dtype)
    ok, err, nbad = compare(p, cij)
    assert ok, f"max err {err:.3e}, {nbad} bad"
    del A, B
    torch.cuda.empty_cache()


# Long K: 2^18 + 16 (4097 stages of the 16-bit kernels, 2049 of FP8, a K
# tail), +-1 inputs so that every sum is an exact integer below 2^24: the
# whole output bit for bit, on both layouts.
@pytest.mark.parametrize("dtype,layout", [("bf16", "tn"), ("fp8", "tn"), ("f16", "nn"), ("fp8", "nn")])
def test_long_k_bit_exact(dtype, layout):
    K = (1 << 18) + 16
    p = make_problem(dtype, layout, 300, 260, K, seed=16000, dist="pm1")
    say(f"case long K {kernel_name(dtype, layout, 300, 260, K)} K={K}")
    cij, pad = c_host(p, run_gpu(p))
    assert pad_untouched(pad, dtype)
    ok, _, nbad = compare(p, cij, exact=True)
    assert ok, f"{dtype} {layout} K={K}: {nbad} elements differ"


# Random shapes, pitches and C placements: M, N up to 700 and K up to 1500
# (log-uniform, so single tiles, ragged edges and several rounds all occur),
# A and B pitches padded by 0-3 16-byte units, C's pitch by 0-5 elements and
# its base 0-7 elements past an allocation; the whole output against the
# oracle, the padding and the storage around C untouched.
@pytest.mark.parametrize("dtype,layout", COMBOS)
def test_random_shapes_pitches_and_offsets(dtype, layout):
    import torch
    from dense_gemm_02_amd import binding
    rng = np.random.default_rng(12000 + COMBOS.index((dtype, layout)))
    for idx in range(12):
        M, N = (int(np.exp(rng.uniform(0, np.log(700)))) for _ in range(2))
        K = int(np.exp(rng.uniform(0, np.log(1500))))
        la, lb, lc = inputs.min_ld(layout, M, N, K)
        lda = aligned_ld(la, dtype, int(rng.integers(0, 4)))
        ldb = aligned_ld(lb, dtype, int(rng.integers(0, 4)))
        ldc = lc + int(rng.integers(0, 6))
        off = int(rng.integers(0, 8))
        p = inputs.make(dtype, layout, M, N, K, 12100 + idx, DIST[dtype], lda=lda, ldb=ldb, ldc=ldc)
        rows = N if layout == "tn" else M
        tdt = torch.int32 if dtype in ("f32", "fp8") else torch.int16
        flat = torch.full((off + rows * ldc + 8,), -1, dtype=tdt, device="cuda")
        C = flat[off:off + rows * ldc].view(rows, ldc)
        say(f"case random {kernel_name(dtype, layout, M, N, K)} M={M} N={N} K={K} ld={lda},{ldb},{ldc} off={off}")
        binding.gemm(dtype, layout, M, N, K, to_dev(p.A), lda, to_dev(p.B), ldb, C, ldc)
        torch.cuda.synchronize()
        f = flat.cpu().numpy()
        assert np.all(f[:off] == -1) and np.all(f[off + rows * ldc:] == -1), "wrote outside C"
        cij, pad = c_host(p, C)
        assert pad_untouched(pad, dtype)
        ok, err, nbad = compare(p, cij)
        assert ok, f"{dtype} {layout} {(M, N, K, lda, ldb, ldc, off)}: max err {err:.3e}, {nbad} bad"


# Larger random shapes (M, N from 700 to 6000, K from 100 to 5000): several
# rounds, part-filled last rounds, split launches and the one-round tiles at
# random sizes, with padded pitches; whole outputs against the oracle's
# full-size form.
@pytest.mark.parametrize("dtype,layout", COMBOS)
def test_random_large_shapes(dtype, layout):
    rng = np.random.default_rng(13000 + COMBOS.index((dtype, layout)))
    for idx in range(3):
        M, N = (int(np.exp(rng.uniform(np.log(700), np.log(6000)))) for _ in range(2))
        K = int(np.exp(rng.uniform(np.log(100), np.log(5000))))
        p = make_problem(dtype, layout, M, N, K, seed=13100 + idx, pad=int(rng.integers(0, 3)))
        say(f"case random large {kernel_name(dtype, layout, M, N, K)} M={M} N={N} K={K}")
        cij, pad = c_host(p, run_gpu(p))
        assert pad_untouched(pad, dtype)
        ok, err, nbad = compare(p, cij)
        assert ok, f"{dtype} {layout} {(M, N, K)}: max err {err:.3e}, {nbad} bad"


# The same for the scaled entry points: random shapes and pitches, per-tensor
# or per-row factors (gemm_fp8_scaled) and E8M0 block scales with a padded
# scale pitch (gemm_mxfp8, K a multiple of 32), whole outputs.
@pytest.mark.parametrize("layout", ["tn", "nn"])
def test_random_shapes_scaled_and_mx(layout):
    rng = np.random.default_rng(12500 + (layout == "nn"))
    for idx in range(10):
        M, N = (int(np.exp(rng.uniform(0, np.log(700)))) for _ in range(2))
        K = int(np.exp(rng.uniform(0, np.log(1500))))
        la, lb, lc = inputs.min_ld(layout, M, N, K)
        lda = aligned_ld(la, "fp8", int(rng.integers(0, 4)))
        ldb = aligned_ld(lb, "fp8", int(rng.integers(0, 4)))
        ldc = lc + int(rng.integers(0, 6))
        p = inputs.make("fp8", layout, M, N, K, 12600 + idx, DIST["fp8"], lda=lda, ldb=ldb, ldc=ldc)
        row = bool(rng.integers(0, 2))
        sa, sb = _factors(rng, M if row else 1), _factors(rng, N if row else 1)
        say(f"case random scaled {kernel_name('fp8s', layout, M, N, K)} M={M} N={N} K={K} per_row={row}")
        cij, pad = c_host(p, run_scaled(p, sa, sb))
        assert pad_untouched(pad, "fp8")
        ok, err = compare_scaled(p, cij, sa, sb)
        assert ok, f"scaled {layout} {(M, N, K, lda, ldb, ldc)}: max err {err:.3e}"
        Km = 32 * max(1, K // 32)
        pm = inputs.make("fp8", layout, M, N, Km, 12700 + idx, DIST["fp8"],
                         lda=aligned_ld(inputs.min_ld(layout, M, N, Km)[0], "fp8", int(rng.integers(0, 4))),
                         ldb=aligned_ld(inputs.min_ld(layout, M, N, Km)[1], "fp8", int(rng.integers(0, 4))),
                         ldc=inputs.min_ld(layout, M, N, Km)[2] + int(rng.integers(0, 6)))
        nb = Km // 32
        ld = ((nb + 15) // 16) * 16 + 16 * int(rng.integers(0, 2))
        SA, SB = mx_scales(rng, M, nb, ld), mx_scales(rng, N, nb, ld)
        say(f"case random mx {kernel_name('mx8', layout, M, N, Km)} M={M} N={N} K={Km} ld={ld}")
        cij, pad = c_host(pm, run_mx(pm, SA, ld, SB, ld))
        assert pad_untouched(pad, "fp8")
        ok, err = compare_mx(pm, cij, SA, ld, SB, ld)
        assert ok, f"mx {layout} {(M, N, Km, ld)}: max err {err:.3e}"


# Grids of extreme aspect: one row of 4096 tiles along q (N = 2^20) and one
# column of 1024 tiles along p (M = 2^18), K two stages: the tile scheduler's
# spread over the XCDs and its grouping with a single tile on one axis, and
# workgroup indices far past one round, against the whole oracle output.
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_extreme_aspect_grids(dtype):
    import torch
    bk = 128 if dtype == "fp8" else 64
    for idx, (M, N) in enumerate([(256, 1 << 20), (1 << 18, 256), (250, (1 << 20) - 3)]):
        K = 2 * bk
        p = make_problem(dtype, "tn", M, N, K, seed=9800 + idx)
        say(f"case aspect {kernel_name(dtype, 'tn', M, N, K)} M={M} N={N} K={K}")
        cij, pad = c_host(p, run_gpu(p))
        assert pad_untouched(pad, dtype)
        ok, err, nbad = compare(p, cij)
        assert ok, f"{dtype} {(M, N, K)}: max err {err:.3e}, {nbad} bad"
        del cij, pad
        torch.cuda.empty_cache()


# The tensor-level calls refuse, before any launch, device tensors too small
# for what the call would read or write, and host, float64 or strided scale
# factors.
def test_binding_rejects_bad_device_tensors():
    import torch
    from dense_gemm_02_amd import binding, matmul
    M, N, K = 64, 48, 256
    A = torch.zeros(M * K, dtype=torch.int16, device="cuda")
    B = torch.zeros(N * K, dtype=torch.int16, device="cuda")
    C = torch.zeros(N * M, dtype=torch.int16, device="cuda")
    binding.gemm("bf16", "tn", M, N, K, A, K, B, K, C, M)

    def short(n):
        return torch.zeros(n, dtype=torch.int16, device="cuda")

    # (a view counts the storage behind it: a slice of A still covers A)
    for a, b, c in ((short(M * K - 1), B, C), (A, short(N * K - 8), C), (A, B, short(N * M - 1)),
                    (A[1:], B, C)):
        with pytest.raises(ValueError):
            binding.gemm("bf16", "tn", M, N, K, a, K, b, K, c, M)
    a8 = torch.zeros((M, K), dtype=torch.uint8, device="cuda").view(torch.float8_e4m3fn)
    b8 = torch.zeros((N, K), dtype=torch.uint8, device="cuda").view(torch.float8_e4m3fn).t()
    good = torch.ones(M, device="cuda")
    for bad in (torch.ones(M), torch.ones(M, dtype=torch.float64, device="cuda"),
                torch.ones(2 * M, device="cuda")[::2]):
        with pytest.raises(TypeError):
            matmul(a8, b8, scale_a=bad, scale_b=torch.ones(1, device="cuda"))
    with pytest.raises(ValueError):
        matmul(a8, b8, scale_a=good[:5], scale_b=torch.ones(1, device="cuda"))
    c32 = torch.zeros(M * N, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        binding.gemm_mx("tn", M, N, K, a8.view(torch.uint8).reshape(-1), K, b8.t().contiguous().view(torch.uint8),
                        K, c32, M, torch.zeros(M * 16 - 1, dtype=torch.uint8, device="cuda"), 16,
                        torch.zeros(N * 16, dtype=torch.uint8, device="cuda"), 16)
    torch.cuda.synchronize()


# The clock trace (diagnostics): each workgroup of a traced four-wave launch
# records stamps whose ratio is an engine clock in a plausible range; the
# result is unchanged, and the trace is off again afterwards.
def test_clock_trace_reports_the_engine_clock():
    import torch
    from dense_gemm_02_amd import binding
    p = make_problem("bf16", "tn", 1024, 768, 512, seed=77)
    A, B = to_dev(p.A), to_dev(p.B)
    grid = int(kernel_name("bf16", "tn", 1024, 768, 512).split("grid=")[1].split()[0])
    buf = torch.zeros(4 * grid + 4, dtype=torch.int64, device="cuda")
    say(f"case clock trace grid={grid}")
    C0 = run_gpu(p, A=A, B=B)
    binding.trace_clock(buf)
    try:
        C1 = run_gpu(p, A=A, B=B)
    finally:
        binding.trace_clock(None)
    assert torch.equal(C0, C1)
    mhz = binding.traced_clock_mhz(buf, grid)
    assert np.all((mhz > 300.0) & (mhz < 3000.0)), mhz
    assert int(buf[4 * grid:].abs().sum()) == 0, "wrote past the requested workgroups"
    buf.zero_()
    run_gpu(p, A=A, B=B)
    assert int(buf.abs().sum()) == 0, "trace still on"
    with pytest.raises(TypeError):
        binding.trace_clock(torch.zeros(8, dtype=torch.int32, device="cuda"))


# The eight-wave ping-pong kernel (gemm_pp.hpp), forced through DGEMM_CONFIG:
# single and partial tiles, several rounds of 256 x 256 tiles, K tails
# (copies with per-lane masks), +-1 bit-exact, repeatable bit for bit, and
# FP8 with per-row scale factors.
@pytest.mark.parametrize("dtype", ["f16", "bf16", "fp8"])
def test_ping_pong_kernel(dtype, monkeypatch):
    import torch
    bk = 128 if dtype == "fp8" else 64
    name = f"{dtype}_tn_256x256_pp"
    monkeypatch.setenv("DGEMM_CONFIG", name)
    shapes = [(256, 256, 2 * bk), (16, 16, 2 * bk), (1, 1, 2 * bk + 16), (300, 521, 2 * bk), (600, 520, 4 * bk),
              (129, 77, 5 * bk + 16), (1000, 1100, 9 * bk + 16), (5120, 5120, 3 * bk), (5120, 5120, 3 * bk + 16),
              (2048, 2048, 64 * bk)]
    for idx, (M, N, K) in enumerate(shapes):
        kern = kernel_name(dtype, "tn", M, N, K)
        assert kern.startswith(name + " "), kern
        p = make_problem(dtype, "tn", M, N, K, seed=9300 + idx, pad=idx % 2)
        say(f"case pp {kern} M={M} N={N} K={K}")
        cij, pad = c_host(p, run_gpu(p))
        assert pad_untouched(pad, dtype)
        ok, err, nbad = compare(p, cij)
        assert ok, f"{name} {(M, N, K)}: max err {err:.3e}, {nbad} bad"
    for idx, (M, N, K) in enumerate([(4096, 4096, 16 * bk), (1000, 1100, 9 * bk + 16)]):
        p = make_problem(dtype, "tn", M, N, K, seed=9400 + idx, dist="pm1")
        say(f"case pp pm1 {name} M={M} N={N} K={K}")
        cij, _ = c_host(p, run_gpu(p))
        ok, _, nbad = compare(p, cij, exact=True)
        assert ok, f"{name} pm1 {(M, N, K)}: {nbad} elements differ"
    p = make_problem(dtype, "tn", 5120, 5120, 4 * bk, seed=9500)
    A, B = to_dev(p.A), to_dev(p.B)
    say(f"case pp determinism {name}")
    assert torch.equal(run_gpu(p, A=A, B=B), run_gpu(p, A=A, B=B))


def test_ping_pong_scaled_fp8(monkeypatch):
    monkeypatch.setenv("DGEMM_CONFIG", "fp8s_tn_256x256_pp")
    rng = np.random.default_rng(9600)
    for idx, (M, N, K) in enumerate([(1000, 1100, 1168), (5120, 5120, 384)]):
        kern = kernel_name("fp8s", "tn", M, N, K)
        assert kern.startswith("fp8s_tn_256x256_pp "), kern
        p = make_problem("fp8", "tn", M, N, K, seed=9610 + idx)
        sa, sb = _factors(rng, M), _factors(rng, N)
        say(f"case pp scaled {kern} M={M} N={N} K={K}")
        cij, pad = c_host(p, run_scaled(p, sa, sb))
        assert pad_untouched(pad, "fp8")
        ok, err = compare_scaled(p, cij, sa, sb)
        assert ok, f"{(M, N, K)}: max err {err:.3e}"


# The four-wave kernel's TN 256 x 256 tile (the eight-wave kernel serves that
# tile by default; the four-wave one stays reachable through DGEMM_CONFIG and
# serves MXFP8), with and without a K tail, +-1 bit-exact.
@pytest.mark.parametrize("dtype", ["f16", "bf16", "fp8"])
def test_four_wave_256_tn_forced(dtype, monkeypatch):
    bk = 128 if dtype == "fp8" else 64
    name = f"{dtype}_tn_256x256_w4"
    monkeypatch.setenv("DGEMM_CONFIG", name)
    for idx, (M, N, K, dist) in enumerate([(5120, 5120, 3 * bk, None), (1000, 1100, 9 * bk + 16, None),
                                           (4096, 4096, 16 * bk, "pm1")]):
        kern = kernel_name(dtype, "tn", M, N, K)
        assert kern.startswith(name + " "), kern
        p = make_problem(dtype, "tn", M, N, K, seed=9700 + idx, dist=dist, pad=idx % 2)
        say(f"case w4 forced {kern} M={M} N={N} K={K}")
        cij, pad = c_host(p, run_gpu(p))
        assert pad_untouched(pad, dtype)
        ok, err, nbad = compare(p, cij, exact=dist == "pm1")
        assert ok, f"{name} {(M, N, K)}: max err {err:.3e}, {nbad} bad"


# Both FP32 tiles on both layouts at ragged multi-tile shapes: the default
# choice (64 x 64 below half a chip of 128 x 128 tiles) and the other tile
# forced through DGEMM_CONFIG, with +-1 inputs bit-exact.
@pytest.mark.parametrize("layout", ["nn", "tn"])
@pytest.mark.parametrize("tile", ["64x64", "128x128"])
def test_f32_tiles_forced(layout, tile, monkeypatch):
    name = f"f32_{layout}_{tile}"
    monkeypatch.setenv("DGEMM_CONFIG", name)
    for idx, (M, N, K, dist) in enumerate([(300, 200, 77, None), (257, 129, 1029, None), (520, 600, 96, "pm1")]):
        kern = kernel_name("f32", layout, M, N, K)
        assert kern.startswith(name + " "), kern
        p = make_problem("f32", layout, M, N, K, seed=9800 + idx, dist=dist, pad=idx % 2)
        say(f"case f32 forced {kern} M={M} N={N} K={K}")
        cij, pad = c_host(p, run_gpu(p))
        assert pad_untouched(pad, "f32")
        ok, err, nbad = compare(p, cij, exact=dist == "pm1")
        assert ok, f"{name} {(M, N, K)}: max err {err:.3e}, {nbad} bad"


# C rows off the 16-byte grid: a C base 2..14 bytes past a 16-byte boundary
# with a 16-byte pitch (every row equally off), and an odd pitch (every
# offset), for the 16-bit outputs; the storage around C stays untouched.
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_c_rows_off_the_16_byte_grid(dtype):
    import torch
    from dense_gemm_02_amd import binding
    for idx, (M, N, K, ldc, off) in enumerate([(600, 300, 256, 608, 1), (600, 300, 256, 608, 7),
                                               (515, 260, 320, 515, 0), (1000, 77, 192, 1001, 3)]):
        p = make_problem(dtype, "tn", M, N, K, seed=9900 + idx)
        p.ldc = ldc
        say(f"case C off-grid {dtype} M={M} N={N} K={K} ldc={ldc} offset={off}")
        flat = torch.full((off + N * ldc + 8,), -1, dtype=torch.int16, device="cuda")
        C = flat[off:off + N * ldc].view(N, ldc)
        binding.gemm(p.dtype, p.layout, M, N, K, to_dev(p.A), p.lda, to_dev(p.B), p.ldb, C, ldc)
        torch.cuda.synchronize()
        f = flat.cpu().numpy().view(np.uint16)
        assert np.all(f[:off] == 0xFFFF) and np.all(f[off + N * ldc:] == 0xFFFF), "wrote outside C"
        cij, pad = c_host(p, C)
        assert pad_untouched(pad, dtype)
        ok, err, nbad = compare(p, cij)
        assert ok, f"{dtype} {(M, N, K, ldc, off)}: max err {err:.3e}, {nbad} bad"
