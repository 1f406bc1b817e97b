"""Pins for the CPU oracle: checks against things other than the oracle itself.

The pages print no worked numeric example of C, so the oracle is pinned by
what mathematics and library routines fix:

* exhaustive codec decoding against numpy / torch casts (every bit pattern);
* round-to-nearest-even encoding against numpy / torch casts, and against an
  exact-rational rounding where the library rounds twice;
* brute force against exact rationals (``fractions.Fraction``) on tiny shapes,
  every format and layout, with padded leading dimensions;
* closed forms (all ones, alternating signs, rank one);
* the identity invariant B = I => C = A ("Optimizing GEMM in HIP", note at the
  top of the tutorial: every step is validated against B = I);
* the +-1 invariant: every partial sum is an integer, so the result is exact
  and must equal an integer matrix product ("FP16 GEMM Optimization on AMD
  RDNA 3 and RDNA 4", section "What We Are Computing"; "FP8 GEMM Optimization
  on AMD RDNA 4", section "Results");
* FP8 exactness: E4M3 values are multiples of 2^-9, so scaled integer matrix
  products give the exact sum;
* thread-count independence and equality with the unblocked triple loop;
* FP8 with scale factors: exact rationals s_ij * sa_i * sb_j rounded once,
  a rank-one closed form, and reduction to the plain product at unit factors;
* MXFP8 block scales: E8M0 decoding, exact rationals with per-block powers of
  two, a closed form that fixes the block width and which operand each
  scale belongs to, and reduction to the plain product at unit scales;
* sensitivity: a transposed operand, a dropped term or a wrong sign each make
  a pin fail (and for the factors: reversed rows, a lost sign, a missing
  factor).
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from dense_gemm_02_amd import inputs

FMT = {"f32": oracle.F32, "f16": oracle.F16, "bf16": oracle.BF16, "fp8": oracle.E4M3}
LAY = {"nn": oracle.NN, "tn": oracle.TN}


# ---- independent library decoders -----------------------------------------

def lib_decode(dtype, bits):
    bits = np.asarray(bits)
    if dtype == "f32":
        return bits.astype(np.uint32).view(np.float32).astype(np.float64)
    if dtype == "f16":
        return bits.astype(np.uint16).view(np.float16).astype(np.float64)
    t = torch.from_numpy(np.ascontiguousarray(bits))
    if dtype == "bf16":
        return t.view(torch.bfloat16).to(torch.float64).numpy()
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def frac_rne(q: Fraction, P: int, emin: int, emax: int) -> float:
    """Exact-rational round-to-nearest-even onto a binary format with P
    significand bits, normal exponents [emin, emax], gradual underflow."""
    if q == 0:
        return 0.0
    sgn = -1.0 if q < 0 else 1.0
    a = abs(q)
    E = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** E > a:
        E -= 1
    while Fraction(2) ** (E + 1) <= a:
        E += 1
    e = max(E, emin)
    quantum = Fraction(2) ** (e - (P - 1))
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = fl * quantum
    if v >= Fraction(2) ** (emax + 1):
        return sgn * float("inf")
    return sgn * float(v)


FMT_PARAMS = {"f16": (11, -14, 15), "bf16": (8, -126, 127), "f32": (24, -126, 127)}


def lib_round(out, x):
    """Round FP64 values to the output format with a library cast (single rounding)."""
    x = np.asarray(x, dtype=np.float64)
    if out == "f32":
        return x.astype(np.float32).astype(np.float64)
    if out == "f16":
        with np.errstate(over="ignore"):
            return x.astype(np.float16).astype(np.float64)
    return np.array([frac_rne(Fraction(float(v)), *FMT_PARAMS["bf16"]) for v in x.ravel()]).reshape(x.shape)


def out_of(dtype):
    return "f32" if dtype in ("f32", "fp8") else dtype


def out_fmt(dtype):
    return FMT[out_of(dtype)]


def run(p, rows=None, threads=0, plain=False):
    return oracle.gemm(FMT[p.dtype], LAY[p.layout], p.M, p.N, p.K, p.A, p.lda, p.B, p.ldb,
                       rows=rows, threads=threads, plain=plain)


def exact_sums(p):
    """Exact rational sums and abs-sums from library-decoded operands."""
    a = lib_decode(p.dtype, p.A)
    b = lib_decode(p.dtype, p.B)
    S = [[Fraction(0)] * p.N for _ in range(p.M)]
    SA = [[Fraction(0)] * p.N for _ in range(p.M)]
    for i in range(p.M):
        for j in range(p.N):
            s = Fraction(0)
            sa = Fraction(0)
            for k in range(p.K):
                av = Fraction(float(a[i, k]))
                bv = Fraction(float(b[k, j] if p.layout == "nn" else b[j, k]))
                s += av * bv
                sa += abs(av * bv)
            S[i][j] = s
            SA[i][j] = sa
    return S, SA


# ---- codecs ------------------------------------------------------------------

@pytest.mark.parametrize("dtype,n", [("f16", 1 << 16), ("bf16", 1 << 16), ("fp8", 256)])
def test_decode_exhaustive(oracle_lib, dtype, n):
    bits = np.arange(n, dtype=np.uint16 if n > 256 else np.uint8)
    ours = oracle.decode(FMT[dtype], bits)
    ref = lib_decode(dtype, bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_decode_e4m3_landmarks(oracle_lib):
    # OCP E4M3: max 448, min normal 2^-6, min subnormal 2^-9, NaN = S.1111.111
    v = oracle.decode(oracle.E4M3, np.array([0x7E, 0x08, 0x01, 0x38, 0x7F, 0xFF, 0x80], dtype=np.uint8))
    assert v[0] == 448.0 and v[1] == 2.0 ** -6 and v[2] == 2.0 ** -9 and v[3] == 1.0
    assert np.isnan(v[4]) and np.isnan(v[5]) and v[6] == 0.0 and np.signbit(v[6])


def _f16_probe_values():
    allv = np.arange(1 << 16, dtype=np.uint16).view(np.float16).astype(np.float64)
    fin = np.sort(np.unique(allv[np.isfinite(allv)]))
    mids = (fin[1:] + fin[:-1]) / 2.0               # exact in FP64
    eps = np.abs(mids) * 2.0 ** -40 + 2.0 ** -60
    return np.concatenate([fin, mids, mids + eps, mids - eps,
                           [65504.0, 65519.0, 65519.999, 65520.0, 1e6, -65520.0, 2.0 ** -25, 2.0 ** -26]])


def test_encode_f16_vs_numpy(oracle_lib):
    x = _f16_probe_values()
    ours = oracle.encode(oracle.F16, x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


def test_encode_bf16_vs_torch_on_fp32_inputs(oracle_lib):
    allv = torch.arange(1 << 16, dtype=torch.int32).to(torch.int16).view(torch.bfloat16).to(torch.float64).numpy()
    fin = np.sort(np.unique(allv[np.isfinite(allv)]))
    mids = ((fin[1:] + fin[:-1]) / 2.0).astype(np.float32)    # exact in FP32
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(-np.inf))
    x32 = np.concatenate([fin.astype(np.float32), mids, up, dn,
                          np.array([3.3895314e38, 3.4e38, np.float32(np.finfo(np.float32).max)], np.float32)])
    ours = oracle.encode(oracle.BF16, x32.astype(np.float64))
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_encode_bf16_double_inputs_vs_exact_rounding(oracle_lib):
    # torch rounds FP64 -> bf16 through FP32 (twice); check single rounding exactly.
    rng = np.random.default_rng(11)
    allv = torch.arange(1 << 16, dtype=torch.int32).to(torch.int16).view(torch.bfloat16).to(torch.float64).numpy()
    fin = np.sort(np.unique(allv[np.isfinite(allv)]))
    pick = rng.choice(len(fin) - 1, 3000)
    mids = (fin[pick] + fin[pick + 1]) / 2.0
    x = np.concatenate([mids, mids * (1 + 2.0 ** -40), mids * (1 - 2.0 ** -40), rng.standard_normal(500)])
    x = x[np.isfinite(x)]
    ours = oracle.decode(oracle.BF16, oracle.encode(oracle.BF16, x))
    ref = np.array([frac_rne(Fraction(float(v)), 8, -126, 127) for v in x])
    assert np.array_equal(ours, ref)


def test_frac_rne_matches_numpy_f16(oracle_lib):
    # The exact-rational rounding used as a reference is itself checked against numpy.
    x = _f16_probe_values()[::37]
    ref = np.array([frac_rne(Fraction(float(v)), 11, -14, 15) for v in x])
    with np.errstate(over="ignore"):
        lib = x.astype(np.float16).astype(np.float64)
    assert np.array_equal(ref, lib)


def test_encode_f32_vs_numpy(oracle_lib):
    rng = np.random.default_rng(12)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000), [0.0, -0.0, 1e39]])
    ours = oracle.encode(oracle.F32, x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float32).view(np.uint32)
    assert np.array_equal(ours, ref)


# ---- brute force against exact rationals ------------------------------------

BRUTE_SHAPES = [(1, 1, 1), (1, 3, 2), (2, 1, 5), (3, 4, 7), (5, 2, 9), (9, 9, 9), (7, 5, 0)]


def _check_against_exact(p, c, s, sab):
    S, SA = exact_sums(p)
    ob = out_of(p.dtype)
    u = 2.0 ** -53
    for i in range(p.M):
        for j in range(p.N):
            ex, exa = S[i][j], SA[i][j]
            bound = float(exa) * p.K * u * 1.01
            assert abs(Fraction(float(s[i, j])) - ex) <= Fraction(bound), (i, j)
            assert abs(Fraction(float(sab[i, j])) - exa) <= Fraction(bound), (i, j)
            # c is the single rounding of the FP64 sum ...
            got = oracle.decode(FMT[ob], np.array([c[i, j]]))[0]
            assert got == lib_round(ob, [s[i, j]])[0] or (got == 0 and lib_round(ob, [s[i, j]])[0] == 0)
            # ... and of the exact sum, whenever the FP64 sum was exact.
            if Fraction(float(s[i, j])) == ex:
                P, emin, emax = FMT_PARAMS[ob]
                assert got == frac_rne(ex, P, emin, emax)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "fp8"])
@pytest.mark.parametrize("layout", ["nn", "tn"])
def test_bruteforce_exact_rationals(oracle_lib, dtype, layout):
    dist = {"f32": "uniform", "f16": "normal", "bf16": "normal", "fp8": "uniform4"}[dtype]
    rng = np.random.default_rng(100 + 10 * FMT[dtype] + LAY[layout])
    shapes = list(BRUTE_SHAPES) + [tuple(int(v) for v in rng.integers(1, 34, 3)) for _ in range(3)]
    for (M, N, K) in shapes:
        la, lb, _ = inputs.min_ld(layout, M, N, K)
        p = inputs.make(dtype, layout, M, N, K, int(rng.integers(1 << 30)), dist,
                        lda=la + int(rng.integers(0, 3)), ldb=lb + int(rng.integers(0, 3)))
        c, s, sab = run(p)
        if K == 0:
            assert np.all(s == 0) and np.all(sab == 0)
            assert np.all(oracle.decode(out_fmt(dtype), c) == 0)
            continue
        _check_against_exact(p, c, s, sab)


def test_bruteforce_integer_valued_inputs_exact(oracle_lib):
    # Small-integer operands: every FP64 sum is exact, so c must be the single
    # rounding of the exact rational sum -- including f16/bf16 overflow to inf.
    rng = np.random.default_rng(7)
    for dtype in ("f32", "f16", "bf16"):
        for layout in ("nn", "tn"):
            M, N, K = 4, 5, 6
            sa, sb = inputs.storage_shapes(layout, M, N, K, *inputs.min_ld(layout, M, N, K)[:2])
            conv = {"f32": np.float32, "f16": np.float16}
            a = rng.integers(-300, 300, sa).astype(np.float64)
            b = rng.integers(-300, 300, sb).astype(np.float64)
            if dtype == "bf16":
                a = np.round(a / 2); b = np.round(b / 2)   # 8 significant bits
                A = torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
                B = torch.from_numpy(b.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            else:
                A = a.astype(conv[dtype]).view(np.uint32 if dtype == "f32" else np.uint16)
                B = b.astype(conv[dtype]).view(np.uint32 if dtype == "f32" else np.uint16)
            la, lb, lc = inputs.min_ld(layout, M, N, K)
            p = inputs.Problem(dtype, layout, M, N, K, A, B, la, lb, lc)
            c, s, sab = run(p)
            _check_against_exact(p, c, s, sab)


# ---- closed forms -------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "fp8"])
def test_closed_forms(oracle_lib, dtype):
    for layout in ("nn", "tn"):
        for K in (1, 2, 3, 17, 256, 257):
            M, N = 3, 4
            p = inputs.make(dtype, layout, M, N, K, 0, "ones")
            c, s, sab = run(p)
            ob = out_of(dtype)
            assert np.all(s == K) and np.all(sab == K)
            assert np.all(oracle.decode(out_fmt(dtype), c) == lib_round(ob, [float(K)])[0])
            # alternating signs along k: A = 1, b(k, j) = (-1)^k  =>  C = K mod 2
            B = p.B.copy()
            neg = inputs.draw(np.random.default_rng(0), (1,), "ones", dtype, 1)[0] | \
                {"f32": np.uint32(0x80000000), "f16": np.uint16(0x8000), "bf16": np.uint16(0x8000),
                 "fp8": np.uint8(0x80)}[dtype]
            if layout == "nn":
                B[1::2, :] = neg
            else:
                B[:, 1::2] = neg
            q = inputs.Problem(dtype, layout, M, N, K, p.A, B, p.lda, p.ldb, p.ldc)
            c2, s2, _ = run(q)
            assert np.all(s2 == K % 2)
    # rank one: A = u 1^T, B = 1 v^T  =>  C_ij = K u_i v_j
    u = np.array([1.0, -2.0, 3.0, 0.5])
    v = np.array([2.0, -1.0, 0.25])
    K = 9
    for layout in ("nn", "tn"):
        Af = np.repeat(u[:, None], K, axis=1)
        Bf = np.repeat(v[None, :], K, axis=0) if layout == "nn" else np.repeat(v[:, None], K, axis=1)
        A = inputs._to_bits(Af, dtype)
        B = inputs._to_bits(Bf, dtype)
        la, lb, lc = inputs.min_ld(layout, 4, 3, K)
        p = inputs.Problem(dtype, layout, 4, 3, K, A, B, la, lb, lc)
        _, s, _ = run(p)
        assert np.array_equal(s, K * np.outer(u, v))


# ---- identity and +-1 invariants -------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "fp8"])
@pytest.mark.parametrize("layout", ["nn", "tn"])
def test_identity(oracle_lib, dtype, layout):
    dist = {"f32": "uniform", "f16": "normal", "bf16": "normal", "fp8": "uniform4"}[dtype]
    M, n = 37, 33
    p0 = inputs.make(dtype, layout, M, n, n, 5, dist)
    p = inputs.identity(dtype, layout, n, p0.A, p0.lda)
    c, s, _ = run(p)
    a = lib_decode(dtype, p0.A)[:, :n]
    assert np.array_equal(s, a)
    if dtype != "fp8":
        assert oracle.bits_equal(c, p0.A[:, :n], out_fmt(dtype))
    else:
        assert np.array_equal(oracle.decode(oracle.F32, c), a)


def test_identity_f32_256_workload(oracle_lib):
    p, ident = inputs.workload("f32_nn_256")
    c, _, _ = run(ident)
    assert oracle.bits_equal(c, p.A, oracle.F32)


@pytest.mark.parametrize("dtype,layout,K", [("f16", "tn", 8192), ("f16", "tn", 8191), ("bf16", "tn", 1000),
                                            ("fp8", "tn", 4096), ("f32", "nn", 2049)])
def test_pm1_exact_against_integer_matmul(oracle_lib, dtype, layout, K):
    M, N = 24, 20
    p = inputs.make(dtype, layout, M, N, K, 2, "pm1")
    c, s, sab = run(p)
    a = lib_decode(dtype, p.A).astype(np.int64)
    b = lib_decode(dtype, p.B).astype(np.int64)
    ref = a @ (b if layout == "nn" else b.T)
    assert np.array_equal(s, ref.astype(np.float64))
    assert np.all(sab == K)
    assert np.all((ref - K) % 2 == 0)
    assert np.array_equal(oracle.decode(out_fmt(dtype), c), lib_round(out_of(dtype), ref.astype(np.float64)))


def test_fp8_exact_against_scaled_integer_matmul(oracle_lib):
    M, N, K = 16, 24, 4096
    p = inputs.make("fp8", "tn", M, N, K, 5, "uniform4")
    _, s, sab = run(p)
    a = (lib_decode("fp8", p.A) * 512).astype(np.int64)     # multiples of 2^-9
    b = (lib_decode("fp8", p.B) * 512).astype(np.int64)
    ref = a @ b.T
    assert np.array_equal(s * 2.0 ** 18, ref.astype(np.float64))
    assert np.array_equal(sab * 2.0 ** 18, (np.abs(a) @ np.abs(b).T).astype(np.float64))


def test_f32_against_library_matmul_bound(oracle_lib):
    p = inputs.make("f32", "nn", 40, 50, 300, 1, "uniform")
    _, s, sab = run(p)
    a = lib_decode("f32", p.A)
    b = lib_decode("f32", p.B)
    ref = a @ b
    assert np.all(np.abs(s - ref) <= 2 * 300 * 2.0 ** -53 * sab)


# ---- determinism and loop equivalence ----------------------------------------

def test_threads_rows_and_plain_loop_agree(oracle_lib):
    for dtype, layout in (("bf16", "tn"), ("f32", "nn"), ("fp8", "tn"), ("f16", "nn")):
        dist = {"f32": "uniform", "f16": "normal", "bf16": "normal", "fp8": "uniform4"}[dtype]
        p = inputs.make(dtype, layout, 23, 19, 301, 3, dist)
        c1, s1, a1 = run(p, threads=1)
        c8, s8, a8 = run(p, threads=8)
        cp, sp, ap = run(p, plain=True)
        for x, y, z in ((c1, c8, cp), (s1, s8, sp), (a1, a8, ap)):
            assert np.array_equal(x.view(np.uint8), y.view(np.uint8))
            assert np.array_equal(x.view(np.uint8), z.view(np.uint8))
        rows = np.array([22, 0, 7, 7, 13])
        cr, sr, ar = run(p, rows=rows)
        assert np.array_equal(cr, c1[rows]) and np.array_equal(sr.view(np.uint64), s1[rows].view(np.uint64))


# ---- the library-product leg (whole outputs at full size) ----------------------

def run_lib(p, rows=None, with_sab=True, block=1024):
    return oracle.gemm_lib(FMT[p.dtype], LAY[p.layout], p.M, p.N, p.K, p.A, p.lda, p.B, p.ldb, rows=rows,
                           with_sab=with_sab, block=block)


@pytest.mark.parametrize("dtype,layout", [(d, l) for d in ("f32", "f16", "bf16", "fp8") for l in ("nn", "tn")])
def test_library_product_equals_the_loop(oracle_lib, dtype, layout):
    # Same decode, same single rounding; only the FP64 summation order
    # differs, so on these inputs (no sum within K 2^-52 sab of an output
    # midpoint) the bits are equal, with padded leading dimensions holding
    # garbage, blocks that do not divide the rows, and row subsets.
    dist = {"f32": "uniform", "f16": "normal", "bf16": "normal", "fp8": "uniform4"}[dtype]
    M, N, K = 70, 45, 777
    la, lb, _ = inputs.min_ld(layout, M, N, K)
    p = inputs.make(dtype, layout, M, N, K, 21, dist, lda=la + 16, ldb=lb + 16)
    c, s, sab = run(p)
    c2, sab2 = run_lib(p, block=32)
    assert np.array_equal(c, c2)
    assert np.all(np.abs(sab - sab2) <= 2 * K * 2.0 ** -53 * sab)
    rows = np.array([69, 3, 3, 40])
    c3, sab3 = run_lib(p, rows=rows, block=3)
    assert np.array_equal(c3, c[rows]) and np.all(np.abs(sab3 - sab[rows]) <= 2 * K * 2.0 ** -53 * sab[rows])
    c4, none = run_lib(p, with_sab=False)
    assert none is None and np.array_equal(c4, c)


@pytest.mark.parametrize("dtype,layout", [("f16", "tn"), ("bf16", "nn"), ("fp8", "tn"), ("f32", "tn")])
def test_library_product_exact_sets(oracle_lib, dtype, layout):
    # +-1 operands at K = 8192 (partial sums exact in any order): the output
    # is the integer matrix product rounded once; the identity gives A back.
    p = inputs.make(dtype, layout, 24, 20, 8192, 2, "pm1")
    c, sab = run_lib(p)
    a = lib_decode(dtype, p.A).astype(np.int64)
    b = lib_decode(dtype, p.B).astype(np.int64)
    ref = a @ (b if layout == "nn" else b.T)
    assert np.all(sab == p.K)
    assert np.array_equal(oracle.decode(out_fmt(dtype), c), lib_round(out_of(dtype), ref.astype(np.float64)))
    q = inputs.make(dtype, layout, 30, 64, 64, 4, "uniform4" if dtype == "fp8" else "normal")
    ident = inputs.identity(dtype, layout, 64, q.A, q.lda)
    ci, _ = run_lib(ident)
    assert np.array_equal(oracle.decode(out_fmt(dtype), ci), lib_decode(dtype, q.A[:, :64]))
    # empty sums and empty row sets
    z, zs = run_lib(inputs.make(dtype, layout, 5, 6, 0, 1, "pm1"))
    assert np.all(z == 0) and np.all(zs == 0)


def test_library_product_catches_planted_mistakes(oracle_lib):
    p = inputs.make("bf16", "tn", 64, 64, 64, 3, "pm1")
    c, _ = run_lib(p, with_sab=False)
    # B read in the other layout (a transposed operand)
    wrong = oracle.gemm_lib(oracle.BF16, oracle.NN, p.M, p.N, p.K, p.A, p.lda, p.B, p.ldb, with_sab=False)[0]
    assert not np.array_equal(wrong, c)
    # one k term dropped (K - 1): every +-1 sum changes parity
    short = oracle.gemm_lib(oracle.BF16, oracle.TN, p.M, p.N, p.K - 1, p.A, p.lda, p.B, p.ldb, with_sab=False)[0]
    assert not np.any(short == c)


# ---- acceptance checker -------------------------------------------------------

def test_checker_accepts_and_rejects_as_predicted(oracle_lib):
    p = inputs.make("bf16", "tn", 16, 16, 64, 9, "normal")
    c, s, sab = run(p)
    ok, err, nbad = oracle.check(c, c, sab, oracle.BF16, oracle.TOL["bf16"])
    assert ok and err == 0 and nbad == 0
    # one bf16 ulp on one element: relative to sab it is well inside 2^-7
    c1 = c.copy(); c1[3, 4] += 1
    ok, err, _ = oracle.check(c1, c, sab, oracle.BF16, oracle.TOL["bf16"])
    assert ok and err > 0
    # an error of 2^-6 * sab on one element must fail
    bad = c.copy()
    target = oracle.decode(oracle.BF16, c)[5, 6] + sab[5, 6] * 2.0 ** -6
    bad[5, 6] = oracle.encode(oracle.BF16, np.array([target]))[0]
    ok, _, nbad = oracle.check(bad, c, sab, oracle.BF16, oracle.TOL["bf16"])
    assert not ok and nbad == 1
    # NaN where the reference is finite fails
    nanc = c.copy(); nanc[0, 0] = 0x7fc0
    assert not oracle.check(nanc, c, sab, oracle.BF16, 1.0)[0]
    # where the reference overflows to +-Inf (or is NaN) only the same kind
    # passes: a finite value, the other infinity or NaN against Inf fail, and
    # so does a finite value or an infinity against NaN, at any tolerance
    pinf, ninf, qnan = 0x7f80, 0xff80, 0x7fc0
    ref = c.copy(); ref[1, 2] = pinf; ref[2, 3] = ninf; ref[4, 4] = qnan
    assert oracle.check(ref, ref, sab, oracle.BF16, oracle.TOL["bf16"])[0]
    for at, planted in (((1, 2), c[1, 2]), ((1, 2), ninf), ((1, 2), qnan), ((2, 3), pinf), ((2, 3), 0x7f7f),
                        ((4, 4), pinf), ((4, 4), 0)):
        got = ref.copy(); got[at] = planted
        ok, _, nbad = oracle.check(got, ref, sab, oracle.BF16, 1e300)
        assert not ok and nbad == 1, (at, hex(int(planted)))
    # the same for an FP32 output (FP8 products) overflowing
    r32 = np.array([[0x7f800000, 0x3f800000]], np.uint32)
    s32 = np.ones((1, 2))
    assert oracle.check(r32, r32, s32, oracle.F32, 2.0 ** -7)[0]
    assert not oracle.check(np.array([[0x7f7fffff, 0x3f800000]], np.uint32), r32, s32, oracle.F32, 1e300)[0]
    # sab == 0 requires exact equality
    z = np.zeros((1, 1), np.uint16)
    assert oracle.check(z, z, np.zeros((1, 1)), oracle.BF16, 1.0)[0]
    assert not oracle.check(z + 1, z, np.zeros((1, 1)), oracle.BF16, 1.0)[0]
    # bit equality treats +0 and -0 alike, nothing else
    assert oracle.bits_equal(np.array([0x8000], np.uint16), np.array([0], np.uint16), oracle.BF16)
    assert not oracle.bits_equal(np.array([0x8001], np.uint16), np.array([1], np.uint16), oracle.BF16)


# ---- FP8 with scale factors -------------------------------------------------

def _factors(rng, n):
    """FP32 factors with full 24-bit significands, both signs, spread exponents."""
    x = rng.uniform(1.0, 2.0, n) * 2.0 ** rng.integers(-8, 9, n) * rng.choice([-1.0, 1.0], n)
    return x.astype(np.float32)


def _scaled(p, sa, sb, rows=None):
    return oracle.gemm_fp8_scaled(LAY[p.layout], p.M, p.N, p.K, p.A, p.lda, p.B, p.ldb, sa, sb, rows=rows)


def _check_scaled_exact(p, sa, sb, c, sab):
    """Bit-exact against exact-rational s_ij * sa_i * sb_j rounded once to FP32."""
    S, SA = exact_sums(p)
    for i in range(p.M):
        for j in range(p.N):
            fa = Fraction(float(sa[i if sa.size > 1 else 0]))
            fb = Fraction(float(sb[j if sb.size > 1 else 0]))
            want = frac_rne(S[i][j] * fa * fb, *FMT_PARAMS["f32"])
            got = float(oracle.decode(oracle.F32, c[i:i + 1, j])[0])
            if got != want:
                return False
            norm = float(SA[i][j] * abs(fa * fb))
            assert abs(sab[i, j] - norm) <= 1e-15 * norm
    return True


def test_scaled_unit_factors_reduce_to_plain(oracle_lib):
    for layout in ("nn", "tn"):
        p = inputs.make("fp8", layout, 9, 7, 70, 31, "uniform4")
        c0, _, sab0 = run(p)
        c, sab = _scaled(p, np.float32([1.0]), np.float32([1.0]))
        assert np.array_equal(c, c0) and np.array_equal(sab, sab0)


@pytest.mark.parametrize("layout", ["nn", "tn"])
@pytest.mark.parametrize("mode", ["tensor", "row"])
def test_scaled_bruteforce_exact_rationals(oracle_lib, layout, mode):
    rng = np.random.default_rng(41 + (layout == "nn"))
    for M, N, K in [(1, 1, 1), (3, 5, 7), (6, 4, 33), (2, 9, 64)]:
        p = inputs.make("fp8", layout, M, N, K, 50 + K, "uniform4")
        sa = _factors(rng, M if mode == "row" else 1)
        sb = _factors(rng, N if mode == "row" else 1)
        c, sab = _scaled(p, sa, sb)
        assert _check_scaled_exact(p, sa, sb, c, sab)
        if mode == "row":
            # rows subset: the same values for the rows asked for
            rows = np.array([M - 1, 0], dtype=np.int64)
            cr, sabr = _scaled(p, sa, sb, rows=rows)
            assert np.array_equal(cr, c[rows]) and np.array_equal(sabr, sab[rows])


def test_scaled_closed_form_rank_one(oracle_lib):
    # A = 1, B = 1 => C_ij = K * sa_i * sb_j: with power-of-two factors exact
    # in FP32, and distinct per row / column so that a swapped role shows.
    for layout in ("nn", "tn"):
        M, N, K = 5, 3, 48
        p = inputs.make("fp8", layout, M, N, K, 0, "ones")
        sa = np.float32([2.0 ** e for e in (-3, 0, 1, 5, -7)])
        sb = np.float32([-4.0, 0.5, 2.0 ** -10])
        c, sab = _scaled(p, sa, sb)
        want = K * np.outer(sa.astype(np.float64), sb.astype(np.float64))
        assert np.array_equal(oracle.decode(oracle.F32, c), want)
        assert np.array_equal(sab, np.abs(want))
    # a zero factor gives an exact zero and a zero normaliser
    c, sab = _scaled(p, np.float32([0.0]), sb)
    assert np.all(oracle.decode(oracle.F32, c) == 0) and np.all(sab == 0)


def test_scaled_pins_catch_planted_mistakes(oracle_lib):
    rng = np.random.default_rng(77)
    p = inputs.make("fp8", "nn", 4, 6, 20, 78, "uniform4")
    sa, sb = _factors(rng, 4), _factors(rng, 6)
    assert _check_scaled_exact(p, sa, sb, *_scaled(p, sa, sb))
    # factors of A applied in reverse row order
    assert not _check_scaled_exact(p, sa, sb, *_scaled(p, sa[::-1].copy(), sb))
    # one factor's sign lost
    assert not _check_scaled_exact(p, sa, sb, *_scaled(p, np.abs(sa), sb))
    # only one of the two factors applied
    assert not _check_scaled_exact(p, sa, sb, *_scaled(p, sa, np.float32([1.0])))


# ---- MXFP8: E8M0 block scales ---------------------------------------------

def _mx(p, SA, ldsa, SB, ldsb, rows=None):
    return oracle.gemm_mxfp8(LAY[p.layout], p.M, p.N, p.K, p.A, p.lda, p.B, p.ldb, SA, ldsa, SB, ldsb, rows=rows)


def _check_mx_exact(p, SA, ldsa, SB, ldsb, c):
    """Bit-exact against the exact-rational block-scaled sum rounded once to FP32."""
    a = lib_decode("fp8", p.A).reshape(-1)
    b = lib_decode("fp8", p.B).reshape(-1)
    for i in range(p.M):
        for j in range(p.N):
            acc = Fraction(0)
            for k in range(p.K):
                blk = k // 32
                av = Fraction(float(a[i * p.lda + k]))
                bv = Fraction(float(b[k * p.ldb + j] if p.layout == "nn" else b[j * p.ldb + k]))
                acc += av * bv * Fraction(2) ** (int(SA[i * ldsa + blk]) - 127) * \
                    Fraction(2) ** (int(SB[j * ldsb + blk]) - 127)
            want = frac_rne(acc, *FMT_PARAMS["f32"])
            if float(oracle.decode(oracle.F32, c[i:i + 1, j])[0]) != want:
                return False
    return True


def test_e8m0_values(oracle_lib):
    e = np.arange(256)
    v = oracle.e8m0(e)
    assert v[127] == 1.0 and v[128] == 2.0 and v[0] == 2.0 ** -127 and v[254] == 2.0 ** 127
    assert np.isnan(v[255]) and np.all(v[:255] == [2.0 ** (x - 127) for x in range(255)])


def test_mx_unit_scales_reduce_to_plain(oracle_lib):
    for layout in ("nn", "tn"):
        p = inputs.make("fp8", layout, 6, 5, 160, 61, "uniform4")
        c0, _, sab0 = run(p)
        c, sab = _mx(p, np.full(6 * 5, 127, np.uint8), 5, np.full(5 * 5, 127, np.uint8), 5)
        assert np.array_equal(c, c0) and np.array_equal(sab, sab0)


@pytest.mark.parametrize("layout", ["nn", "tn"])
def test_mx_bruteforce_exact_rationals(oracle_lib, layout):
    rng = np.random.default_rng(90 + (layout == "nn"))
    for M, N, K in [(1, 1, 32), (3, 4, 64), (4, 3, 96)]:
        p = inputs.make("fp8", layout, M, N, K, 70 + K, "uniform4")
        nb = K // 32
        ldsa, ldsb = nb + 1, nb + 3          # padded rows; the padding holds NaN codes
        SA = np.full(M * ldsa, 255, np.uint8)
        SB = np.full(N * ldsb, 255, np.uint8)
        for i in range(M):
            SA[i * ldsa:i * ldsa + nb] = rng.integers(112, 143, nb)
        for j in range(N):
            SB[j * ldsb:j * ldsb + nb] = rng.integers(112, 143, nb)
        c, sab = _mx(p, SA, ldsa, SB, ldsb)
        assert _check_mx_exact(p, SA, ldsa, SB, ldsb, c)
        assert np.all(np.isfinite(sab))
        rows = np.array([M - 1, 0], dtype=np.int64)
        cr, _ = _mx(p, SA, ldsa, SB, ldsb, rows=rows)
        assert np.array_equal(cr, c[rows])


def test_mx_closed_form(oracle_lib):
    # A = B = 1, SA[i][b] = 127 + b, SB[j][b] = 127 + j:
    # C_ij = 32 * 2^j * (2^nb - 1).  Blocks of any other width than 32, or
    # the two operands' scales exchanged, give other values.
    for layout in ("nn", "tn"):
        M, N, K = 3, 4, 160
        nb = K // 32
        p = inputs.make("fp8", layout, M, N, K, 0, "ones")
        SA = np.array([127 + blk for _ in range(M) for blk in range(nb)], np.uint8)
        SB = np.array([127 + j for j in range(N) for _ in range(nb)], np.uint8)
        c, sab = _mx(p, SA, nb, SB, nb)
        want = np.array([[32.0 * 2.0 ** j * (2.0 ** nb - 1) for j in range(N)] for _ in range(M)])
        assert np.array_equal(oracle.decode(oracle.F32, c), want) and np.array_equal(sab, want)
    # a NaN scale (code 255) makes its outputs NaN
    SA2 = SA.copy()
    SA2[0] = 255
    c, _ = _mx(p, SA2, nb, SB, nb)
    assert np.all(np.isnan(oracle.decode(oracle.F32, c[0]))) and not np.any(np.isnan(oracle.decode(oracle.F32, c[1:])))


def test_mx_pins_catch_planted_mistakes(oracle_lib):
    rng = np.random.default_rng(95)
    p = inputs.make("fp8", "tn", 3, 4, 96, 96, "uniform4")
    SA = rng.integers(118, 137, 3 * 3).astype(np.uint8)
    SB = rng.integers(118, 137, 4 * 3).astype(np.uint8)
    assert _check_mx_exact(p, SA, 3, SB, 3, _mx(p, SA, 3, SB, 3)[0])
    # scale blocks of A's rows in reverse order
    rev = SA.reshape(3, 3)[:, ::-1].reshape(-1).copy()
    assert not _check_mx_exact(p, SA, 3, SB, 3, _mx(p, rev, 3, SB, 3)[0])
    # A's and B's scales exchanged (first three rows)
    assert not _check_mx_exact(p, SA, 3, SB, 3, _mx(p, SB[:9].copy(), 3, np.concatenate([SA, SA[:3]]), 3)[0])
    # one scale off by one
    off = SB.copy()
    off[5] += 1
    assert not _check_mx_exact(p, SA, 3, SB, 3, _mx(p, SA, 3, off, 3)[0])


# ---- sensitivity: planted mistakes must trip a pin ---------------------------

def test_pins_catch_planted_mistakes(oracle_lib):
    p = inputs.make("f16", "tn", 6, 6, 40, 21, "pm1")
    a = lib_decode("f16", p.A).astype(np.int64)
    b = lib_decode("f16", p.B).astype(np.int64)
    ref = a @ b.T
    assert np.array_equal(run(p)[1], ref)
    # transposed operand: read the square TN B storage as if it were NN
    sq = inputs.make("f16", "tn", 6, 6, 6, 23, "pm1")
    sref = lib_decode("f16", sq.A).astype(np.int64) @ lib_decode("f16", sq.B).astype(np.int64).T
    _, s_t, _ = oracle.gemm(oracle.F16, oracle.NN, 6, 6, 6, sq.A, 6, sq.B, 6)
    assert not np.array_equal(s_t, sref)
    # dropped term: K - 1 instead of K
    _, s_d, _ = oracle.gemm(oracle.F16, oracle.TN, 6, 6, 39, p.A, p.lda, p.B, p.ldb)
    assert not np.array_equal(s_d, ref)
    # wrong sign of one operand
    _, s_n, _ = oracle.gemm(oracle.F16, oracle.TN, 6, 6, 40, p.A ^ np.uint16(0x8000), p.lda, p.B, p.ldb)
    assert not np.array_equal(s_n, ref)
    # wrong index: row i of A paired with row i+1
    _, s_i, _ = oracle.gemm(oracle.F16, oracle.TN, 5, 6, 40, p.A[1:].copy(), p.lda, p.B, p.ldb)
    assert not np.array_equal(s_i, ref[:5])
