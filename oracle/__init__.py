"""CPU oracle for the dense GEMM C = A x B.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports it, and the two share no code.

The arithmetic lives in ``oracle.cpp`` (built with g++, OpenMP over rows, FP64
accumulation, one round-to-nearest-even rounding to the output format).  This
module only builds and loads that library, marshals numpy arrays, applies
the FP8 scale factors to the exact sums (``gemm_fp8_scaled``), computes the
block-scaled MXFP8 product from per-block library matrix products in FP64
(``gemm_mxfp8``), gives the same definition with the FP64 sum taken by a
library matrix product for whole outputs at full size (``gemm_lib``), and
holds the acceptance check.

Definition followed: "Optimizing GEMM in HIP", section "GEMM fundamentals"
(C_ij = inner product of row i of A and column j of B); storage layouts from
"FP16 GEMM Optimization on AMD RDNA 3 and RDNA 4", section "What We Are
Computing" (TN: A row-major, B column-major, C column-major, ld = M).

Parity status: pinned (see tests/test_oracle_pins.py).
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, F16, BF16, E4M3 = 0, 1, 2, 3
NN, TN = 0, 1

FMT = {"f32": F32, "f16": F16, "bf16": BF16, "e4m3": E4M3}
_BITS_DTYPE = {F32: np.uint32, F16: np.uint16, BF16: np.uint16, E4M3: np.uint8}

# Acceptance bounds on max_ij |c - c_ref| / sum_k |a_ik b_kj|, per output.
TOL = {"f32": 1e-6, "f16": 2.0 ** -10, "bf16": 2.0 ** -7, "fp8": 2.0 ** -7}


def build(force: bool = False) -> str:
    """Compile liboracle.so with g++ (no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["g++", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-std=c++17", "-fPIC", "-shared", _SRC, "-o", tmp]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        i64, vp, dp = ctypes.c_int64, ctypes.c_void_p, ctypes.POINTER(ctypes.c_double)
        L.oracle_gemm.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, i64, i64, i64,
                                  vp, i64, vp, i64, vp, i64, vp, vp, vp, ctypes.c_int]
        L.oracle_gemm.restype = ctypes.c_int
        L.oracle_gemm_plain.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, i64, i64, i64,
                                        vp, i64, vp, i64, vp, vp, vp]
        L.oracle_gemm_plain.restype = ctypes.c_int
        L.oracle_decode.argtypes = [ctypes.c_int, vp, i64, vp]
        L.oracle_decode.restype = None
        L.oracle_encode.argtypes = [ctypes.c_int, vp, i64, vp]
        L.oracle_encode.restype = None
        L.oracle_max_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def out_fmt_of(in_fmt: int) -> int:
    """FP8 inputs produce FP32 output; every other input format is its own output format."""
    return F32 if in_fmt == E4M3 else in_fmt


def gemm(in_fmt, layout, M, N, K, A, lda, B, ldb, rows=None, threads=0, plain=False):
    """Run the oracle.

    A, B are numpy arrays of raw storage bits (uint32 for f32, uint16 for
    f16/bf16, uint8 for e4m3) holding the operands in their storage layout
    (flattened with the given leading dimensions).  Returns (c_bits, s, sab),
    each shaped [len(rows) or M][N] and indexed [i][j] whatever the layout.
    """
    A = np.ascontiguousarray(A).view(_BITS_DTYPE[in_fmt])
    B = np.ascontiguousarray(B).view(_BITS_DTYPE[in_fmt])
    of = out_fmt_of(in_fmt)
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
    nr = M if rows is None else len(rows)
    c = np.zeros((nr, N), dtype=np.uint32 if of == F32 else np.uint16)
    s = np.zeros((nr, N), dtype=np.float64)
    sab = np.zeros((nr, N), dtype=np.float64)
    if plain:
        if rows is not None:
            raise ValueError("plain loop computes all rows")
        rc = lib().oracle_gemm_plain(in_fmt, of, layout, M, N, K, _ptr(A), lda, _ptr(B), ldb,
                                     _ptr(c), _ptr(s), _ptr(sab))
    else:
        rc = lib().oracle_gemm(in_fmt, of, layout, M, N, K, _ptr(A), lda, _ptr(B), ldb,
                               _ptr(rows), nr, _ptr(c), _ptr(s), _ptr(sab), int(threads))
    if rc != 0:
        raise ValueError("oracle_gemm rejected its arguments")
    return c, s, sab


def _decode_a_rows(in_fmt, K, A, lda, rows):
    """a[i][k] = A[i*lda + k] for the requested rows, decoded exactly with the
    oracle's own decoder ("Optimizing GEMM in HIP", GEMM fundamentals)."""
    A2 = np.asarray(A).reshape(-1, lda)
    return decode(in_fmt, np.ascontiguousarray(A2[rows, :K]))


def _decode_b(in_fmt, layout, N, K, B, ldb):
    """b as a K x N array: B[k*ldb + j] (NN) or B[j*ldb + k] (TN: B stored
    column-major, "FP16 GEMM Optimization on AMD RDNA 3 and RDNA 4", What We
    Are Computing), decoded exactly.  For TN the result is a transposed view
    of the decoded N x K storage (the library product takes it as it is)."""
    B2 = np.asarray(B).reshape(-1, ldb)
    if layout == NN:
        return decode(in_fmt, np.ascontiguousarray(B2[:K, :N]))
    return decode(in_fmt, np.ascontiguousarray(B2[:N, :K])).T


def gemm_lib(in_fmt, layout, M, N, K, A, lda, B, ldb, rows=None, with_sab=True, block=1024):
    """The definition ``gemm`` computes, with the FP64 sum formed by a library
    matrix product (numpy's BLAS) instead of the triple loop; for checking
    whole outputs at sizes where the loop would take minutes.

    Steps, per element (i, j): a(i,k) and b(k,j) decoded exactly (the same
    decoder as ``gemm``), s_ij = sum_k a(i,k) b(k,j) in FP64,
    sab_ij = sum_k |a(i,k) b(k,j)| in FP64 (skipped when ``with_sab`` is
    false, e.g. for bit-exact comparisons), and s_ij rounded once to the
    output format (the same encoder).  The library sums in its own order:
    where every partial sum is exact in FP64 (E4M3 operands: multiples of
    2^-18 below 2^49; +-1 and identity operands) the result equals ``gemm``'s
    bit for bit; otherwise s differs from the loop's by FP64 rounding
    (<= K 2^-52 sab), which changes the rounded output only where s lies that
    close to a rounding midpoint of the output format.

    Returns (c_bits, sab) shaped [len(rows) or M][N] (sab is None without
    ``with_sab``).  Rows are processed in blocks of ``block``.
    """
    rows = np.arange(M, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    of = out_fmt_of(in_fmt)
    c = np.empty((len(rows), N), dtype=np.uint32 if of == F32 else np.uint16)
    sab = np.empty((len(rows), N), dtype=np.float64) if with_sab else None
    for r0, cb, sb in gemm_lib_blocks(in_fmt, layout, M, N, K, A, lda, B, ldb, rows, with_sab, block):
        c[r0:r0 + len(cb)] = cb
        if with_sab:
            sab[r0:r0 + len(cb)] = sb
    return c, sab


def gemm_lib_blocks(in_fmt, layout, M, N, K, A, lda, B, ldb, rows=None, with_sab=True, block=1024):
    """``gemm_lib`` one block of rows at a time: yields (r0, c_bits, sab) for
    rows[r0 : r0 + block] (sab None without ``with_sab``).  The arrays of a
    block are reused for the next one."""
    rows = np.arange(M, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    of = out_fmt_of(in_fmt)
    if len(rows) == 0:
        return
    nb = min(block, len(rows))
    cbuf = np.zeros((nb, N), dtype=np.uint32 if of == F32 else np.uint16)
    sbuf = np.zeros((nb, N), dtype=np.float64) if with_sab else None
    if K == 0 or N == 0:
        for r0 in range(0, len(rows), block):
            n = len(rows[r0:r0 + block])
            yield r0, cbuf[:n], (sbuf[:n] if with_sab else None)
        return
    b = _decode_b(in_fmt, layout, N, K, B, ldb)
    babs = None
    if with_sab:
        babs = np.abs(b.T).T if layout == TN else np.abs(b)   # elementwise, in storage order
    acc = np.empty((nb, N), dtype=np.float64)
    aabs = np.empty((nb, K), dtype=np.float64) if with_sab else None
    with np.errstate(invalid="ignore", over="ignore"):
        for r0 in range(0, len(rows), block):
            blk = rows[r0:r0 + block]
            n = len(blk)
            a = _decode_a_rows(in_fmt, K, A, lda, blk)
            np.matmul(a, b, out=acc[:n])
            cbuf[:n] = encode(of, acc[:n])
            if with_sab:
                np.abs(a, out=aabs[:n])
                np.matmul(aabs[:n], babs, out=sbuf[:n])
            yield r0, cbuf[:n], (sbuf[:n] if with_sab else None)


def scale_vector(scale, n):
    """A factor vector of length 1 (one factor for all) or n, as FP64 values of n entries."""
    f = np.asarray(scale, dtype=np.float32).reshape(-1).astype(np.float64)
    if f.size == 1:
        return np.full(n, f[0])
    if f.size != n:
        raise ValueError("a factor vector holds 1 or %d values" % n)
    return f


def gemm_fp8_scaled(layout, M, N, K, A, lda, B, ldb, scale_a, scale_b, rows=None, threads=0):
    """E4M3 GEMM with per-tensor or per-row FP32 scale factors.

    The factors a quantized FP8 kernel carries, applied after the sum ("FP8
    GEMM Optimization on AMD RDNA 4", section "What Changes at FP8"):
    C_ij = s_ij * sa_i * sb_j, where s_ij is the exact sum from ``gemm``
    (exact in FP64 for E4M3 operands), sa_i = scale_a[i] (M values) or
    scale_a[0] (one value), sb_j = scale_b[j] (N values) or scale_b[0].  The
    product is formed in FP64 (sa_i * sb_j exactly) and rounded once more to
    FP32 with round-to-nearest-even.  (s_ij * sa_i * sb_j can need more than
    53 bits, so this is two roundings; they differ from one only when the
    FP64 value falls exactly on an FP32 tie.)

    Returns (c_bits, sab): FP32 output bits [len(rows) or M][N] and the
    normaliser S_ij * |sa_i * sb_j| of the acceptance check.
    """
    _, s, sab = gemm(E4M3, layout, M, N, K, A, lda, B, ldb, rows=rows, threads=threads)
    sa = scale_vector(scale_a, M)
    sb = scale_vector(scale_b, N)
    if rows is not None:
        sa = sa[np.asarray(rows, dtype=np.int64)]
    f = sa[:, None] * sb[None, :]
    with np.errstate(invalid="ignore", over="ignore"):
        c = encode(F32, s * f)
        return c.astype(np.uint32), sab * np.abs(f)


def e8m0(bits) -> np.ndarray:
    """Values of E8M0 scale bytes: 2^(e - 127), and NaN for e = 255 (OCP
    Microscaling (MX) format, the shared-scale element type)."""
    e = np.asarray(bits, dtype=np.int64)
    v = np.ldexp(1.0, e - 127)
    return np.where(e == 255, np.nan, v)


def operands_fp64(in_fmt, layout, M, N, K, A, lda, B, ldb):
    """a[i][k] and b[k][j] decoded exactly, whatever the storage layout."""
    A = np.asarray(A).reshape(-1)
    B = np.asarray(B).reshape(-1)
    i, j, k = np.arange(M)[:, None], np.arange(N)[None, :], np.arange(K)
    a = decode(in_fmt, A[i * lda + k[None, :]])                   # A(i,k) = A[i*lda + k]
    if layout == NN:
        b = decode(in_fmt, B[k[:, None] * ldb + j])               # B(k,j) = B[k*ldb + j]
    else:
        b = decode(in_fmt, B[j * ldb + k[:, None]])               # B(k,j) = B[j*ldb + k]
    return a.reshape(M, K), b.reshape(K, N)


def gemm_mxfp8(layout, M, N, K, A, lda, B, ldb, SA, ldsa, SB, ldsb, rows=None):
    """MXFP8 GEMM: E4M3 operands with one E8M0 scale per 32 consecutive k of
    each row of A (SA[i*ldsa + b]) and each column of B (SB[j*ldsb + b]).

    The block-scaled dot product of the OCP Microscaling (MX) format, the
    scaled variant that "FP8 GEMM Optimization on AMD RDNA 4" (section "What
    Changes at FP8") leaves for later work:
        C_ij = sum_b 2^(SA_ib - 127) 2^(SB_jb - 127) sum_{k in block b} a_ik b_kj.
    Each block's sum is a library matrix product in FP64 and exact (E4M3
    products are multiples of 2^-18 below 2^18 in magnitude, so 32 of them
    need under 42 bits), and so is its product with the two powers of two;
    the sum over blocks is rounded in FP64 (relative error below
    (K/32) * 2^-53) and then once to FP32 with round-to-nearest-even.

    Returns (c_bits, sab): FP32 output bits [len(rows) or M][N] and the
    normaliser sum_b 2^.. 2^.. sum_k |a_ik b_kj| of the acceptance check.
    """
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    nb = K // 32
    a, b = operands_fp64(E4M3, layout, M, N, K, A, lda, B, ldb)
    SA = np.asarray(SA).reshape(-1)
    SB = np.asarray(SB).reshape(-1)
    ia = np.arange(M) if rows is None else np.asarray(rows, dtype=np.int64)
    a = a[ia]
    sa = e8m0(np.array([[SA[i * ldsa + blk] for blk in range(nb)] for i in ia], dtype=np.int64).reshape(len(ia), nb))
    sb = e8m0(np.array([[SB[j * ldsb + blk] for blk in range(nb)] for j in range(N)], dtype=np.int64).reshape(N, nb))
    c = np.zeros((len(ia), N))
    sab = np.zeros((len(ia), N))
    with np.errstate(invalid="ignore", over="ignore"):
        for blk in range(nb):
            ks = slice(32 * blk, 32 * blk + 32)
            f = sa[:, blk][:, None] * sb[:, blk][None, :]
            c += (a[:, ks] @ b[ks, :]) * f
            sab += (np.abs(a[:, ks]) @ np.abs(b[ks, :])) * f
        return encode(F32, c).astype(np.uint32), sab


def decode(fmt, bits) -> np.ndarray:
    bits = np.ascontiguousarray(bits).view(_BITS_DTYPE[fmt])
    out = np.empty(bits.shape, dtype=np.float64)
    lib().oracle_decode(fmt, _ptr(bits), bits.size, _ptr(out))
    return out


def encode(fmt, x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint32 if fmt == F32 else np.uint16)
    lib().oracle_encode(fmt, _ptr(x), x.size, _ptr(out))
    return out


def max_threads() -> int:
    return lib().oracle_max_threads()


def check(c_bits, c_ref_bits, sab, out_fmt, tol):
    """Acceptance check of a computed C against the oracle.

    err_ij = |c_ij - c_ref_ij| / sab_ij with both values decoded exactly, in
    FP64.  Passes when max err <= tol, every element with sab == 0 matches
    exactly, no NaN/Inf appears where the reference is finite, and where the
    reference is not finite the result is of the same kind: the same signed
    infinity (an overflow of the output format), or NaN for NaN.
    Returns (ok, max_err, n_bad).
    """
    c = decode(out_fmt, c_bits)
    r = decode(out_fmt, c_ref_bits)
    sab = np.asarray(sab, dtype=np.float64)
    finite_ref = np.isfinite(r)
    same_kind = (np.isnan(r) & np.isnan(c)) | (np.isinf(r) & (c == r))
    bad_nonfinite = (finite_ref & ~np.isfinite(c)) | (~finite_ref & ~same_kind)
    diff = np.abs(c - r)
    zero = sab == 0
    with np.errstate(divide="ignore", invalid="ignore"):
        err = np.where(zero, 0.0, diff / np.where(zero, 1.0, sab))
    err = np.where(finite_ref, err, 0.0)
    bad_zero = zero & finite_ref & (c != r)
    bad = bad_nonfinite | bad_zero | (err > tol) | np.isnan(err)
    max_err = float(np.nanmax(err)) if err.size else 0.0
    return (not bad.any()), max_err, int(bad.sum())


def bits_equal(c_bits, c_ref_bits, out_fmt) -> bool:
    """Bit-exact comparison that treats +0 and -0 as equal."""
    c = np.asarray(c_bits)
    r = np.asarray(c_ref_bits)
    sign = np.uint32(0x80000000) if out_fmt == F32 else np.uint16(0x8000)
    mag_c = c & ~sign
    mag_r = r & ~sign
    both_zero = (mag_c == 0) & (mag_r == 0)
    return bool(np.all(both_zero | (c == r)))
