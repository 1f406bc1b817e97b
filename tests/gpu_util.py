"""Helpers for GPU parity tests: move a Problem's storage to the device, run it
through the C ABI, bring C back in [i][j] order, and compare with the oracle."""

from __future__ import annotations

import sys

import numpy as np

import oracle

FMT = {"f32": oracle.F32, "f16": oracle.F16, "bf16": oracle.BF16, "fp8": oracle.E4M3}
LAY = {"nn": oracle.NN, "tn": oracle.TN}
OUT_FMT = {"f32": oracle.F32, "f16": oracle.F16, "bf16": oracle.BF16, "fp8": oracle.F32}


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def to_dev(bits):
    import torch
    arr = np.ascontiguousarray(bits)
    if arr.dtype == np.uint32:
        t = torch.from_numpy(arr.view(np.int32))
    elif arr.dtype == np.uint16:
        t = torch.from_numpy(arr.view(np.int16))
    else:
        t = torch.from_numpy(arr.view(np.uint8))
    return t.cuda()


def out_is_32(dtype):
    return dtype in ("f32", "fp8")


def c_shape(p):
    return (p.N, p.ldc) if p.layout == "tn" else (p.M, p.ldc)


def alloc_c(p):
    """C storage filled with all-ones bits (a NaN in every output format)."""
    import torch
    dt = torch.int32 if out_is_32(p.dtype) else torch.int16
    return torch.full(c_shape(p), -1, dtype=dt, device="cuda")


def run_gpu(p, A=None, B=None, C=None, stream=None, sync=True):
    """Runs the problem; returns the device C tensor (storage layout)."""
    from dense_gemm_02_amd import binding
    A = to_dev(p.A) if A is None else A
    B = to_dev(p.B) if B is None else B
    C = alloc_c(p) if C is None else C
    binding.gemm(p.dtype, p.layout, p.M, p.N, p.K, A, p.lda, B, p.ldb, C, p.ldc, stream=stream)
    if sync:
        import torch
        torch.cuda.synchronize()
    return C


def c_host(p, C):
    """C as an [M][N] array of output bits, plus the untouched padding."""
    cs = C.cpu().numpy()
    cs = cs.view(np.uint32) if out_is_32(p.dtype) else cs.view(np.uint16)
    if p.layout == "tn":
        return np.ascontiguousarray(cs[:, :p.M].T), cs[:, p.M:]
    return np.ascontiguousarray(cs[:, :p.N]), cs[:, p.N:]


def pad_untouched(pad, dtype):
    full = np.uint32(0xFFFFFFFF) if out_is_32(dtype) else np.uint16(0xFFFF)
    return bool(np.all(pad == full))


def oracle_ref(p, rows=None):
    return oracle.gemm(FMT[p.dtype], LAY[p.layout], p.M, p.N, p.K, p.A, p.lda, p.B, p.ldb, rows=rows)


# Above this many multiply-adds a whole output is checked with the oracle's
# library-product leg (the same definition, pinned to the loop bit for bit),
# block by block; below it the triple loop itself is the reference.
LOOP_MACS = 5e8


def compare(p, cij, rows=None, exact=False, tol=None):
    """Compare GPU output rows (all of them when rows is None) with the
    oracle.  Returns (ok, max_err, n_bad)."""
    of = OUT_FMT[p.dtype]
    tol = oracle.TOL[p.dtype] if tol is None else tol
    if rows is None and p.M * p.N * max(p.K, 1) > LOOP_MACS:
        ok, max_err, nbad = True, 0.0, 0
        for r0, c_ref, sab in oracle.gemm_lib_blocks(FMT[p.dtype], LAY[p.layout], p.M, p.N, p.K, p.A, p.lda,
                                                     p.B, p.ldb, with_sab=not exact, block=2048):
            got = cij[r0:r0 + len(c_ref)]
            if exact:
                if not oracle.bits_equal(got, c_ref, of):
                    ok = False
                    nbad += int(np.sum(got != c_ref))
            else:
                o, e, nb = oracle.check(got, c_ref, sab, of, tol)
                ok, max_err, nbad = ok and o, max(max_err, e), nbad + nb
        return ok, max_err, nbad
    c_ref, _, sab = oracle_ref(p, rows)
    got = cij if rows is None else cij[np.asarray(rows)]
    if exact:
        ok = oracle.bits_equal(got, c_ref, of)
        nbad = 0 if ok else int(np.sum(got != c_ref))
        return ok, 0.0, nbad
    return oracle.check(got, c_ref, sab, of, tol)


def sample_rows(M, n_random=16, seed=0, tile=256):
    rows = {0, 1, M - 1, M - 2}
    for edge in range(tile, M, tile * 7):
        rows.update({edge - 1, edge})
    rng = np.random.default_rng(seed)
    rows.update(int(v) for v in rng.integers(0, M, n_random))
    return np.array(sorted(r for r in rows if 0 <= r < M), dtype=np.int64)
