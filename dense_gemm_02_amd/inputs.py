"""Seeded synthetic operands for C = A x B.

This module only draws random numbers and stores them in an operand format;
it performs no step of the product itself.  Both the HIP path's tests/bench
and the CPU oracle's tests consume the arrays it returns.

Every generator uses ``numpy.random.default_rng(seed)`` (PCG64) and returns
raw storage bits as numpy arrays (uint32 for FP32, uint16 for FP16/BF16,
uint8 for FP8 E4M3), shaped in storage order:

* NN: A is M x K row-major, B is K x N row-major.
* TN: A is M x K row-major, B is K x N column-major, i.e. stored N x K.

Rounding recipes (each a library cast, round-to-nearest-even):

* FP32  : FP64 draw -> float32 (numpy).
* FP16  : FP64 draw -> float16 (numpy, one rounding from FP64).
* BF16  : FP64 draw -> float32 (numpy) -> bfloat16 (torch).
* E4M3  : FP64 draw -> float32 (numpy) -> float8_e4m3fn (torch, OCP E4M3).

Distributions follow the workloads: uniform[-1,1) FP32; N(0,1)/sqrt(K) for
FP16/BF16; uniform[-4,4) rounded to E4M3; +-1 with p = 1/2; and B = I.
Within one problem A is drawn before B from the same generator.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

DTYPES = ("f32", "f16", "bf16", "fp8")
_BITS = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16, "fp8": np.uint8}


@dataclass
class Problem:
    dtype: str          # "f32" | "f16" | "bf16" | "fp8"
    layout: str         # "nn" | "tn"
    M: int
    N: int
    K: int
    A: np.ndarray       # storage bits, 2-D (rows x ld)
    B: np.ndarray
    lda: int
    ldb: int
    ldc: int
    name: str = ""
    meta: dict = field(default_factory=dict)

    @property
    def flops(self) -> float:
        return 2.0 * self.M * self.N * self.K


def _to_bits(x64: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return x64.astype(np.float32).view(np.uint32)
    if dtype == "f16":
        return x64.astype(np.float16).view(np.uint16)
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x64.astype(np.float32)))
    if dtype == "bf16":
        return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if dtype == "fp8":
        return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().view(np.uint8)
    raise ValueError(dtype)


def draw(rng: np.random.Generator, shape, dist: str, dtype: str, K: int) -> np.ndarray:
    """One operand's storage bits.  dist: uniform | normal | uniform4 | pm1 | ones."""
    if dist == "uniform":
        x = rng.uniform(-1.0, 1.0, size=shape)
    elif dist == "normal":
        x = rng.standard_normal(size=shape) / np.sqrt(float(max(K, 1)))
    elif dist == "uniform4":
        x = rng.uniform(-4.0, 4.0, size=shape)
    elif dist == "pm1":
        x = rng.integers(0, 2, size=shape).astype(np.float64) * 2.0 - 1.0
    elif dist == "ones":
        x = np.ones(shape, dtype=np.float64)
    else:
        raise ValueError(dist)
    return _to_bits(x, dtype)


def storage_shapes(layout: str, M: int, N: int, K: int, lda: int, ldb: int):
    if layout == "nn":
        return (M, lda), (K, ldb)
    if layout == "tn":
        return (M, lda), (N, ldb)
    raise ValueError(layout)


def min_ld(layout: str, M: int, N: int, K: int):
    """Smallest legal (lda, ldb, ldc) for a layout."""
    if layout == "nn":
        return max(K, 1), max(N, 1), max(N, 1)
    return max(K, 1), max(K, 1), max(M, 1)


def make(dtype: str, layout: str, M: int, N: int, K: int, seed: int, dist: str,
         lda: int | None = None, ldb: int | None = None, ldc: int | None = None,
         rng: np.random.Generator | None = None, name: str = "") -> Problem:
    """A problem with A drawn before B.  Padding columns (ld beyond the
    logical extent) are filled with large garbage values so that a kernel
    reading past K or N shows up in the result."""
    la, lb, lc = min_ld(layout, M, N, K)
    lda = la if lda is None else lda
    ldb = lb if ldb is None else ldb
    ldc = lc if ldc is None else ldc
    rng = np.random.default_rng(seed) if rng is None else rng
    sa, sb = storage_shapes(layout, M, N, K, lda, ldb)
    A = draw(rng, sa, dist, dtype, K)
    B = draw(rng, sb, dist, dtype, K)
    kcols_a = K
    kcols_b = K if layout == "tn" else N
    garbage = {"f32": np.float32(1e30).view(np.uint32), "f16": np.uint16(0x7bff),
               "bf16": np.uint16(0x7f7f), "fp8": np.uint8(0x7e)}[dtype]
    if lda > kcols_a:
        A[:, kcols_a:] = garbage
    if ldb > kcols_b:
        B[:, kcols_b:] = garbage
    return Problem(dtype, layout, M, N, K, A, B, lda, ldb, ldc, name=name,
                   meta={"seed": seed, "dist": dist})


def identity(dtype: str, layout: str, n: int, A: np.ndarray, lda: int, ldb: int | None = None) -> Problem:
    """B = I (K = N = n) with the given A: C must equal A exactly."""
    one = {"f32": np.float32(1.0).view(np.uint32), "f16": np.uint16(0x3c00),
           "bf16": np.uint16(0x3f80), "fp8": np.uint8(0x38)}[dtype]
    ldb = n if ldb is None else ldb
    B = np.zeros((n, ldb), dtype=_BITS[dtype])
    B[np.arange(n), np.arange(n)] = one
    lc = n if layout == "nn" else A.shape[0]
    return Problem(dtype, layout, A.shape[0], n, n, A, B, lda, ldb, lc, name="identity")


# ---- the five workload families, with their seeds --------------------------

def workload(name: str) -> list[Problem]:
    """Named workloads.  Each entry is a list of problems in draw order."""
    if name == "f32_nn_256":
        p = make("f32", "nn", 256, 256, 256, 0, "uniform", name="f32_nn_256_uniform")
        return [p, identity("f32", "nn", 256, p.A, p.lda)]
    if name == "f32_nn_4096":
        p = make("f32", "nn", 4096, 4096, 4096, 1, "uniform", name="f32_nn_4096_uniform")
        return [p, identity("f32", "nn", 4096, p.A, p.lda)]
    if name == "f16_tn_8192_pm1":
        return [make("f16", "tn", 8192, 8192, 8192, 2, "pm1", name=name)]
    if name == "f16_tn_8192_normal":
        return [make("f16", "tn", 8192, 8192, 8192, 3, "normal", name=name)]
    if name.startswith("bf16_tn_"):
        M, N, K = (int(v) for v in name[len("bf16_tn_"):].split("x"))
        return [make("bf16", "tn", M, N, K, 4, "normal", name=name)]
    if name.startswith("fp8_tn_"):
        M, N, K = (int(v) for v in name[len("fp8_tn_"):].split("x"))
        rng = np.random.default_rng(5)
        a = make("fp8", "tn", M, N, K, 5, "uniform4", rng=rng, name=name + "_uniform4")
        b = make("fp8", "tn", M, N, K, 5, "pm1", rng=rng, name=name + "_pm1")
        return [a, b]
    raise KeyError(name)


BF16_SHAPES = [(4096, 14336, 4096), (4096, 4096, 14336), (8191, 8190, 8200), (16, 8192, 8192),
               (8192, 8192, 8192)]
FP8_SHAPES = [(8192, 8192, 8192), (4096, 14336, 4096), (4096, 4096, 14336), (8192, 28672, 8192)]
