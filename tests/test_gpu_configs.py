"""GPU parity at the five workload configurations' full sizes, in the launch
configuration the benchmark times.  The GPU computes every element and every
element is compared with the oracle: at these sizes through its
library-product leg (the definition of the triple loop with the FP64 sum
taken by a library matrix product, pinned to the loop bit for bit), block by
block.  Bit-exact on +-1 inputs and B = I; otherwise within the per-format
tolerance on |c - c_ref| / sum_k |a b|.

Workloads: FP32 NN 256^3 and 4096^3 (uniform[-1,1), seeds 0 and 1, plus
B = I); FP16 TN 8192^3 (+-1 seed 2, N(0,1)/sqrt(K) seed 3); BF16 TN at
(4096,14336,4096), (4096,4096,14336), (8191,8190,8200), (16,8192,8192) and
8192^3 (N(0,1)/sqrt(K), seed 4); FP8 TN at 8192^3, (4096,14336,4096),
(4096,4096,14336), (8192,28672,8192) (uniform[-4,4) then +-1, seed 5)."""

import time

import numpy as np
import pytest

from dense_gemm_02_amd import inputs
from gpu_util import c_host, compare, oracle, run_gpu, say, to_dev

pytestmark = pytest.mark.gpu


def _check(p, exact):
    say(f"case {p.name} M={p.M} N={p.N} K={p.K} exact={exact}")
    C = run_gpu(p)
    cij, pad = c_host(p, C)
    t0 = time.perf_counter()
    ok, err, nbad = compare(p, cij, exact=exact)
    assert ok, f"{p.name}: max err {err:.3e}, {nbad} elements bad"
    say(f"  ok max_err={err:.3e} (oracle {time.perf_counter() - t0:.1f} s)")
    return C


def test_f32_nn_256_full():
    p, ident = inputs.workload("f32_nn_256")
    _check(p, exact=False)
    C = run_gpu(ident)
    cij, _ = c_host(ident, C)
    assert oracle.bits_equal(cij, p.A, oracle.F32)


def test_f32_nn_4096():
    p, ident = inputs.workload("f32_nn_4096")
    _check(p, exact=False)
    import torch
    C = run_gpu(ident)
    A = to_dev(p.A)
    assert torch.equal(C, A), "B = I must give C = A exactly"


def test_f16_tn_8192_pm1():
    (p,) = inputs.workload("f16_tn_8192_pm1")
    _check(p, exact=True)


def test_f16_tn_8192_normal():
    (p,) = inputs.workload("f16_tn_8192_normal")
    _check(p, exact=False)


@pytest.mark.parametrize("shape", inputs.BF16_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_bf16_tn(shape):
    (p,) = inputs.workload("bf16_tn_%dx%dx%d" % shape)
    _check(p, exact=False)


@pytest.mark.parametrize("shape", inputs.FP8_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_fp8_tn(shape):
    a, b = inputs.workload("fp8_tn_%dx%dx%d" % shape)
    _check(a, exact=False)
    _check(b, exact=True)
