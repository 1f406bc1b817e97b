"""GPU parity at the five workload configurations' full sizes, in the launch
configuration the benchmark times.  The GPU computes every element; the
oracle recomputes a seeded sample of whole rows (every column, so every
q tile), and properties that hold at any size are checked on all of C:

* +-1 inputs: every element is an integer, |c| <= K and c = K (mod 2);
* B = I: C equals A bit for bit.

Workloads: FP32 NN 256^3 and 4096^3 (uniform[-1,1), seeds 0 and 1, plus
B = I); FP16 TN 8192^3 (+-1 seed 2, N(0,1)/sqrt(K) seed 3); BF16 TN at
(4096,14336,4096), (4096,4096,14336), (8191,8190,8200), (16,8192,8192) and
8192^3 (N(0,1)/sqrt(K), seed 4); FP8 TN at 8192^3, (4096,14336,4096),
(4096,4096,14336), (8192,28672,8192) (uniform[-4,4) then +-1, seed 5)."""

import numpy as np
import pytest

from dense_gemm_02_amd import inputs
from gpu_util import c_host, compare, oracle, run_gpu, sample_rows, say, to_dev

pytestmark = pytest.mark.gpu


def _full_props_pm1(p, C):
    import torch
    v = C.view(torch.float32) if p.dtype in ("f32", "fp8") else (
        C.view(torch.float16) if p.dtype == "f16" else C.view(torch.bfloat16))
    v = v[:, :p.M] if p.layout == "tn" else v[:, :p.N]
    v = v.float()
    assert bool(torch.isfinite(v).all())
    assert bool((v == torch.round(v)).all())
    assert float(v.abs().max()) <= p.K
    assert bool((torch.remainder(v - p.K, 2) == 0).all())


def _check(p, rows, exact):
    say(f"case {p.name} M={p.M} N={p.N} K={p.K} rows={len(rows)}")
    C = run_gpu(p)
    cij, pad = c_host(p, C)
    ok, err, nbad = compare(p, cij, rows=rows, exact=exact)
    assert ok, f"{p.name}: max err {err:.3e}, {nbad} bad in sampled rows"
    say(f"  ok max_err={err:.3e}")
    return C


def test_f32_nn_256_full():
    p, ident = inputs.workload("f32_nn_256")
    _check(p, np.arange(256), exact=False)
    C = run_gpu(ident)
    cij, _ = c_host(ident, C)
    assert oracle.bits_equal(cij, p.A, oracle.F32)


def test_f32_nn_4096():
    p, ident = inputs.workload("f32_nn_4096")
    _check(p, sample_rows(4096, tile=128), exact=False)
    import torch
    C = run_gpu(ident)
    A = to_dev(p.A)
    assert torch.equal(C, A), "B = I must give C = A exactly"


def test_f16_tn_8192_pm1():
    (p,) = inputs.workload("f16_tn_8192_pm1")
    C = _check(p, sample_rows(8192, n_random=8), exact=True)
    _full_props_pm1(p, C)


def test_f16_tn_8192_normal():
    (p,) = inputs.workload("f16_tn_8192_normal")
    _check(p, sample_rows(8192, n_random=8), exact=False)


@pytest.mark.parametrize("shape", inputs.BF16_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_bf16_tn(shape):
    (p,) = inputs.workload("bf16_tn_%dx%dx%d" % shape)
    _check(p, sample_rows(p.M, n_random=8), exact=False)


@pytest.mark.parametrize("shape", inputs.FP8_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_fp8_tn(shape):
    a, b = inputs.workload("fp8_tn_%dx%dx%d" % shape)
    _check(a, sample_rows(a.M, n_random=6), exact=False)
    C = _check(b, sample_rows(b.M, n_random=4), exact=True)
    _full_props_pm1(b, C)
