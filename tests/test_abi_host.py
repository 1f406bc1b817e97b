"""Host-only checks of libdgemm.so: it loads, exports every declared symbol,
rejects bad arguments before touching the GPU, and its host helpers (tile map,
LDS sizing) behave as the pages' numbers say.  No kernel is launched here."""

import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")


@pytest.fixture(scope="module")
def lib():
    from dense_gemm_02_amd import binding
    if not os.path.exists(binding.library_path()):
        from dense_gemm_02_amd import build
        build.build()
    return binding.load_library()


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "dgemm.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(\w+)\s*\(", text)) - {"if", "defined"})


def test_exports_every_declared_symbol(lib):
    syms = declared_symbols()
    assert {"gemm_f32", "gemm_f16", "gemm_bf16", "gemm_fp8", "gemm_fp8_scaled", "gemm_mxfp8",
            "gemm_strerror"} <= set(syms)
    for s in syms:
        assert hasattr(lib, s), s


def test_strerror(lib):
    for st in range(8):
        assert lib.gemm_strerror(st)
    assert lib.gemm_strerror(99) == b"unknown status"


FAKE = 1 << 20            # 16-byte aligned fake device address; never dereferenced here


def call(lib, name, M, N, K, A, lda, B, ldb, C, ldc, layout):
    fn = getattr(lib, name)
    return fn(M, N, K, A, lda, B, ldb, C, ldc, layout, None)


@pytest.mark.parametrize("name,elem", [("gemm_f32", 4), ("gemm_f16", 2), ("gemm_bf16", 2), ("gemm_fp8", 1)])
def test_argument_validation_order(lib, name, elem):
    al = 16 // elem
    # layout first
    assert call(lib, name, -1, 4, 4, FAKE, al, FAKE, al, FAKE, 8, 7) == 4
    # negative dims
    assert call(lib, name, -1, 4, 4, FAKE, al, FAKE, al, FAKE, 8, 1) == 1
    assert call(lib, name, 4, 4, -3, FAKE, al, FAKE, al, FAKE, 8, 0) == 1
    # empty output: success without any work, even with null pointers and bad ld
    assert call(lib, name, 0, 4, 4, None, 0, None, 0, None, 0, 1) == 0
    assert call(lib, name, 4, 0, 4, None, 0, None, 0, None, 0, 0) == 0
    # null pointers
    assert call(lib, name, 4, 4, 4, None, al, FAKE, al, FAKE, 4, 1) == 2
    assert call(lib, name, 4, 4, 4, FAKE, al, None, al, FAKE, 4, 1) == 2
    assert call(lib, name, 4, 4, 4, FAKE, al, FAKE, al, None, 4, 1) == 2
    # ld below minimum: TN lda >= K, ldb >= K, ldc >= M; NN ldb >= N, ldc >= N
    assert call(lib, name, 4, 4, 2 * al, FAKE, al, FAKE, 2 * al, FAKE, 4, 1) == 3
    assert call(lib, name, 4, 4, al, FAKE, al, FAKE, al, FAKE, 3, 1) == 3
    assert call(lib, name, 4, 2 * al, al, FAKE, al, FAKE, al, FAKE, 2 * al, 0) == 3
    assert call(lib, name, 4, al, al, FAKE, al, FAKE, al, FAKE, al - 1, 0) == 3
    # misaligned A / B base, or pitch not a multiple of 16 bytes
    assert call(lib, name, 4, 4, al, FAKE + elem, al, FAKE, al, FAKE, 4, 1) == 5
    assert call(lib, name, 4, 4, al, FAKE, al, FAKE + 8, al, FAKE, 4, 1) == 5
    if al > 1:
        assert call(lib, name, 4, 4, al - 1, FAKE, al + 1, FAKE, al, FAKE, 4, 1) == 5
    # C only needs element alignment
    if elem < 4 or name == "gemm_fp8":
        oe = 4 if name in ("gemm_f32", "gemm_fp8") else 2
        if oe > 1:
            assert call(lib, name, 4, 4, al, FAKE, al, FAKE, al, FAKE + 1, 4, 1) == 5


def scaled(lib, M, N, K, A, lda, B, ldb, C, ldc, sa, na, sb, nb, layout):
    return lib.gemm_fp8_scaled(M, N, K, A, lda, B, ldb, C, ldc, sa, na, sb, nb, layout, None)


def test_scaled_argument_validation(lib):
    # the factor counts are checked with the dimensions, before the empty case
    assert scaled(lib, 4, 5, 16, FAKE, 16, FAKE, 16, FAKE, 4, FAKE, 4, FAKE, 5, 9) == 4
    assert scaled(lib, 4, 5, 16, FAKE, 16, FAKE, 16, FAKE, 4, FAKE, 2, FAKE, 5, 1) == 1
    assert scaled(lib, 4, 5, 16, FAKE, 16, FAKE, 16, FAKE, 4, FAKE, 4, FAKE, 4, 1) == 1
    assert scaled(lib, 4, 5, 16, FAKE, 16, FAKE, 16, FAKE, 4, FAKE, 0, FAKE, 1, 1) == 1
    assert scaled(lib, 0, 5, 16, None, 16, None, 16, None, 4, None, 1, None, 5, 1) == 0
    assert scaled(lib, 0, 5, 16, None, 16, None, 16, None, 4, None, 3, None, 5, 1) == 1
    # null and misaligned factor pointers
    assert scaled(lib, 4, 5, 16, FAKE, 16, FAKE, 16, FAKE, 4, None, 1, FAKE, 5, 1) == 2
    assert scaled(lib, 4, 5, 16, FAKE, 16, FAKE, 16, FAKE, 4, FAKE, 4, None, 1, 1) == 2
    assert scaled(lib, 4, 5, 16, FAKE, 16, FAKE, 16, FAKE, 4, FAKE + 2, 1, FAKE, 5, 1) == 5
    assert scaled(lib, 4, 5, 16, FAKE, 16, FAKE, 16, FAKE, 8, FAKE, 1, FAKE + 1, 1, 0) == 5
    # the operand checks of gemm_fp8 still apply
    assert scaled(lib, 4, 5, 16, FAKE, 8, FAKE, 16, FAKE, 4, FAKE, 1, FAKE, 1, 1) == 3
    assert scaled(lib, 4, 5, 16, FAKE + 4, 16, FAKE, 16, FAKE, 4, FAKE, 1, FAKE, 1, 1) == 5


def mx(lib, M, N, K, A, lda, B, ldb, C, ldc, sa, ldsa, sb, ldsb, layout):
    return lib.gemm_mxfp8(M, N, K, A, lda, B, ldb, C, ldc, sa, ldsa, sb, ldsb, layout, None)


def test_mxfp8_argument_validation(lib):
    # K must be a whole number of 32-element blocks (checked with the dimensions)
    assert mx(lib, 4, 5, 48, FAKE, 48, FAKE, 48, FAKE, 4, FAKE, 16, FAKE, 16, 1) == 1
    assert mx(lib, 0, 5, 48, None, 48, None, 48, None, 4, None, 16, None, 16, 1) == 1
    assert mx(lib, 0, 5, 64, None, 64, None, 64, None, 4, None, 16, None, 16, 1) == 0
    assert mx(lib, 4, 5, 64, FAKE, 64, FAKE, 64, FAKE, 4, FAKE, 16, FAKE, 16, 7) == 4
    # null scale pointers
    assert mx(lib, 4, 5, 64, FAKE, 64, FAKE, 64, FAKE, 4, None, 16, FAKE, 16, 1) == 2
    assert mx(lib, 4, 5, 64, FAKE, 64, FAKE, 64, FAKE, 4, FAKE, 16, None, 16, 1) == 2
    # scale rows shorter than K/32
    assert mx(lib, 4, 5, 1024, FAKE, 1024, FAKE, 1024, FAKE, 4, FAKE, 16, FAKE, 32, 1) == 3
    assert mx(lib, 4, 5, 1024, FAKE, 1024, FAKE, 1024, FAKE, 4, FAKE, 32, FAKE, 16, 1) == 3
    # 16-byte alignment of the scale arrays and their rows
    assert mx(lib, 4, 5, 64, FAKE, 64, FAKE, 64, FAKE, 4, FAKE + 4, 16, FAKE, 16, 1) == 5
    assert mx(lib, 4, 5, 64, FAKE, 64, FAKE, 64, FAKE, 4, FAKE, 16, FAKE, 8, 1) == 5
    # a 256-row block of scales spanning 2^31 bytes
    assert mx(lib, 4, 5, 64, FAKE, 64, FAKE, 64, FAKE, 4, FAKE, 1 << 23, FAKE, 16, 1) == 6


def test_size_limits_unsupported(lib):
    # a K-contiguous operand whose 256-row block would span >= 2^31 bytes
    # (M = 300 selects the block-tiled kernel; the call must be rejected
    # before anything touches the fake pointers)
    big = (1 << 23) + 8
    assert call(lib, "gemm_bf16", 300, 4, 8, FAKE, big, FAKE, 8, FAKE, 300, 1) == 6


def tile_map(lib, tp, tq, g, pid):
    a, b = ctypes.c_int64(), ctypes.c_int64()
    rc = lib.dgemm_tile_map(tp, tq, g, pid, ctypes.byref(a), ctypes.byref(b))
    return rc, a.value, b.value


@pytest.mark.parametrize("tp,tq,g", [(1, 1, 8), (32, 32, 8), (3, 5, 8), (7, 13, 4), (16, 56, 8), (33, 31, 8),
                                     (1, 100, 8), (100, 1, 8), (64, 4, 3), (13, 17, 1), (9, 9, 16)])
def test_tile_map_is_a_bijection(lib, tp, tq, g):
    seen = set()
    for pid in range(tp * tq):
        rc, a, b = tile_map(lib, tp, tq, g, pid)
        assert rc == 0 and 0 <= a < tp and 0 <= b < tq
        seen.add((a, b))
    assert len(seen) == tp * tq
    assert tile_map(lib, tp, tq, g, tp * tq)[0] == -1


def test_tile_map_keeps_xcd_neighbours_together(lib):
    # 32 x 32 tiles, group 8: the 32 blocks that one XCD runs first (pid = x + 8*t)
    # form an 8 x 4 patch of tiles -- 8 p-panels and 4 q-panels.
    for xcd in range(8):
        tiles = [tile_map(lib, 32, 32, 8, xcd + 8 * t)[1:] for t in range(32)]
        ps = {a for a, _ in tiles}
        qs = {b for _, b in tiles}
        assert len(ps) == 8 and len(qs) == 4


def load_golden(name):
    rows = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#", 1)[0].strip()
        if line:
            rows.append([int(v) for v in line.split()])
    return rows


def test_lds_bytes_matches_the_pages(lib):
    rows = load_golden("lds_sizes.txt")
    assert len(rows) >= 8
    for bm, bn, bk, elem, pad, bufs, expect in rows:
        assert lib.dgemm_lds_bytes(bm, bn, bk, elem, pad, bufs) == expect


def test_kernel_config_description(lib):
    buf = ctypes.create_string_buffer(256)
    assert lib.dgemm_kernel_config(2, 1, 8192, 8192, 8192, buf, 256) == 0
    d = buf.value.decode()
    assert "bf16_tn" in d and "grid=1024" in d
    assert lib.dgemm_kernel_config(0, 0, 4096, 4096, 4096, buf, 256) == 0
    assert "f32_nn" in buf.value.decode()
    assert lib.dgemm_kernel_config(1, 1, 0, 5, 5, buf, 256) == 0
    assert lib.dgemm_kernel_config(1, 9, 5, 5, 5, buf, 256) == 4


def _kernel(lib, dt, layout, M, N, K):
    buf = ctypes.create_string_buffer(256)
    assert lib.dgemm_kernel_config(dt, layout, M, N, K, buf, 256) == 0
    return buf.value.decode()


@pytest.mark.parametrize("layout,M,N,K,tile", [
    (0, 256, 256, 256, "64x64"),         # 4 tiles of 128^2 -> 16 of 64^2
    (1, 256, 256, 256, "64x64"),
    (0, 1024, 1024, 1024, "64x64"),      # 64 < 128 tiles of 128^2
    (0, 1408, 1408, 64, "64x64"),        # 11^2 = 121 tiles of 128^2
    (0, 1536, 1408, 64, "128x128"),      # 12 x 11 = 132
    (0, 2048, 2048, 2048, "128x128"),
    (1, 4096, 4096, 4096, "128x128"),
])
def test_f32_tile_by_grid(lib, layout, M, N, K, tile):
    d = _kernel(lib, 0, layout, M, N, K)
    assert d.startswith(f"f32_{'tn' if layout else 'nn'}_{tile}"), d


# Tile choice (TN 256 x 256 runs the eight-wave ping-pong kernel, every other
# tile the four-wave kernel): rounds of workgroups over 256 CUs
# times the time of one round. 256 x 256 tiles cost 1 per round, 128 x 128
# ones (two per CU, two stages) 1/0.78 * 1/2, 256 x 128 ones 1/0.76 * 1/2;
# 128 x 128 with four stages (one per CU) 1/0.47 * 1/4, for one round only;
# 192 x 256 (TN) and 256 x 192 (K >= 4096) 1/0.87 * 3/4, for one round only.
@pytest.mark.parametrize("M,N,K,tile16,tile8nn,tile16tn", [
    (8192, 8192, 8192, "256x256_w4", "256x256_w4", None),  # 1024 tiles: 4 rounds vs 8 of 128 x 128, 6 of 192 x 256
    (4096, 4096, 4096, "256x256_w4", "256x256_w4", None),  # one full round vs two
    # 192 tiles of 256 x 256: one round (1) vs 256 of 192 x 256 or 256 x 192 (0.86); NN (p along N) has 256 x 192 only
    (3072, 4096, 8192, "256x256_w4", "256x256_w4", ("192x256_w4", "256x192_w4")),
    (1536, 8192, 8192, "256x256_w4", "256x256_w4", ("192x256_w4", "256x192_w4")),
    (4096, 3072, 8192, "256x256_w4", "256x256_w4", ("256x192_w4", "256x256_w4")),
    (5120, 5120, 1024, "256x256_w4", "256x256_w4", None),  # 400 tiles: 2 rounds (2) vs 4 (2.56)
    (3072, 4096, 2048, "256x256_w4", "256x256_w4", None),  # below K = 4096 no 192 x 256
    (2560, 2304, 4096, "128x128_w4", "256x128_w4", None),  # 360 tiles of 128 x 128: one round at two per CU
    (2048, 2048, 2048, "128x128_w4_s4", "256x128_w4", None),  # 256 tiles of 128 x 128, one per CU
    (300, 521, 512, "128x128_w4_s4", "256x128_w4", None),
])
def test_tile_choice(lib, M, N, K, tile16, tile8nn, tile16tn):
    for dt in (1, 2, 3, 4, 5):
        for layout in (0, 1):
            full = _kernel(lib, dt, layout, M, N, K)
            d = full.split()[0]
            want = tile8nn if dt >= 3 and layout == 0 else tile16
            if tile16tn:
                want = tile16tn[0] if layout == 1 else tile16tn[1]
            if dt == 5 and want.endswith("_s4"):
                want = want[:-3]          # MXFP8 keeps two LDS stages (its scale ring)
            if want == "256x256_w4" and layout == 1 and dt != 5:
                want = "256x256_pp"       # TN 256 x 256: the eight-wave ping-pong kernel
            assert d.endswith(want), (dt, layout, full)
            assert " + " not in full, full


# A 256 x 256 grid that ends in a partial round: its whole rounds run as one
# launch over the first part of q (TN: columns of C) or p, the rest as a
# second launch with the tile the table picks for it.
# (TN with the eight-wave main launch splits only when the last round is
# less than half full.)
@pytest.mark.parametrize("dt,layout,M,N,K,axis,at,tail", [
    (5, 1, 4096, 14336, 4096, "q", 12288, "mx8_tn_128x128_w4"),     # 896 tiles: 3 rounds + 4096 x 2048
    (2, 0, 4096, 14336, 4096, "p", 12288, "bf16_nn_128x128_w4"),    # NN: p runs along N
    (3, 0, 4096, 14336, 4096, "p", 12288, "fp8_nn_256x128_w4"),
    (1, 0, 6144, 6144, 4096, "q", 5376, "f16_nn_128x128_w4"),        # 576 tiles: 504 + 48 x 6 of 128
    (2, 1, 6144, 6144, 4096, "q", 5376, "bf16_tn_128x128_w4"),       # TN, last round a quarter full
    (2, 1, 4352, 4352, 1024, "q", 3840, "bf16_tn_128x128_w4_s4"),    # 289 tiles: 255 + 136 of 128, one per CU
    (4, 1, 2560, 14336, 2048, "q", 13056, "fp8s_tn_128x128_w4_s4"),  # (K >= 4096: 750 tiles of 256 x 192)
    (5, 1, 5120, 5120, 4096, "q", 3072, "mx8_tn_192x256_w4"),        # 400 tiles: 240 + 216 of 192 x 256
])
def test_split_choice(lib, dt, layout, M, N, K, axis, at, tail):
    full = _kernel(lib, dt, layout, M, N, K)
    main, rest = full.split(" + ")
    big = "256x256_pp" if layout == 1 and dt != 5 else "256x256_w4"
    assert main.split()[0].endswith(big), full
    assert rest.split()[0] == tail, full
    assert rest.endswith(f"from {axis}={at}"), full


@pytest.mark.parametrize("dt,M,N,K", [
    (2, 4096, 14336, 4096), (3, 4096, 14336, 4096),   # 896 tiles: last round half full
    (2, 14336, 4096, 4096), (2, 5120, 5120, 4096),    # 1.56 rounds
    (1, 3584, 8192, 8192),                            # 1.75 rounds
])
def test_tn_single_launch_when_the_last_round_is_half_full(lib, dt, M, N, K):
    k = _kernel(lib, dt, 1, M, N, K)
    assert " + " not in k and "_256x256_pp " in k, k


@pytest.mark.parametrize("M,N,K", [(8192, 8192, 8192), (3584, 8192, 2048), (8191, 8190, 8200), (3072, 4096, 8192)])
def test_no_split_when_rounds_are_whole_or_it_does_not_pay(lib, M, N, K):
    for dt in (1, 2, 3):
        assert " + " not in _kernel(lib, dt, 1, M, N, K)
    # 256 x 256 runs one tile per workgroup for every dtype (16 x 16 MFMA
    # tiles): the grid is the tile count.
    for dt, name in ((3, "fp8_tn_256x256_pp"), (5, "mx8_tn_256x256_w4")):
        k = _kernel(lib, dt, 1, 5120, 5120, 1024)
        assert k.split()[0] == name and "grid=400 " in k, k
    # K not a whole number of 16-byte chunks: the eight-wave kernel.
    assert "_w4" not in _kernel(lib, 2, 1, 4096, 4096, 4100)


def test_matmul_rejects_host_and_mismatched_tensors():
    import torch
    from dense_gemm_02_amd import matmul
    with pytest.raises(TypeError):
        matmul(torch.ones(2, 3), torch.ones(3, 4))
    with pytest.raises(TypeError):
        matmul(np.ones((2, 3)), np.ones((3, 4)))


# ---- tensor-level binding checks (host side, no GPU work) --------------------

def test_binding_rejects_host_tensors():
    import torch
    from dense_gemm_02_amd import binding
    a = torch.zeros(64, dtype=torch.int16)
    f = torch.ones(1)
    with pytest.raises(TypeError):
        binding.gemm("bf16", "tn", 8, 8, 8, a, 8, a, 8, a, 8)
    u8, c32 = torch.zeros(64, dtype=torch.uint8), torch.zeros(64, dtype=torch.int32)
    with pytest.raises(TypeError):
        binding.gemm_scaled("tn", 8, 8, 8, u8, 8, u8, 8, c32, 8, f, f)
    with pytest.raises(TypeError):
        binding.gemm_mx("tn", 8, 8, 32, u8, 32, u8, 32, c32, 8, u8, 16, u8, 16)


@pytest.mark.parametrize("layout", ["nn", "tn"])
def test_binding_extent_checks(layout):
    import torch
    from dense_gemm_02_amd import binding
    M, N, K, lda, ldb, ldc = 5, 7, 16, 24, 32, 9

    def t(n, dtype=torch.int16):
        return torch.zeros(n, dtype=dtype)

    nb_rows = K if layout == "nn" else N
    c_last = (M - 1) * ldc + N if layout == "nn" else (N - 1) * ldc + M
    ok = dict(A=t(M * lda), B=t(nb_rows * ldb), C=t(c_last))
    binding._check_extents(layout, M, N, K, ok["A"], lda, ok["B"], ldb, ok["C"], ldc, 2, 2)
    for which, short in (("A", t(M * lda - 1)), ("B", t(nb_rows * ldb - 1)), ("C", t(c_last - 1))):
        args = dict(ok, **{which: short})
        with pytest.raises(ValueError, match=which):
            binding._check_extents(layout, M, N, K, args["A"], lda, args["B"], ldb, args["C"], ldc, 2, 2)
    # a view that starts inside its storage counts only what follows it
    big = t(M * lda + 8)
    binding._check_extents(layout, M, N, K, big[8:], lda, ok["B"], ldb, ok["C"], ldc, 2, 2)
    with pytest.raises(ValueError):
        binding._check_extents(layout, M, N, K, big[9:], lda, ok["B"], ldb, ok["C"], ldc, 2, 2)
    # nothing is read at K = 0, nothing at all for an empty output
    binding._check_extents(layout, M, N, 0, t(0), lda, t(0), ldb, ok["C"], ldc, 2, 2)
    binding._check_extents(layout, 0, N, K, t(0), lda, t(0), ldb, t(0), ldc, 2, 2)


def test_binding_factor_checks():
    import torch
    from dense_gemm_02_amd import binding
    binding._factor_vector(torch.ones(1), 9, "scale_a")
    binding._factor_vector(torch.ones(9), 9, "scale_a")
    with pytest.raises(TypeError):
        binding._factor_vector(torch.ones(9, dtype=torch.float64), 9, "scale_a")
    with pytest.raises(TypeError):
        binding._factor_vector(torch.ones(9, dtype=torch.bfloat16), 9, "scale_a")
    with pytest.raises(TypeError):
        binding._factor_vector(torch.ones(18)[::2], 9, "scale_a")
    with pytest.raises(ValueError):
        binding._factor_vector(torch.ones(8), 9, "scale_a")


def test_binding_declares_every_entry_point():
    # ctypes passes an undeclared argument as a C int: a 64-bit device
    # pointer would be cut to its low 32 bits.  Every function the header
    # declares must have its argument and result types set by the binding,
    # one per parameter, a pointer type wherever the header has a pointer.
    from dense_gemm_02_amd import binding
    L = binding.load_library()
    hdr = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "dgemm.h")).read(), flags=re.S)
    decls = re.findall(r"^\s*(?:int|int64_t|const char\*)\s+(\w+)\(([^)]*)\);", hdr, re.M)
    assert len(decls) >= 13
    for name, params in decls:
        fn = getattr(L, name)
        assert fn.argtypes is not None and fn.restype is not None, name
        ps = [p.strip() for p in params.split(",") if p.strip() and p.strip() != "void"]
        assert len(fn.argtypes) == len(ps), name
        for p, t in zip(ps, fn.argtypes):
            is_ptr = t in (ctypes.c_void_p, ctypes.c_char_p) or t.__name__.startswith("LP_")
            assert is_ptr == ("*" in p), (name, p, t)
