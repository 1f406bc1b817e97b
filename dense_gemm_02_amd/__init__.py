"""MI355X (gfx950) tiled dense GEMM: C = A x B in FP32, FP16, BF16 and FP8 E4M3
with FP32 accumulation, behind the C-ABI library ``libdgemm.so``.

The compute path is hand-written HIP in ``csrc/``; this package only marshals
arguments to it (``dense_gemm_02_amd.binding``).  Importing the package does
not load the library; the first call does, and fails loudly if it is missing.
"""

from .binding import (gemm, gemm_f32, gemm_f16, gemm_bf16, gemm_fp8, gemm_fp8_scaled, gemm_mxfp8,  # noqa: F401
                      gemm_scaled, gemm_mx, matmul, gemm_strerror, DgemmError, library_path, load_library)
