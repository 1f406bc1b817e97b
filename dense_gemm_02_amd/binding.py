"""ctypes binding of ``libdgemm.so`` (declared in ``include/dgemm.h``).

Argument marshalling only: every step of the product runs in the library's
HIP kernels.  PyTorch supplies device memory and the current HIP stream.
There is no fallback: if the library is missing or a call fails, a
``DgemmError`` is raised.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIBNAME = "libdgemm.so"

DGEMM_NN, DGEMM_TN = 0, 1
_LAYOUTS = {"nn": DGEMM_NN, "tn": DGEMM_TN}


class DgemmError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        msg = f"{what}: {gemm_strerror(status)} (status {status})"
        if status == 7 and _lib is not None:
            code = _lib.dgemm_last_hip_error()
            msg += f" [hipError {code}: {_lib.dgemm_hip_error_string(code).decode()}]"
        super().__init__(msg)


def library_path() -> str:
    return os.path.join(_HERE, _LIBNAME)


_lib = None


def load_library():
    """Load libdgemm.so (built by ``__graft_entry__.build()``); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run __graft_entry__.build() first")
    # One HIP runtime per process.  PyTorch ships its own copy of the HIP
    # runtime (soname libamdhip64.so.7) and loads it by another file name, so
    # if libdgemm.so came first the process would hold two runtimes, and the
    # one initialised second finds no device (hipErrorNoDevice at launch).
    # With torch loaded first, libdgemm.so binds to torch's copy by soname.
    import torch  # noqa: F401
    L = ctypes.CDLL(path)
    i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    for name in ("gemm_f32", "gemm_f16", "gemm_bf16", "gemm_fp8"):
        fn = getattr(L, name)
        fn.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, ci, vp]
        fn.restype = ci
    L.gemm_fp8_scaled.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, vp, i64, vp, i64, ci, vp]
    L.gemm_fp8_scaled.restype = ci
    L.gemm_mxfp8.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, vp, i64, vp, i64, ci, vp]
    L.gemm_mxfp8.restype = ci
    L.dgemm_last_hip_error.argtypes = []
    L.dgemm_last_hip_error.restype = ci
    L.dgemm_hip_error_string.argtypes = [ci]
    L.dgemm_hip_error_string.restype = ctypes.c_char_p
    L.gemm_strerror.argtypes = [ci]
    L.gemm_strerror.restype = ctypes.c_char_p
    L.dgemm_tile_map.argtypes = [i64, i64, i64, i64, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    L.dgemm_tile_map.restype = ci
    L.dgemm_lds_bytes.argtypes = [ci, ci, ci, ci, ci, ci]
    L.dgemm_lds_bytes.restype = i64
    L.dgemm_kernel_config.argtypes = [ci, ci, i64, i64, i64, ctypes.c_char_p, i64]
    L.dgemm_kernel_config.restype = ci
    L.dgemm_trace_clock.argtypes = [vp, i64]
    L.dgemm_trace_clock.restype = ci
    _lib = L
    return L


def gemm_strerror(status: int) -> str:
    try:
        return load_library().gemm_strerror(int(status)).decode()
    except ImportError:
        return "unknown status"


def _stream_handle(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _raw(fn_name, M, N, K, A, lda, B, ldb, C, ldc, layout, stream):
    L = load_library()
    lay = _LAYOUTS.get(layout, layout) if isinstance(layout, str) else layout
    st = getattr(L, fn_name)(int(M), int(N), int(K), A, int(lda), B, int(ldb), C, int(ldc),
                             int(lay), _stream_handle(stream))
    if st != 0:
        raise DgemmError(st, fn_name)


def gemm_f32(M, N, K, A, lda, B, ldb, C, ldc, layout="nn", stream=None):
    """Raw-pointer call: A, B, C are device addresses (ints)."""
    _raw("gemm_f32", M, N, K, A, lda, B, ldb, C, ldc, layout, stream)


def gemm_f16(M, N, K, A, lda, B, ldb, C, ldc, layout="tn", stream=None):
    _raw("gemm_f16", M, N, K, A, lda, B, ldb, C, ldc, layout, stream)


def gemm_bf16(M, N, K, A, lda, B, ldb, C, ldc, layout="tn", stream=None):
    _raw("gemm_bf16", M, N, K, A, lda, B, ldb, C, ldc, layout, stream)


def gemm_fp8(M, N, K, A, lda, B, ldb, C, ldc, layout="tn", stream=None):
    _raw("gemm_fp8", M, N, K, A, lda, B, ldb, C, ldc, layout, stream)


def gemm_fp8_scaled(M, N, K, A, lda, B, ldb, C, ldc, scale_a, n_scale_a, scale_b, n_scale_b, layout="tn",
                    stream=None):
    """Raw-pointer call with FP32 scale factors (device addresses): n_scale_a
    is 1 (per tensor) or M (per row of A), n_scale_b is 1 or N (per column
    of B)."""
    L = load_library()
    lay = _LAYOUTS.get(layout, layout) if isinstance(layout, str) else layout
    st = L.gemm_fp8_scaled(int(M), int(N), int(K), A, int(lda), B, int(ldb), C, int(ldc), scale_a, int(n_scale_a),
                           scale_b, int(n_scale_b), int(lay), _stream_handle(stream))
    if st != 0:
        raise DgemmError(st, "gemm_fp8_scaled")


def gemm_mxfp8(M, N, K, A, lda, B, ldb, C, ldc, scale_a, ldsa, scale_b, ldsb, layout="tn", stream=None):
    """Raw-pointer call with E8M0 block scales (device addresses): byte
    scale_a[i*ldsa + b] scales k block b of row i of A, scale_b[j*ldsb + b]
    block b of column j of B."""
    L = load_library()
    lay = _LAYOUTS.get(layout, layout) if isinstance(layout, str) else layout
    st = L.gemm_mxfp8(int(M), int(N), int(K), A, int(lda), B, int(ldb), C, int(ldc), scale_a, int(ldsa), scale_b,
                      int(ldsb), int(lay), _stream_handle(stream))
    if st != 0:
        raise DgemmError(st, "gemm_mxfp8")


_BY_DTYPE = {"f32": gemm_f32, "f16": gemm_f16, "bf16": gemm_bf16, "fp8": gemm_fp8}
_ELEM = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1}


def _bytes_after(t) -> int:
    """Bytes of t's storage from its first element to the end of the storage."""
    return t.untyped_storage().nbytes() - t.storage_offset() * t.element_size()


def _need(t, nbytes, what):
    if nbytes > 0 and _bytes_after(t) < nbytes:
        raise ValueError(f"{what} holds {_bytes_after(t)} bytes from its first element, the call reads or "
                         f"writes {nbytes}")


def _check_extents(layout, M, N, K, A, lda, B, ldb, C, ldc, ein, eout):
    """The extents include/dgemm.h requires of the caller's memory: A over
    M*lda elements and B over K*ldb (NN) or N*ldb (TN) when K > 0 (whole rows
    of the pitch: the kernels copy 16-byte pieces), and C over the last
    element written, (M-1)*ldc + N (NN) or (N-1)*ldc + M (TN)."""
    if M <= 0 or N <= 0:
        return
    if K > 0:
        _need(A, M * lda * ein, "A")
        _need(B, (K if layout in ("nn", DGEMM_NN) else N) * ldb * ein, "B")
    last = (M - 1) * ldc + N if layout in ("nn", DGEMM_NN) else (N - 1) * ldc + M
    _need(C, last * eout, "C")


def _device_tensors(names, *ts):
    import torch
    for t in ts:
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise TypeError(f"{names} must be device tensors")


def _factor_vector(t, n, what):
    import torch
    if t.dtype != torch.float32 or not t.is_contiguous():
        raise TypeError(f"{what} must be a contiguous float32 tensor")
    if t.numel() not in (1, n):
        raise ValueError(f"{what} holds {t.numel()} values, not 1 or {n}")


def gemm(dtype, layout, M, N, K, A, lda, B, ldb, C, ldc, stream=None):
    """Tensor-level call.  A, B, C are torch device tensors holding the
    operands' storage (any integer or float dtype of the right width); the
    leading dimensions are in elements.  The storage behind each tensor must
    cover what the call reads or writes (checked here)."""
    _device_tensors("A, B and C", A, B, C)
    ebytes = _ELEM[dtype]
    if A.element_size() != ebytes or B.element_size() != ebytes:
        raise TypeError(f"{dtype} operands need {ebytes}-byte elements")
    cbytes = 4 if dtype in ("f32", "fp8") else 2
    if C.element_size() != cbytes:
        raise TypeError(f"{dtype} output needs {cbytes}-byte elements")
    _check_extents(layout, M, N, K, A, lda, B, ldb, C, ldc, ebytes, cbytes)
    _BY_DTYPE[dtype](M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, C.data_ptr(), ldc, layout, stream)


def gemm_scaled(layout, M, N, K, A, lda, B, ldb, C, ldc, scale_a, scale_b, stream=None):
    """Tensor-level FP8 call with scale factors: A, B hold E4M3 bytes, C FP32
    storage, scale_a / scale_b are contiguous FP32 device tensors of 1 or M /
    1 or N values."""
    _device_tensors("A, B, C and the scale factors", A, B, C, scale_a, scale_b)
    if A.element_size() != 1 or B.element_size() != 1 or C.element_size() != 4:
        raise TypeError("fp8 operands need 1-byte elements and a 4-byte output")
    _factor_vector(scale_a, M, "scale_a")
    _factor_vector(scale_b, N, "scale_b")
    _check_extents(layout, M, N, K, A, lda, B, ldb, C, ldc, 1, 4)
    gemm_fp8_scaled(M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, C.data_ptr(), ldc, scale_a.data_ptr(),
                    scale_a.numel(), scale_b.data_ptr(), scale_b.numel(), layout, stream)


def gemm_mx(layout, M, N, K, A, lda, B, ldb, C, ldc, scale_a, ldsa, scale_b, ldsb, stream=None):
    """Tensor-level MXFP8 call: A, B hold E4M3 bytes, C FP32 storage,
    scale_a / scale_b E8M0 bytes (device tensors covering M*ldsa / N*ldsb
    bytes) with row pitches ldsa / ldsb."""
    _device_tensors("A, B, C and the block scales", A, B, C, scale_a, scale_b)
    if A.element_size() != 1 or B.element_size() != 1 or C.element_size() != 4:
        raise TypeError("fp8 operands need 1-byte elements and a 4-byte output")
    if scale_a.element_size() != 1 or scale_b.element_size() != 1:
        raise TypeError("block scales are bytes")
    _check_extents(layout, M, N, K, A, lda, B, ldb, C, ldc, 1, 4)
    if M > 0 and N > 0 and K > 0:
        _need(scale_a, M * ldsa, "scale_a")
        _need(scale_b, N * ldsb, "scale_b")
    gemm_mxfp8(M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, C.data_ptr(), ldc, scale_a.data_ptr(), ldsa,
               scale_b.data_ptr(), ldsb, layout, stream)


def trace_clock(buf):
    """Set (an int64 device tensor of 4 * n values, n workgroups) or clear
    (None) the calling thread's clock trace: later four-wave launches record
    each workgroup's start and end stamps of the core clock counter and of
    the 100 MHz real-time counter."""
    import torch
    if buf is None:
        st = load_library().dgemm_trace_clock(None, 0)
    else:
        _device_tensors("buf", buf)
        if buf.dtype != torch.int64 or not buf.is_contiguous():
            raise TypeError("buf must be a contiguous int64 device tensor")
        st = load_library().dgemm_trace_clock(buf.data_ptr(), buf.numel() // 4)
    if st != 0:
        raise DgemmError(st, "dgemm_trace_clock")


def traced_clock_mhz(buf, n):
    """Engine clock (MHz) of each of the first n traced workgroups, from the
    host copy of a trace buffer."""
    import numpy as np
    t = np.asarray(buf.cpu()).reshape(-1, 4)[:n].astype(np.float64)
    dr = t[:, 3] - t[:, 1]
    return np.where(dr > 0, (t[:, 2] - t[:, 0]) / np.where(dr > 0, dr, 1.0) * 100.0, np.nan)


_TORCH_DT = None


def _dtype_name(t):
    import torch
    global _TORCH_DT
    if _TORCH_DT is None:
        _TORCH_DT = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16",
                     torch.float8_e4m3fn: "fp8"}
    if t.dtype not in _TORCH_DT:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _TORCH_DT[t.dtype]


def matmul(a, b, out=None, scale_a=None, scale_b=None, stream=None):
    """C = A x B for device tensors, the layout read from the strides.

    a: M x K row-major (stride(1) == 1).  b: K x N, either row-major (NN) or
    column-major (stride(0) == 1, TN: e.g. ``bt.t()`` of an N x K row-major
    tensor).  The result has the layout the library writes: row-major M x N
    for NN, column-major M x N (a transposed N x M tensor) for TN.  FP8
    (``torch.float8_e4m3fn``) returns float32; ``scale_a`` / ``scale_b``
    (float32 tensors of 1 or M / 1 or N values) select gemm_fp8_scaled.
    ``out`` may be given with the same layout and dtype.
    """
    import torch
    for t in (a, b):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise TypeError("a and b must be device tensors")
    if a.dim() != 2 or b.dim() != 2 or a.shape[1] != b.shape[0]:
        raise ValueError(f"shapes {tuple(a.shape)} and {tuple(b.shape)} do not chain")
    dt = _dtype_name(a)
    if _dtype_name(b) != dt:
        raise TypeError("a and b must share a dtype")
    M, K = a.shape
    N = b.shape[1]
    if a.stride(1) != 1 and M * K > 1:
        raise ValueError("a must be row-major (stride(1) == 1)")
    lda = a.stride(0) if M > 1 else max(K, 1)
    if b.stride(1) == 1 and (b.stride(0) != 1 or N == 1):
        layout, ldb = "nn", (b.stride(0) if K > 1 else max(N, 1))
    elif b.stride(0) == 1:
        layout, ldb = "tn", (b.stride(1) if N > 1 else max(K, 1))
    else:
        raise ValueError("b must be row-major or column-major")
    odt = torch.float32 if dt in ("f32", "fp8") else a.dtype
    if out is None:
        out = (torch.empty((M, N), dtype=odt, device=a.device) if layout == "nn"
               else torch.empty((N, M), dtype=odt, device=a.device).t())
    if out.shape != (M, N) or out.dtype != odt or not out.is_cuda:
        raise ValueError("out must be a device tensor of shape (M, N) and the output dtype")
    if layout == "nn":
        if out.stride(1) != 1 and M * N > 1:
            raise ValueError("NN writes a row-major C")
        ldc = out.stride(0) if M > 1 else max(N, 1)
    else:
        if out.stride(0) != 1 and M * N > 1:
            raise ValueError("TN writes a column-major C")
        ldc = out.stride(1) if N > 1 else max(M, 1)
    ein = _ELEM[dt]
    _check_extents(layout, M, N, K, a, lda, b, ldb, out, ldc, ein, out.element_size())
    if scale_a is not None or scale_b is not None:
        if dt != "fp8" or scale_a is None or scale_b is None:
            raise ValueError("scale factors go with fp8 operands, both of them")
        _device_tensors("scale factors", scale_a, scale_b)
        _factor_vector(scale_a, M, "scale_a")
        _factor_vector(scale_b, N, "scale_b")
        gemm_fp8_scaled(M, N, K, a.data_ptr(), lda, b.data_ptr(), ldb, out.data_ptr(), ldc, scale_a.data_ptr(),
                        scale_a.numel(), scale_b.data_ptr(), scale_b.numel(), layout, stream)
    else:
        _raw("gemm_" + dt, M, N, K, a.data_ptr(), lda, b.data_ptr(), ldb, out.data_ptr(), ldc, layout, stream)
    return out
