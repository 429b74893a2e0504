"""Python binding of the MI355X (gfx950) bf16 GEMM library.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libgemm_bf16.so`` (built from ``csrc/``).  There is no CPU or
PyTorch fallback: if the library is missing, every call raises.

Raw entry points mirror the C ABI in ``include/gemm_bf16.h`` (pointers are
passed as integers).  ``gemm`` is a convenience wrapper for torch tensors:
torch supplies device memory and the current stream, nothing else.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "EPILOGUES", "GemmError", "LIB_PATH", "gemm", "gemm_bf16", "gemm_bf16_kernel_name", "gemm_bf16_noalloc",
    "gemm_bf16_last_hip_error", "gemm_bf16_q8", "gemm_bf16_q8_kernel_name", "gemm_bf16_status_string",
    "gemm_fp8", "gemm_fp8_kernel_name", "gemm_q8", "library",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgemm_bf16.so")

EPILOGUES = {"none": 0, "gelu_tanh": 1, "relu": 2}
GEMM_OK = 0

_lib = None


class GemmError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"gemm_bf16 failed with status {status}: {message}")
        self.status = status


def library() -> ctypes.CDLL:
    """Load libgemm_bf16.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m bf16_gemm_fp32_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    i64, vp, f32, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_int
    lib.gemm_bf16.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, f32, f32, vp, i32, vp]
    lib.gemm_bf16.restype = i32
    lib.gemm_bf16_noalloc.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, f32, f32, vp, i32, vp]
    lib.gemm_bf16_noalloc.restype = i32
    lib.gemm_bf16_status_string.argtypes = [i32]
    lib.gemm_bf16_status_string.restype = ctypes.c_char_p
    lib.gemm_bf16_last_hip_error.argtypes = []
    lib.gemm_bf16_last_hip_error.restype = i32
    lib.gemm_bf16_kernel_name.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, f32, vp, i32]
    lib.gemm_bf16_kernel_name.restype = ctypes.c_char_p
    lib.gemm_bf16_q8.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, vp, i64, f32, f32, vp, i32, vp,
                                 ctypes.c_int32, vp]
    lib.gemm_bf16_q8.restype = i32
    lib.gemm_bf16_q8_kernel_name.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, vp, i64, f32, vp, i32]
    lib.gemm_bf16_q8_kernel_name.restype = ctypes.c_char_p
    lib.gemm_fp8.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, f32, f32, vp, vp, vp, i32, vp]
    lib.gemm_fp8.restype = i32
    lib.gemm_fp8_kernel_name.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, i32]
    lib.gemm_fp8_kernel_name.restype = ctypes.c_char_p
    _lib = lib
    return lib


def gemm_bf16(M, N, K, A, lda, B, ldb, C, ldc, alpha, beta, bias, epilogue, stream) -> int:
    """Raw C-ABI call; pointers and the stream are integers (0 / None = NULL)."""
    return library().gemm_bf16(M, N, K, A or None, lda, B or None, ldb, C or None, ldc,
                               alpha, beta, bias or None, epilogue, stream or None)


def gemm_bf16_noalloc(M, N, K, A, lda, B, ldb, C, ldc, alpha, beta, bias, epilogue, stream) -> int:
    """Raw C-ABI call of the entry point that allocates nothing (split-K
    scratch in the library's static device array; see the header)."""
    return library().gemm_bf16_noalloc(M, N, K, A or None, lda, B or None, ldb, C or None, ldc,
                                       alpha, beta, bias or None, epilogue, stream or None)


def gemm_bf16_q8(M, N, K, A, lda, B, ldb, C, ldc, Q, ldq, alpha, beta, bias, epilogue, scale,
                 zero_point, stream) -> int:
    """Raw C-ABI call of the int8-output entry point (pointers as integers)."""
    return library().gemm_bf16_q8(M, N, K, A or None, lda, B or None, ldb, C or None, ldc, Q or None, ldq,
                                  alpha, beta, bias or None, epilogue, scale or None, int(zero_point),
                                  stream or None)


def gemm_bf16_q8_kernel_name(M, N, K, A, lda, B, ldb, C, ldc, Q, ldq, beta=0.0, scale=None,
                             epilogue=0) -> str:
    return library().gemm_bf16_q8_kernel_name(M, N, K, A or None, lda, B or None, ldb, C or None, ldc,
                                              Q or None, ldq, beta, scale or None, epilogue).decode()


def gemm_fp8(M, N, K, A, lda, B, ldb, C, ldc, alpha, beta, scale_a, scale_b, bias, epilogue, stream) -> int:
    """Raw C-ABI call of the FP8 (E4M3) input entry point (pointers as integers)."""
    return library().gemm_fp8(M, N, K, A or None, lda, B or None, ldb, C or None, ldc, alpha, beta,
                              scale_a or None, scale_b or None, bias or None, epilogue, stream or None)


def gemm_fp8_kernel_name(M, N, K, A, lda, B, ldb, C, ldc, epilogue=0) -> str:
    return library().gemm_fp8_kernel_name(M, N, K, A or None, lda, B or None, ldb, C or None, ldc,
                                          epilogue).decode()


def gemm_bf16_status_string(status: int) -> str:
    return library().gemm_bf16_status_string(status).decode()


def gemm_bf16_last_hip_error() -> int:
    return library().gemm_bf16_last_hip_error()


def gemm_bf16_kernel_name(M, N, K, A, lda, B, ldb, C, ldc, beta=0.0, bias=None, epilogue=0) -> str:
    return library().gemm_bf16_kernel_name(M, N, K, A or None, lda, B or None, ldb, C or None, ldc,
                                           beta, bias or None, epilogue).decode()


def _operand(t, name, rows, cols):
    import torch
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be torch.bfloat16, got {t.dtype}")
    if t.dim() != 2 or tuple(t.shape) != (rows, cols):
        raise ValueError(f"{name} must have shape ({rows}, {cols}), got {tuple(t.shape)}")
    if cols > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} rows must be contiguous (stride(1) == 1)")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    ld = t.stride(0) if rows > 1 else max(cols, 1)
    return t.data_ptr(), max(ld, cols, 1)


def gemm(A, Bt, Ct, alpha: float = 1.0, beta: float = 0.0, bias=None, epilogue: str = "none",
         stream=None):
    """C <- epi(alpha*A*B + beta*C + bias) on torch bf16 device tensors.

    A:  (M, K) with contiguous rows          -> row-major A, lda = A.stride(0)
    Bt: (N, K) with contiguous rows          -> column-major B, ldb = Bt.stride(0)
    Ct: (N, M) with contiguous rows, in/out  -> column-major C, ldc = Ct.stride(0)
    bias: None or (N,) contiguous.
    Enqueued on `stream` (default: torch's current stream); returns Ct.
    """
    import torch
    M, K = A.shape
    N = Bt.shape[0]
    a_ptr, lda = _operand(A, "A", M, K)
    b_ptr, ldb = _operand(Bt, "Bt", N, K)
    c_ptr, ldc = _operand(Ct, "Ct", N, M)
    bias_ptr = 0
    if bias is not None:
        if bias.dtype != torch.bfloat16 or bias.numel() != N or not bias.is_contiguous() or not bias.is_cuda:
            raise ValueError("bias must be a contiguous bf16 device tensor of N elements")
        bias_ptr = bias.data_ptr()
    if stream is None:
        stream = torch.cuda.current_stream(Ct.device)
    st = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    status = gemm_bf16(M, N, K, a_ptr, lda, b_ptr, ldb, c_ptr, ldc, float(alpha), float(beta),
                       bias_ptr, EPILOGUES[epilogue], st)
    if status != GEMM_OK:
        msg = gemm_bf16_status_string(status)
        if status == -5:
            msg += f" (hipError {gemm_bf16_last_hip_error()})"
        raise GemmError(status, msg)
    return Ct


def gemm_q8(A, Bt, Qt, scale, zero_point: int = 0, alpha: float = 1.0, beta: float = 0.0, Ct=None,
            bias=None, epilogue: str = "none", stream=None):
    """Qt <- sat8(rne(epi(alpha*A*B + beta*C + bias) * scale[m] + zero_point)).

    A, Bt, bias as in gemm; Qt: (N, M) int8 with contiguous rows (column-major
    Q, ldq = Qt.stride(0)); scale: (M,) contiguous float32; Ct: (N, M) bf16
    input C0, only needed when beta != 0.  Returns Qt.
    """
    import torch
    M, K = A.shape
    N = Bt.shape[0]
    a_ptr, lda = _operand(A, "A", M, K)
    b_ptr, ldb = _operand(Bt, "Bt", N, K)
    c_ptr, ldc = (0, max(M, 1)) if Ct is None else _operand(Ct, "Ct", N, M)
    if Qt.dtype != torch.int8 or tuple(Qt.shape) != (N, M) or (M > 1 and Qt.stride(1) != 1) or not Qt.is_cuda:
        raise ValueError("Qt must be an (N, M) int8 device tensor with contiguous rows")
    ldq = max(Qt.stride(0) if N > 1 else M, M, 1)
    if scale.dtype != torch.float32 or scale.numel() != M or not scale.is_contiguous() or not scale.is_cuda:
        raise ValueError("scale must be a contiguous float32 device tensor of M elements")
    bias_ptr = 0
    if bias is not None:
        if bias.dtype != torch.bfloat16 or bias.numel() != N or not bias.is_contiguous() or not bias.is_cuda:
            raise ValueError("bias must be a contiguous bf16 device tensor of N elements")
        bias_ptr = bias.data_ptr()
    if stream is None:
        stream = torch.cuda.current_stream(Qt.device)
    st = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    status = gemm_bf16_q8(M, N, K, a_ptr, lda, b_ptr, ldb, c_ptr, ldc, Qt.data_ptr(), ldq, float(alpha),
                          float(beta), bias_ptr, EPILOGUES[epilogue], scale.data_ptr(), int(zero_point), st)
    if status != GEMM_OK:
        msg = gemm_bf16_status_string(status)
        if status == -5:
            msg += f" (hipError {gemm_bf16_last_hip_error()})"
        raise GemmError(status, msg)
    return Qt
