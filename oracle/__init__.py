"""CPU oracle for the bf16 GEMM: plain, slow, fp64-accumulating reference.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  The product (the HIP
library and its Python binding) never imports, links or calls it, and it
shares no code with the product.

The arithmetic lives in ``gemm_oracle.c`` (compiled with gcc, no fast-math,
no FP contraction).  This module only marshals numpy arrays into it.

What it computes (see the C file for the sources):

    C_out[m,n] = bf16_rne(epi(alpha * sum_k A[m,k] B[k,n]
                              + beta * C_in[m,n] + bias[n]))

with A row-major (A[m*lda+k]), B column-major (B[k+n*ldb]) and C
column-major (C[m+n*ldc]); sums in double with k ascending; one
round-to-nearest-even to bf16 at the end.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gemm_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

EPI_CODES = {"none": 0, "gelu_tanh": 1, "relu": 2}

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/liboracle.so``."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off",
               "-fno-fast-math", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    i64, u16p, f64 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_double
    lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f64.restype = f64
    lib.oracle_bf16_from_f64.argtypes = [f64]
    lib.oracle_bf16_from_f64.restype = ctypes.c_uint16
    lib.oracle_gelu_tanh.argtypes = [f64]
    lib.oracle_gelu_tanh.restype = f64
    for name in ("oracle_bf16_to_f64_array", "oracle_bf16_from_f64_array",
                 "oracle_gelu_tanh_array"):
        getattr(lib, name).argtypes = [ctypes.c_void_p, ctypes.c_void_p, i64]
        getattr(lib, name).restype = None
    lib.oracle_gemm.argtypes = [i64, i64, i64, u16p, i64, u16p, i64, u16p, i64,
                                f64, f64, u16p, ctypes.c_int, u16p,
                                ctypes.c_void_p, ctypes.c_int]
    lib.oracle_gemm.restype = ctypes.c_int
    lib.oracle_gemm_elems.argtypes = [i64, i64, i64, u16p, i64, u16p, i64, u16p, i64,
                                      f64, f64, u16p, ctypes.c_int, i64,
                                      ctypes.c_void_p, ctypes.c_void_p, u16p,
                                      ctypes.c_void_p, ctypes.c_int]
    lib.oracle_gemm_elems.restype = ctypes.c_int
    lib.oracle_relu.argtypes = [f64]
    lib.oracle_relu.restype = f64
    lib.oracle_quantize_i8.argtypes = [f64, ctypes.c_float, ctypes.c_int32, ctypes.c_void_p]
    lib.oracle_quantize_i8.restype = ctypes.c_int
    lib.oracle_gemm_q8.argtypes = [i64, i64, i64, u16p, i64, u16p, i64, u16p, i64, f64, f64, u16p,
                                   ctypes.c_int, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, i64,
                                   ctypes.c_void_p, ctypes.c_int]
    lib.oracle_gemm_q8.restype = ctypes.c_int
    lib.oracle_quantize_i8_array.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                             ctypes.c_void_p, ctypes.c_void_p, i64]
    lib.oracle_quantize_i8_array.restype = None
    lib.oracle_fp8_e4m3_to_f64.argtypes = [ctypes.c_uint8]
    lib.oracle_fp8_e4m3_to_f64.restype = f64
    lib.oracle_fp8_e4m3_to_f64_array.argtypes = [ctypes.c_void_p, ctypes.c_void_p, i64]
    lib.oracle_fp8_e4m3_to_f64_array.restype = None
    lib.oracle_gemm_fp8.argtypes = [i64, i64, i64, ctypes.c_void_p, i64, ctypes.c_void_p, i64, u16p, i64,
                                    f64, f64, ctypes.c_void_p, ctypes.c_void_p, u16p, ctypes.c_int, u16p,
                                    ctypes.c_void_p, ctypes.c_int]
    lib.oracle_gemm_fp8.restype = ctypes.c_int
    lib.oracle_gemm_fp8_elems.argtypes = [i64, i64, i64, ctypes.c_void_p, i64, ctypes.c_void_p, i64, u16p, i64,
                                          f64, f64, ctypes.c_void_p, ctypes.c_void_p, u16p, ctypes.c_int, i64,
                                          ctypes.c_void_p, ctypes.c_void_p, u16p, ctypes.c_int]
    lib.oracle_gemm_fp8_elems.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _u16(a, name):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"{name} must hold raw bf16 bits as uint16, got {a.dtype}")
    return a.reshape(-1)


def bf16_to_f64(bits) -> np.ndarray:
    """Exact decode of raw bf16 bit patterns (any shape) to float64."""
    lib = _load()
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(b.shape, dtype=np.float64)
    lib.oracle_bf16_to_f64_array(_ptr(b), _ptr(out), b.size)
    return out


def bf16_from_f64(x) -> np.ndarray:
    """Round float64 values (any shape) to bf16 bits, nearest-even, once."""
    lib = _load()
    a = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(a.shape, dtype=np.uint16)
    lib.oracle_bf16_from_f64_array(_ptr(a), _ptr(out), a.size)
    return out


def gelu_tanh(x) -> np.ndarray:
    """GELU, tanh form, in float64 (any shape)."""
    lib = _load()
    a = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(a.shape, dtype=np.float64)
    lib.oracle_gelu_tanh_array(_ptr(a), _ptr(out), a.size)
    return out


def gemm(M, N, K, A, lda, B, ldb, C_in=None, ldc=None, alpha=1.0, beta=0.0,
         bias=None, epilogue="none", nthreads=0, return_pre=False):
    """Whole-product oracle on flat storage-order buffers of bf16 bits.

    A holds at least (M-1)*lda+K elements (row-major), B at least
    (N-1)*ldb+K (column-major), C_in (only read if beta != 0) at least
    (N-1)*ldc+M (column-major).  Returns C_out as a flat uint16 array of
    N*ldc elements (column-major, leading dimension ldc; padding rows are 0),
    and with return_pre=True also the pre-rounding float64 values as an
    (N, M) array (row n holds column n of C).
    """
    lib = _load()
    if ldc is None:
        ldc = max(1, M)
    A, B, C_in, bias = _u16(A, "A"), _u16(B, "B"), _u16(C_in, "C_in"), _u16(bias, "bias")
    if M > 0 and K > 0 and A.size < (M - 1) * lda + K:
        raise ValueError("A too small")
    if N > 0 and K > 0 and B.size < (N - 1) * ldb + K:
        raise ValueError("B too small")
    if beta != 0.0 and M > 0 and N > 0 and (C_in is None or C_in.size < (N - 1) * ldc + M):
        raise ValueError("C_in too small")
    if bias is not None and bias.size < N:
        raise ValueError("bias too small")
    out = np.zeros(max(N * ldc, 1), dtype=np.uint16)
    pre = np.zeros((max(N, 1), max(M, 1)), dtype=np.float64) if return_pre else None
    rc = lib.oracle_gemm(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C_in), ldc,
                         float(alpha), float(beta), _ptr(bias), EPI_CODES[epilogue],
                         _ptr(out), _ptr(pre), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_gemm rejected its arguments")
    out = out[: N * ldc]
    if return_pre:
        return out, pre[:N, :M]
    return out


def gemm_elems(M, N, K, A, lda, B, ldb, ms, ns, C_in=None, ldc=None, alpha=1.0,
               beta=0.0, bias=None, epilogue="none", nthreads=0, return_pre=False):
    """The same definition evaluated only at coordinates (ms[i], ns[i])."""
    lib = _load()
    if ldc is None:
        ldc = max(1, M)
    A, B, C_in, bias = _u16(A, "A"), _u16(B, "B"), _u16(C_in, "C_in"), _u16(bias, "bias")
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    if ms.shape != ns.shape:
        raise ValueError("ms and ns differ in shape")
    out = np.zeros(max(ms.size, 1), dtype=np.uint16)
    pre = np.zeros(max(ms.size, 1), dtype=np.float64) if return_pre else None
    rc = lib.oracle_gemm_elems(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C_in), ldc,
                               float(alpha), float(beta), _ptr(bias), EPI_CODES[epilogue],
                               ms.size, _ptr(ms), _ptr(ns), _ptr(out), _ptr(pre),
                               int(nthreads))
    if rc != 0:
        raise ValueError("oracle_gemm_elems rejected its arguments")
    if return_pre:
        return out[: ms.size], pre[: ms.size]
    return out[: ms.size]


def relu(y: float) -> float:
    """ReLU of one value, in float64 (NaN passes through)."""
    return _load().oracle_relu(float(y))


def quantize_i8(y: float, scale: float, zero_point: int):
    """(code, t_exact): the int8 code of one epilogue value and y*scale+zp in double."""
    t = ctypes.c_double()
    q = _load().oracle_quantize_i8(float(y), float(scale), int(zero_point), ctypes.byref(t))
    return q, t.value


def gemm_q8(M, N, K, A, lda, B, ldb, scale, zero_point=0, C_in=None, ldc=None, ldq=None, alpha=1.0,
            beta=0.0, bias=None, epilogue="none", nthreads=0):
    """Int8-output oracle: returns (Q, t_exact).

    Q is a flat int8 array of N*ldq elements (column-major, leading dimension
    ldq; padding rows are 0); t_exact is the (N, M) float64 array of
    y*scale[m] + zero_point before the fp32 decision.  scale holds M float32.
    """
    lib = _load()
    if ldc is None:
        ldc = max(1, M)
    if ldq is None:
        ldq = max(1, M)
    A, B, C_in, bias = _u16(A, "A"), _u16(B, "B"), _u16(C_in, "C_in"), _u16(bias, "bias")
    scale = np.ascontiguousarray(scale, dtype=np.float32).reshape(-1)
    if scale.size < M:
        raise ValueError("scale too small")
    Q = np.zeros(max(N * ldq, 1), dtype=np.int8)
    t = np.zeros((max(N, 1), max(M, 1)), dtype=np.float64)
    rc = lib.oracle_gemm_q8(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C_in), ldc, float(alpha), float(beta),
                            _ptr(bias), EPI_CODES[epilogue], _ptr(scale), int(zero_point), _ptr(Q), ldq,
                            _ptr(t), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_gemm_q8 rejected its arguments")
    return Q[: N * ldq], t[:N, :M]


def quantize_i8_array(y, scale, zero_point):
    """Vector form of quantize_i8: y (float64) and per-element scales (float32)
    of the same length; returns (codes int8, t_exact float64)."""
    lib = _load()
    y = np.ascontiguousarray(y, dtype=np.float64).reshape(-1)
    s = np.ascontiguousarray(scale, dtype=np.float32).reshape(-1)
    if s.size != y.size:
        raise ValueError("y and scale differ in length")
    q = np.zeros(max(y.size, 1), dtype=np.int8)
    t = np.zeros(max(y.size, 1), dtype=np.float64)
    lib.oracle_quantize_i8_array(_ptr(y), _ptr(s), int(zero_point), _ptr(q), _ptr(t), y.size)
    return q[: y.size], t[: y.size]


def fp8_to_f64(bits) -> np.ndarray:
    """Exact decode of OCP FP8 E4M3 bytes (any shape) to float64."""
    lib = _load()
    b = np.ascontiguousarray(bits, dtype=np.uint8)
    out = np.empty(b.shape, dtype=np.float64)
    lib.oracle_fp8_e4m3_to_f64_array(_ptr(b), _ptr(out), b.size)
    return out


def gemm_fp8(M, N, K, A, lda, B, ldb, C_in=None, ldc=None, alpha=1.0, beta=0.0, scale_a=None,
             scale_b=None, bias=None, epilogue="none", nthreads=0, return_pre=False):
    """fp8 (E4M3) input oracle: A, B flat uint8 buffers (A row-major, B
    column-major), optional per-row scale_a (M floats) and per-column
    scale_b (N floats); returns C_out as gemm() does."""
    lib = _load()
    if ldc is None:
        ldc = max(1, M)
    A = np.ascontiguousarray(A, dtype=np.uint8).reshape(-1)
    B = np.ascontiguousarray(B, dtype=np.uint8).reshape(-1)
    C_in, bias = _u16(C_in, "C_in"), _u16(bias, "bias")
    sa = None if scale_a is None else np.ascontiguousarray(scale_a, dtype=np.float32).reshape(-1)
    sb = None if scale_b is None else np.ascontiguousarray(scale_b, dtype=np.float32).reshape(-1)
    if M > 0 and K > 0 and A.size < (M - 1) * lda + K:
        raise ValueError("A too small")
    if N > 0 and K > 0 and B.size < (N - 1) * ldb + K:
        raise ValueError("B too small")
    if (sa is not None and sa.size < M) or (sb is not None and sb.size < N):
        raise ValueError("scales too small")
    out = np.zeros(max(N * ldc, 1), dtype=np.uint16)
    pre = np.zeros((max(N, 1), max(M, 1)), dtype=np.float64) if return_pre else None
    rc = lib.oracle_gemm_fp8(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C_in), ldc, float(alpha), float(beta),
                             _ptr(sa), _ptr(sb), _ptr(bias), EPI_CODES[epilogue], _ptr(out), _ptr(pre),
                             int(nthreads))
    if rc != 0:
        raise ValueError("oracle_gemm_fp8 rejected its arguments")
    out = out[: N * ldc]
    if return_pre:
        return out, pre[:N, :M]
    return out


def gemm_fp8_elems(M, N, K, A, lda, B, ldb, ms, ns, C_in=None, ldc=None, alpha=1.0, beta=0.0, scale_a=None,
                   scale_b=None, bias=None, epilogue="none", nthreads=0):
    """The fp8 definition evaluated only at coordinates (ms[i], ns[i])."""
    lib = _load()
    if ldc is None:
        ldc = max(1, M)
    A = np.ascontiguousarray(A, dtype=np.uint8).reshape(-1)
    B = np.ascontiguousarray(B, dtype=np.uint8).reshape(-1)
    C_in, bias = _u16(C_in, "C_in"), _u16(bias, "bias")
    sa = None if scale_a is None else np.ascontiguousarray(scale_a, dtype=np.float32).reshape(-1)
    sb = None if scale_b is None else np.ascontiguousarray(scale_b, dtype=np.float32).reshape(-1)
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    out = np.zeros(max(ms.size, 1), dtype=np.uint16)
    rc = lib.oracle_gemm_fp8_elems(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C_in), ldc, float(alpha),
                                   float(beta), _ptr(sa), _ptr(sb), _ptr(bias), EPI_CODES[epilogue], ms.size,
                                   _ptr(ms), _ptr(ns), _ptr(out), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_gemm_fp8_elems rejected its arguments")
    return out[: ms.size]
