"""The C-ABI library loads, exports every function include/gemm_bf16.h
declares, and rejects bad arguments on the host before any HIP call (these
calls never reach the device, so they run without a GPU)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import bf16_gemm_fp32_amd as gb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemm_bf16.h")

OK, ERR_DIM, ERR_LD, ERR_NULL, ERR_EPI, ERR_HIP = 0, -1, -2, -3, -4, -5
P = 4096  # a fake non-NULL pointer: never dereferenced on these paths


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gemm_\w*)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = gb.library()
    names = declared_functions()
    assert "gemm_bf16" in names and len(names) >= 4
    for name in names:
        assert hasattr(lib, name), f"{name} declared in the header but not exported"


def test_status_codes_match_header():
    text = open(HEADER).read()
    for name, val in [("GEMM_OK", 0), ("GEMM_ERR_DIM", -1), ("GEMM_ERR_LD", -2),
                      ("GEMM_ERR_NULL", -3), ("GEMM_ERR_EPILOGUE", -4), ("GEMM_ERR_HIP", -5),
                      ("GEMM_EPI_NONE", 0), ("GEMM_EPI_GELU_TANH", 1), ("GEMM_EPI_RELU", 2)]:
        assert re.search(rf"\b{name}\s*=\s*{val}\b", text), name
    assert gb.EPILOGUES == {"none": 0, "gelu_tanh": 1, "relu": 2}


def call(M, N, K, A=P, lda=None, B=P, ldb=None, C=P, ldc=None, alpha=1.0, beta=0.0, bias=0, epi=0):
    lda = max(K, 1) if lda is None else lda
    ldb = max(K, 1) if ldb is None else ldb
    ldc = max(M, 1) if ldc is None else ldc
    return gb.gemm_bf16(M, N, K, A, lda, B, ldb, C, ldc, alpha, beta, bias, epi, 0)


@pytest.mark.parametrize("args,want", [
    ((-1, 4, 4), ERR_DIM), ((4, -1, 4), ERR_DIM), ((4, 4, -1), ERR_DIM),
    ((4, 4, 4, P, 3), ERR_LD), ((4, 4, 4, P, 4, P, 3), ERR_LD),
    ((4, 4, 4, P, 4, P, 4, P, 3), ERR_LD), ((4, 4, 0, P, 0), ERR_LD),
    ((4, 4, 4, 0), ERR_NULL), ((4, 4, 4, P, 4, 0), ERR_NULL), ((4, 4, 4, P, 4, P, 4, 0), ERR_NULL),
])
def test_argument_errors(args, want):
    assert call(*args) == want


def call_noalloc(M, N, K, A=P, lda=None, B=P, ldb=None, C=P, ldc=None, alpha=1.0, beta=0.0, bias=0, epi=0):
    lda = max(K, 1) if lda is None else lda
    ldb = max(K, 1) if ldb is None else ldb
    ldc = max(M, 1) if ldc is None else ldc
    return gb.gemm_bf16_noalloc(M, N, K, A, lda, B, ldb, C, ldc, alpha, beta, bias, epi, 0)


@pytest.mark.parametrize("args,want", [
    ((-1, 4, 4), ERR_DIM), ((4, 4, 4, P, 3), ERR_LD), ((4, 4, 4, P, 4, P, 4, P, 3), ERR_LD),
    ((4, 4, 4, 0), ERR_NULL), ((4, 4, 4, P, 4, P, 4, 0), ERR_NULL),
    ((0, 4, 4), OK), ((4, 0, 4), OK),
])
def test_noalloc_argument_errors(args, want):
    """The entry point that allocates nothing validates exactly as gemm_bf16,
    before it touches its scratch (so these run without a GPU)."""
    assert call_noalloc(*args) == want
    assert call(*args) == want


def test_noalloc_bad_epilogue():
    assert call_noalloc(4, 4, 4, epi=7) == ERR_EPI


def call_q8(M, N, K, A=P, lda=None, B=P, ldb=None, C=0, ldc=None, Q=P, ldq=None, alpha=1.0, beta=0.0,
            bias=0, epi=0, scale=P, zp=0):
    lda = max(K, 1) if lda is None else lda
    ldb = max(K, 1) if ldb is None else ldb
    ldc = max(M, 1) if ldc is None else ldc
    ldq = max(M, 1) if ldq is None else ldq
    return gb.gemm_bf16_q8(M, N, K, A, lda, B, ldb, C, ldc, Q, ldq, alpha, beta, bias, epi, scale, zp, 0)


def test_q8_argument_errors():
    assert call_q8(-1, 4, 4) == ERR_DIM
    assert call_q8(4, 4, 4, ldq=3) == ERR_LD
    assert call_q8(4, 4, 4, beta=0.5, C=P, ldc=3) == ERR_LD
    assert call_q8(4, 4, 4, Q=0) == ERR_NULL
    assert call_q8(4, 4, 4, scale=0) == ERR_NULL
    assert call_q8(4, 4, 4, beta=0.5, C=0) == ERR_NULL
    assert call_q8(4, 4, 4, epi=3) == ERR_EPI
    # beta == 0: C and ldc are not looked at; empty outputs launch nothing
    assert call_q8(0, 4, 4, Q=0, scale=0) == OK
    name = gb.gemm_bf16_q8_kernel_name
    assert name(4096, 4096, 4096, P, 4096, P, 4096, 0, 1, P, 4096, 0.0, P, 2) == "ring256x256x64_q8"
    assert name(4000, 4000, 1000, P, 1000, P, 1000, P, 4000, P, 4000, 0.5, P, 1) == "ring256x256x64_q8_masked"
    assert name(1, 4096, 4096, P, 4096, P, 4096, 0, 1, P + 3, 1, 0.0, P, 2) == "skinny_q8"    # any Q alignment
    assert name(64, 8192, 8192, P, 8192, P, 8192, 0, 64, P, 64, 0.0, P, 0) == "skinny_q8"
    assert name(8192, 64, 8192, P, 8192, P, 8192, 0, 8192, P, 8192, 0.0, P, 0) == "skinny_q8_t"
    assert name(1000, 17, 3000, P, 3000, P, 3000, 0, 1000, P + 3, 1001, 0.0, P, 0) == "skinny_q8_t"
    assert name(65536, 64, 1024, P, 1024, P, 1024, 0, 65536, P, 65536, 0.0, P, 0) != "skinny_q8_t"  # short K
    assert name(65, 8192, 8192, P, 8192, P, 8192, 0, 72, P, 72, 0.0, P, 0) != "skinny_q8"
    assert name(4096, 4096, 4096, P, 4096, P, 4096, 0, 1, P + 8, 4096, 0.0, P, 0) == "generic64x64x32"
    assert name(4096, 4096, 4096, P, 4096, P, 4096, 0, 1, P, 4100, 0.0, P, 0) == "generic64x64x32"
    assert name(100, 100, 64, P, 64, P, 64, 0, 1, P, 112, 0.0, P, 0) == "generic64x64x32"
    # small grids of 128-tiles with enough K-slices: split-K, the reduction quantizing
    assert name(1024, 1024, 4096, P, 4096, P, 4096, 0, 1, P, 1024, 0.0, P, 2) == "splitk128x128x64_q8"
    assert name(1024, 1024, 4096, P, 4096, P, 4096, 0, 1, P, 1028, 0.0, P, 2) == "generic64x64x32"
    # too few slices to split: whole K on 128x128 tiles through the same reduction
    assert name(1024, 1024, 512, P, 512, P, 512, 0, 1, P, 1024, 0.0, P, 2) == "tile128x128x64_q8"  # 8 slices
    assert name(2048, 2048, 4096, P, 4096, P, 4096, 0, 1, P, 2048, 0.0, P, 2) == "tile128x128x64_q8"
    assert name(1504, 1504, 512, P, 512, P, 512, 0, 1, P, 1504, 0.0, P, 2) == "tile128x128x64_q8_masked"
    assert name(2048, 2048, 256, P, 256, P, 256, 0, 1, P, 2048, 0.0, P, 2) == "ring256x256x64_q8"  # 4 slices
    assert name(3072, 2048, 4096, P, 4096, P, 4096, 0, 1, P, 3072, 0.0, P, 2) == "ring256x256x64_q8"  # too big
    # with tails: the masked split
    assert name(1000, 1000, 4096, P, 4096, P, 4096, 0, 1, P, 1000, 0.0, P, 2) == "splitk128x128x64_q8_masked"
    assert name(1001, 777, 2048, P, 2048, P, 2048, 0, 1, P, 1008, 0.0, P, 2) == "splitk128x128x64_q8_masked"
    # mid-sized grids too large to split: whole K on 128x128 tiles while the
    # workspace holds every tile, then the ring from more than 32 ring tiles
    assert name(2048, 1024, 4096, P, 4096, P, 4096, 0, 1, P, 2048, 0.0, P, 2) == "tile128x128x64_q8"
    assert name(4096, 1536, 4096, P, 4096, P, 4096, 0, 1, P, 4096, 0.0, P, 2) == "ring256x256x64_q8"
    assert name(2304, 2048, 256, P, 256, P, 256, 0, 1, P, 2304, 0.0, P, 2) == "ring256x256x64_q8"
    assert name(2048, 1024, 256, P, 256, P, 256, 0, 1, P, 2048, 0.0, P, 2) == "generic64x64x32"


def test_fp8_argument_errors_and_names():
    f = gb.gemm_fp8
    assert f(-1, 4, 4, P, 4, P, 4, P, 4, 1.0, 0.0, 0, 0, 0, 0, 0) == ERR_DIM
    assert f(4, 4, 4, P, 3, P, 4, P, 4, 1.0, 0.0, 0, 0, 0, 0, 0) == ERR_LD
    assert f(4, 4, 4, 0, 4, P, 4, P, 4, 1.0, 0.0, 0, 0, 0, 0, 0) == ERR_NULL
    assert f(4, 4, 4, P, 4, P, 4, P, 4, 1.0, 0.0, 0, 0, 0, 7, 0) == ERR_EPI
    assert f(0, 4, 4, 0, 4, P, 4, 0, 1, 1.0, 0.0, 0, 0, 0, 2, 0) == OK
    name = gb.gemm_fp8_kernel_name
    assert name(4096, 4096, 4096, P, 4096, P, 4096, P, 4096) == "fp8_256x256x128"
    # tails: the masked instance (K a multiple of 16)
    assert name(4096, 4096, 4032, P, 4032, P, 4032, P, 4096) == "fp8_256x256x128_masked"  # K % 128 != 0
    assert name(4000, 4096, 4096, P, 4096, P, 4096, P, 4000) == "fp8_256x256x128_masked"
    assert name(4096, 4096, 4040, P, 4048, P, 4048, P, 4096) == "generic64x64x32"   # K % 16 != 0
    assert name(4096, 4096, 4096, P + 8, 4096, P, 4096, P, 4096) == "generic64x64x32"  # unaligned A
    assert name(4000, 4096, 4096, P, 4096, P, 4096, P, 4004) == "fp8_256x256x128_masked"  # ldc % 8 != 0: element-wise C
    assert name(4096, 4096, 4096, P, 4096, P, 4096, P, 4100) == "fp8_256x256x128_masked"  # exact tiles, odd ldc
    # one to four rows: the matrix-vector kernel (any ldc)
    assert name(1, 4096, 4096, P, 4096, P, 4096, P, 1) == "gemv_fp8"
    assert name(2, 8192, 8192, P, 8192, P, 8192, P, 2) == "gemv_fp8"
    assert name(3, 8192, 8192, P, 8192, P, 8192, P, 3) == "skinny_fp8"   # large B: A shared per strip
    assert name(4, 16384, 4096, P, 4096, P, 4096, P, 4) == "skinny_fp8"
    # grids where the 256x256 tiles fill less than half the CUs take the
    # 128x128 tiles, splitting K by the bf16 rule (5 nk >= 96 + 2 tiles)
    assert name(1024, 1024, 4096, P, 4096, P, 4096, P, 1024) == "fp8_128x128x128"         # 64 tiles, 32 slices
    assert name(512, 512, 8192, P, 8192, P, 8192, P, 512) == "splitk_fp8_128x128x128"     # 16 tiles, 64 slices
    assert name(256, 256, 8192, P, 8192, P, 8192, P, 256) == "splitk_fp8_128x128x128"     # 4 tiles
    assert name(1024, 1024, 384, P, 384, P, 384, P, 1024) == "fp8_128x128x128"           # 3 slices
    assert name(1000, 1000, 4096, P, 4096, P, 4096, P, 1000) == "fp8_128x128x128_masked"
    assert name(1000, 1000, 208, P, 208, P, 208, P, 1000) == "fp8_128x128x128_masked"    # K tail
    assert name(500, 500, 8192, P, 8192, P, 8192, P, 504) == "splitk_fp8_128x128x128_masked"
    assert name(2048, 4096, 4096, P, 4096, P, 4096, P, 2048) == "fp8_128x128x128"  # 128 tiles of 256x256: half
    assert name(2304, 4096, 4096, P, 4096, P, 4096, P, 2304) == "fp8_256x256x128"  # 144 tiles of 256x256
    assert name(2048, 2048, 4096, P, 4096, P, 4096, P, 2048) == "fp8_128x128x128"  # 256 tiles of 128x128
    assert name(3072, 3072, 2048, P, 2048, P, 2048, P, 3072) == "fp8_256x256x128"  # 144 tiles of 256x256
    assert name(4, 4096, 4096, P, 4096, P, 4096, P + 2, 5) == "gemv_fp8"
    assert name(5, 4096, 4096, P, 4096, P, 4096, P, 8) == "skinny_fp8"
    assert name(64, 8192, 8192, P, 8192, P, 8192, P, 64) == "skinny_fp8"
    assert name(8192, 64, 8192, P, 8192, P, 8192, P, 8192) == "skinny_fp8_t"
    assert name(8192, 1, 4096, P, 4096, P, 4096, P, 8192) == "skinny_fp8_t"
    assert name(8192, 64, 4104, P, 4104, P, 4104, P, 8192) != "skinny_fp8_t"   # K % 16 != 0
    # more than two strips per compute unit over fewer than 8 slices of 512
    assert name(64, 65536, 1024, P, 1024, P, 1024, P, 64) == "fp8_128x128x128_masked"
    assert name(65536, 64, 2048, P, 2048, P, 2048, P, 65536) == "fp8_128x128x128_masked"
    assert name(64, 16384, 2048, P, 2048, P, 2048, P, 64) == "skinny_fp8"
    assert name(64, 65536, 4096, P, 4096, P, 4096, P, 64) == "skinny_fp8"
    assert name(65, 4096, 4096, P, 4096, P, 4096, P, 72) == "splitk_fp8_128x128x128_masked"  # 32 tiles, 32 slices
    assert name(1024, 512, 4096, P, 4096, P, 4096, P, 1024) == "splitk_fp8_128x128x128"  # 32 tiles, 32 slices
    assert name(768, 768, 4096, P, 4096, P, 4096, P, 768) == "fp8_128x128x128"  # 36 tiles, 32 slices
    assert name(65, 4096, 16384, P, 16384, P, 16384, P, 72) == "splitk_fp8_128x128x128_masked"
    assert name(1024, 1024, 2048, P, 2048, P, 2048, P, 1024) == "fp8_128x128x128"
    assert name(2048, 1024, 4096, P, 4096, P, 4096, P, 2048) == "fp8_128x128x128"  # 128 tiles: no split
    assert name(512, 512, 4096, P, 4096, P, 4096, P, 512) == "splitk_fp8_128x128x128"  # 16 tiles, 32 slices
    assert name(512, 512, 2048, P, 2048, P, 2048, P, 512) == "fp8_128x128x128"         # 16 tiles, 16 slices
    assert name(1, 4096, 4040, P, 4048, P, 4048, P, 1) == "generic64x64x32"          # K % 16 != 0


def test_fp8_forced_mfma_form_names(monkeypatch):
    # exact FP8 tiles run on 16x16x128 and tails on 32x32x64 MFMAs; the other
    # form of each runs only when forced
    name = gb.gemm_fp8_kernel_name
    monkeypatch.setenv("GEMM_BF16_FORCE_KERNEL", "fp8_256x256x128_mfma32")
    assert name(4096, 4096, 4096, P, 4096, P, 4096, P, 4096) == "fp8_256x256x128_mfma32"
    assert name(4000, 4096, 4096, P, 4096, P, 4096, P, 4000) == "fp8_256x256x128_masked"
    monkeypatch.setenv("GEMM_BF16_FORCE_KERNEL", "fp8_256x256x128_mfma16_masked")
    assert name(4096, 4096, 4096, P, 4096, P, 4096, P, 4096) == "fp8_256x256x128_mfma16_masked"
    assert name(4000, 4096, 4096, P, 4096, P, 4096, P, 4000) == "fp8_256x256x128_mfma16_masked"
    monkeypatch.setenv("GEMM_BF16_FORCE_KERNEL", "fp8_256x256x128")
    assert name(1024, 1024, 4096, P, 4096, P, 4096, P, 1024) == "fp8_256x256x128"  # unsplit when forced
    monkeypatch.setenv("GEMM_BF16_FORCE_KERNEL", "splitk_fp8_256x256x128")
    assert name(1024, 1024, 4096, P, 4096, P, 4096, P, 1024) == "splitk_fp8_256x256x128"
    assert name(1000, 1000, 4096, P, 4096, P, 4096, P, 1000) == "splitk_fp8_256x256x128_masked"
    monkeypatch.setenv("GEMM_BF16_FORCE_KERNEL", "fp8_128x128x128")
    assert name(4096, 4096, 4096, P, 4096, P, 4096, P, 4096) == "fp8_128x128x128"
    assert name(4000, 4096, 4096, P, 4096, P, 4096, P, 4000) == "fp8_128x128x128_masked"
    monkeypatch.setenv("GEMM_BF16_FORCE_KERNEL", "splitk_fp8_128x128x128")
    assert name(1024, 1024, 4096, P, 4096, P, 4096, P, 1024) == "splitk_fp8_128x128x128"
    assert name(4096, 4096, 4096, P, 4096, P, 4096, P, 4096) == "fp8_256x256x128"  # no split on 1024 tiles


def test_relu_is_accepted():
    # M == 0: nothing to launch, so the status is decided by validation alone
    assert call(0, 4, 4, A=0, C=0, epi=2) == OK
    assert call(0, 4, 4, A=0, C=0, epi=3) == ERR_EPI


def test_error_order_dim_before_ld_before_null_before_epilogue():
    assert call(-1, 4, 4, 0, 0, 0, 0, 0, 0, epi=9) == ERR_DIM
    assert call(4, 4, 4, 0, 0, 0, 0, 0, 0, epi=9) == ERR_LD
    assert call(4, 4, 4, 0, 4, 0, 4, 0, 4, epi=9) == ERR_NULL
    assert call(4, 4, 4, epi=9) == ERR_EPI
    assert call(4, 4, 4, epi=-1) == ERR_EPI


def test_empty_outputs_are_no_ops_without_device():
    # M == 0 or N == 0: nothing to compute, no HIP call, NULL operands allowed
    assert call(0, 5, 7, 0, 7, P, 7, 0, 1) == OK      # B is non-empty, so it must be given
    assert call(5, 0, 7, P, 7, 0, 7, 0, 5) == OK      # A is non-empty, so it must be given
    assert call(0, 0, 0, 0, 1, 0, 1, 0, 1) == OK


def test_status_strings():
    for s in (OK, ERR_DIM, ERR_LD, ERR_NULL, ERR_EPI, ERR_HIP, 12345):
        assert isinstance(gb.gemm_bf16_status_string(s), str) and gb.gemm_bf16_status_string(s)
    assert gb.gemm_bf16_last_hip_error() == 0


def test_kernel_selection_names():
    # pointer alignment and divisibility decide the path; P is 16-byte aligned
    name = gb.gemm_bf16_kernel_name
    assert name(4096, 4096, 4096, P, 4096, P, 4096, P, 4096) == "ring256x256x64"
    assert name(8192, 14336, 4096, P, 4096, P, 4096, P, 8192) == "ring256x256x64"
    # tails (K not a multiple of 64, M or N not of 256): the masked ring kernel
    assert name(4096, 4096, 4064, P, 4064, P, 4064, P, 4096) == "ring256x256x64_masked"
    assert name(4000, 4000, 4000, P, 4000, P, 4000, P, 4000) == "ring256x256x64_masked"
    assert name(2048, 4096, 4096, P, 4096, P, 4096, P, 2048) == "tile128x128x64_s4"  # 128 ring tiles: half the CUs
    assert name(2304, 4096, 4096, P, 4096, P, 4096, P, 2304) == "ring256x256x64"     # 144 ring tiles
    assert name(4000, 2000, 1000, P, 1000, P, 1000, P, 4000) == "tile128x128x64_s4_masked"  # 128 ring tiles: half
    assert name(4000, 2100, 1000, P, 1000, P, 1000, P, 4000) == "ring256x256x64_masked"     # 144 ring tiles
    assert name(256, 256, 256, P, 256, P, 256, P, 256) == "tile128x128x64_s4"
    # small grids of 128-tiles with enough K-slices: split-K
    assert name(1024, 1024, 4096, P, 4096, P, 4096, P, 1024) == "splitk128x128x64"
    assert name(512, 512, 8192, P, 8192, P, 8192, P, 512) == "splitk128x128x64"
    assert name(512, 512, 2048, P, 2048, P, 2048, P, 512) == "splitk128x128x64"     # 16 tiles, 32 slices
    assert name(1024, 1024, 2048, P, 2048, P, 2048, P, 1024) == "tile128x128x64_s4"  # 64 tiles: K too short to split
    assert name(1024, 512, 2048, P, 2048, P, 2048, P, 1024) == "splitk128x128x64"     # 32 tiles, 32 slices
    assert name(768, 768, 2048, P, 2048, P, 2048, P, 768) == "tile128x128x64_s4"     # 36 tiles, 32 slices
    assert name(1024, 1024, 1024, P, 1024, P, 1024, P, 1024) == "tile128x128x64_s4"
    assert name(512, 512, 512, P, 512, P, 512, P, 512) == "tile128x128x64_s4"   # 8 slices: no split
    assert name(2048, 2048, 4096, P, 4096, P, 4096, P, 2048) == "tile128x128x64_s4"  # 256 tiles
    assert name(1000, 1000, 1000, P, 1000, P, 1000, P, 1000) == "tile128x128x64_s4_masked"
    assert name(1000, 1000, 4096, P, 4096, P, 4096, P, 1000) == "splitk128x128x64_masked"
    assert name(1000, 1000, 1004, P, 1004, P, 1004, P, 1000) == "generic64x64x32"   # K % 8 != 0
    assert name(64, 8192, 8192, P, 8192, P, 8192, P, 64) == "skinny"
    assert name(32, 4096, 1024, P, 1024, P, 1024, P, 32) == "skinny"
    assert name(48, 4096, 1024, P, 1024, P, 1024, P, 48) == "skinny"
    assert name(1, 4096, 4096, P, 4096, P, 4096, P, 8) == "gemv"
    assert name(4, 4096, 4096, P, 4096, P, 4096, P, 4) == "gemv"
    assert name(2, 8192, 8192, P, 8192, P, 8192, P, 2) == "gemv"
    assert name(3, 8192, 8192, P, 8192, P, 8192, P, 3) == "skinny"   # large B: A shared per strip
    assert name(4, 16384, 8192, P, 8192, P, 8192, P, 4) == "skinny"
    # more strips than compute units: the matrix-vector kernel over a K of
    # 2048 to 8191, the masked 128x128 tiles below that
    assert name(4, 16384, 4096, P, 4096, P, 4096, P, 4) == "gemv"
    assert name(3, 65536, 2048, P, 2048, P, 2048, P, 3) == "gemv"
    assert name(3, 65536, 1024, P, 1024, P, 1024, P, 3) == "tile128x128x64_s4_masked"
    assert name(4, 4096, 16376, P, 16376, P, 16376, P, 4) == "gemv"    # N * K just below 2^26
    assert name(5, 4096, 4096, P, 4096, P, 4096, P, 8) == "skinny"
    assert name(1, 4096, 4100, P, 4100, P, 4100, P, 1) == "generic64x64x32"   # K % 8 != 0
    assert name(48, 4096, 1020, P, 1020, P, 1020, P, 48) == "generic64x64x32"
    assert name(65, 4096, 1024, P, 1024, P, 1024, P, 72) != "skinny"
    # at most 64 columns: the streaming kernel on the transposed product
    assert name(8192, 64, 8192, P, 8192, P, 8192, P, 8192) == "skinny_t"
    assert name(8192, 1, 8192, P, 8192, P, 8192, P, 8192) == "skinny_t"
    assert name(1000, 17, 3000, P, 3000, P, 3000, P, 1001) == "skinny_t"
    assert name(64, 64, 4096, P, 4096, P, 4096, P, 64) == "skinny"       # both small: the direct kernel
    assert name(8192, 65, 8192, P, 8192, P, 8192, P, 8192) != "skinny_t"
    assert name(8192, 48, 1020, P, 1020, P, 1020, P, 8192) == "generic64x64x32"   # K % 8 != 0
    assert name(8192, 48, 1024, P + 2, 1024, P, 1024, P, 8192) != "skinny_t"     # A not 16-byte aligned
    # more 32-wide strips than compute units over fewer than 8 slices of 256:
    # the masked 128x128 tiles
    assert name(64, 65536, 512, P, 512, P, 512, P, 64) == "tile128x128x64_s4_masked"
    assert name(65536, 64, 1024, P, 1024, P, 1024, P, 65536) == "tile128x128x64_s4_masked"
    assert name(65536, 1, 512, P, 512, P, 512, P, 65536) == "tile128x128x64_s4_masked"
    assert name(65536, 64, 2048, P, 2048, P, 2048, P, 65536) == "skinny_t"
    assert name(64, 65536, 2048, P, 2048, P, 2048, P, 64) == "skinny"
    assert name(64, 8192, 256, P, 256, P, 256, P, 64) == "skinny"       # one strip per compute unit
    assert name(8192, 64, 256, P, 256, P, 256, P, 8192) == "skinny_t"
    assert name(4096, 4096, 4096, P + 2, 4096, P, 4096, P, 4096) == "generic64x64x32"
    assert name(4096, 4096, 4100, P, 4100, P, 4100, P, 4096) == "generic64x64x32"
    assert name(4096, 4096, 0, P, 1, P, 1, P, 4096) == "generic64x64x32"
    assert name(0, 4096, 4096, P, 4096, P, 4096, P, 1) == "none"
    # maximum sizes: the fast kernels address a tile's rows with 32-bit byte
    # offsets; leading dimensions too large for that take the next kernel
    # whose offsets still fit, down to the bounds-checked one (64-bit indexing)
    big = 1 << 22   # 256 rows * 2^22 elements * 2 bytes = 2^31
    assert name(4096, 4096, 4096, P, big, P, 4096, P, 4096) == "tile128x128x64_s4"
    assert name(4096, 4096, 4096, P, 2 * big, P, 4096, P, 4096) == "generic64x64x32"
    assert name(64, 8192, 8192, P, big * 2, P, 8192, P, 64) == "skinny"      # 64 rows: 2^30 bytes
    assert name(64, 8192, 8192, P, big * 4, P, 8192, P, 64) == "generic64x64x32"
    assert name(8192, 64, 8192, P, 8192, P, big * 2, P, 8192) == "skinny_t"  # 64 columns of B: 2^30 bytes
    assert name(8192, 64, 8192, P, 8192, P, big * 4, P, 8192) != "skinny_t"
    assert name(1, 4096, 4096, P, 4096, P, big * 32, P, 1) == "gemv"          # 4 columns: 2^30 bytes
    assert name(1, 4096, 4096, P, 4096, P, big * 64, P, 1) == "generic64x64x32"
    assert name(-1, 4096, 4096, P, 4096, P, 4096, P, 1) == "none"


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(gb, "_lib", None)
    monkeypatch.setattr(gb, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        gb.library()
