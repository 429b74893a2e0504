"""Seeded synthetic inputs for the bf16 GEMM workloads.

This module only draws random numbers and stores them as bf16 bit patterns
(uint16).  It holds none of the GEMM's arithmetic, so the GPU path and the
CPU oracle can both be fed from it without sharing any of their code.

Recipe (the pages initialise every matrix from a normal distribution with
mean 0 and standard deviation 1 -- "Outperforming cuBLAS on H100: a worklog",
section "Experimental setup"):

* operand j of workload i is drawn from numpy's PCG64 generator seeded with
  ``1000*i + j`` (j = 1: A, 2: B, 3: the initial C, 4: bias);
* values are float32 standard normals (bias: multiplied by 0.1 in float32,
  i.e. standard deviation 0.1), rounded to bf16 nearest-even;
* buffers are filled in storage order: A as M rows of K (row-major), B as N
  columns of K (column-major), C0 as N columns of M (column-major);
* int8-output workloads also draw one float32 scale per row (operand j = 5),
  uniform in [lo, hi), and use a fixed zero point;
* fp8-input workloads round the same float32 normals to OCP FP8 E4M3 (torch's
  float8_e4m3fn conversion, nearest-even; N(0,1) samples never reach its
  range limit of 448) and draw per-row and per-column float32 scales
  (operands j = 6 and 7), uniform in [0.5, 2).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    index: int          # seed block: seeds are 1000*index + operand id
    M: int
    N: int
    K: int
    alpha: float = 1.0
    beta: float = 0.0
    bias: bool = False
    epilogue: str = "none"
    bound: str = "mfma"  # which roofline limits it: "mfma" or "hbm"
    out: str = "bf16"    # "bf16", or "int8" (per-row quantized output)
    inp: str = "bf16"    # "bf16", or "fp8" (E4M3 operands with per-row / per-column scales)
    scale_range: tuple = (0.25, 0.75)  # int8 output: per-row scales, uniform
    zero_point: int = 0                # int8 output: zero point
    notes: str = field(default="", compare=False)

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def in_bytes(self) -> int:
        return 1 if self.inp == "fp8" else 2

    @property
    def algorithmic_bytes(self) -> int:
        """Minimum HBM bytes: read A and B once, write C once (read C0 if
        beta); an int8 output writes 1 byte per element and reads M scales."""
        b = self.in_bytes * (self.M * self.K + self.K * self.N)
        b += (1 if self.out == "int8" else 2) * self.M * self.N
        if self.inp == "fp8":
            b += 4 * (self.M + self.N)
        if self.beta != 0.0:
            b += 2 * self.M * self.N
        if self.bias:
            b += 2 * self.N
        if self.out == "int8":
            b += 4 * self.M
        return b


# The five workloads: A row-major, B and C column-major, fp32 accumulation,
# bf16 output.  The 4096^3 square is the pages' headline shape.
WORKLOADS = {
    w.name: w
    for w in [
        Workload("square_256", 0, 256, 256, 256,
                 notes="smallest case; the oracle checks every element"),
        Workload("square_4096", 1, 4096, 4096, 4096,
                 notes="headline shape of the worklog"),
        Workload("square_8192", 2, 8192, 8192, 8192,
                 notes="large grid: several tiles per compute unit"),
        Workload("gelu_8192x14336x4096", 3, 8192, 14336, 4096,
                 alpha=1.0, beta=0.5, bias=True, epilogue="gelu_tanh",
                 notes="C = GELU_tanh(1.0*A*B + 0.5*C0 + bias[n])"),
        Workload("skinny_64x8192x8192", 4, 64, 8192, 8192, bound="hbm",
                 notes="memory-bound: B (128 MiB) is streamed once"),
        # beyond the five: a shape with tails in M, N and K (tiles of 256 and
        # K-slices of 64 do not divide it), for the masked fast path
        Workload("ragged_4000x4000x4000", 5, 4000, 4000, 4000,
                 notes="tails in every dimension: 4000 = 15*256 + 160 = 62*64 + 32"),
        # the fused quantizing epilogue of the DeepGEMM article (section
        # 6.2) on the epilogue case's shape: bias, ReLU, per-row int8
        Workload("q8relu_8192x14336x4096", 6, 8192, 14336, 4096, bias=True, epilogue="relu",
                 out="int8", zero_point=-20,
                 notes="Q = sat8(rne(relu(A*B + bias[n]) * scale[m] - 20))"),
        # the DeepGEMM article's small shapes (section 5.1): one-row decode
        # (memory-bound: B is read once) and a small square-ish product
        Workload("decode_1x4096x4096", 7, 1, 4096, 4096, bound="hbm",
                 notes="M = 1: a matrix-vector product, B (32 MiB) streamed once"),
        Workload("mid_1024x1024x4096", 8, 1024, 1024, 4096,
                 notes="64 tiles of 128x128 for 256 compute units"),
        # FP8 inputs (the DeepGEMM article, sections 1.2 and 6.3) on the
        # headline shape: E4M3 operands, per-row / per-column scales
        Workload("fp8_4096", 9, 4096, 4096, 4096, inp="fp8",
                 notes="C = sa[m] sb[n] (A*B), A and B in OCP FP8 E4M3"),
        # the memory-bound case with FP8 operands: B (64 MiB) streamed once
        Workload("fp8_skinny_64x8192x8192", 10, 64, 8192, 8192, inp="fp8", bound="hbm",
                 notes="C = sa[m] sb[n] (A*B), E4M3 operands, 64 rows"),
        # FP8 on the small grid of the DeepGEMM article's shapes (section 5.1)
        Workload("fp8_mid_1024x1024x4096", 11, 1024, 1024, 4096, inp="fp8",
                 notes="64 tiles of 128x128 for 256 compute units, E4M3 operands"),
        # the memory-bound case transposed: 64 columns, so A (128 MiB) is
        # the operand streamed once
        Workload("tall_8192x64x8192", 12, 8192, 64, 8192, bound="hbm",
                 notes="N = 64: A (128 MiB) streamed once"),
    ]
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 samples to bf16 bit patterns, nearest-even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("input samples must be finite")
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def normal_bf16(seed: int, numel: int, scale: float = 1.0) -> np.ndarray:
    """numel i.i.d. N(0, scale^2) samples as bf16 bits (uint16), seeded."""
    g = np.random.Generator(np.random.PCG64(seed))
    x = g.standard_normal(numel, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return f32_to_bf16_bits(x)


def operand_seed(index: int, operand: str) -> int:
    return 1000 * index + {"A": 1, "B": 2, "C0": 3, "bias": 4, "scale": 5, "scale_a": 6, "scale_b": 7}[operand]


def normal_fp8(seed: int, numel: int, scale: float = 1.0) -> np.ndarray:
    """numel i.i.d. N(0, scale^2) samples as OCP FP8 E4M3 bytes (uint8), seeded."""
    import torch
    g = np.random.Generator(np.random.PCG64(seed))
    x = g.standard_normal(numel, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    if numel and float(np.abs(x).max()) >= 448.0:
        raise ValueError("sample outside the E4M3 range")
    return torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def uniform_f32(seed: int, numel: int, lo: float, hi: float) -> np.ndarray:
    """numel i.i.d. float32 samples, uniform in [lo, hi), seeded."""
    g = np.random.Generator(np.random.PCG64(seed))
    return (np.float32(lo) + g.random(numel, dtype=np.float32) * np.float32(hi - lo)).astype(np.float32)


def make_inputs(w: Workload, lda=None, ldb=None, ldc=None) -> dict:
    """Host buffers (flat uint16, storage order) for workload w.

    With padded leading dimensions the padding elements are filled from the
    same stream (they must never influence the result).
    """
    lda = w.K if lda is None else lda
    ldb = w.K if ldb is None else ldb
    ldc = w.M if ldc is None else ldc
    draw = normal_fp8 if w.inp == "fp8" else normal_bf16
    out = {
        "A": draw(operand_seed(w.index, "A"), w.M * lda),
        "B": draw(operand_seed(w.index, "B"), w.N * ldb),
        "lda": lda, "ldb": ldb, "ldc": ldc,
    }
    if w.inp == "fp8":
        out["scale_a"] = uniform_f32(operand_seed(w.index, "scale_a"), w.M, 0.5, 2.0)
        out["scale_b"] = uniform_f32(operand_seed(w.index, "scale_b"), w.N, 0.5, 2.0)
    if w.beta != 0.0:
        out["C0"] = normal_bf16(operand_seed(w.index, "C0"), w.N * ldc)
    if w.bias:
        out["bias"] = normal_bf16(operand_seed(w.index, "bias"), w.N, scale=0.1)
    if w.out == "int8":
        out["scale"] = uniform_f32(operand_seed(w.index, "scale"), w.M, *w.scale_range)
    return out


def random_case(seed: int, M: int, N: int, K: int, lda=None, ldb=None, ldc=None,
                with_c0: bool = False, with_bias: bool = False) -> dict:
    """Ad-hoc seeded case for tests: same recipe, seeds seed+1..seed+4."""
    lda = K if lda is None else lda
    ldb = K if ldb is None else ldb
    ldc = max(M, 1) if ldc is None else ldc
    out = {
        "A": normal_bf16(seed + 1, max(M * lda, 0)),
        "B": normal_bf16(seed + 2, max(N * ldb, 0)),
        "lda": max(lda, 1), "ldb": max(ldb, 1), "ldc": ldc,
    }
    if with_c0:
        out["C0"] = normal_bf16(seed + 3, N * ldc)
    if with_bias:
        out["bias"] = normal_bf16(seed + 4, N, scale=0.1)
    return out
