"""Seeded random shapes through all three entry points, each against the
oracle element by element (the DeepGEMM article's section 4.2: boundaries
and indexing over shapes the fixed cases do not name).

Every case is a valid call: sizes from 1 to about 2100 (log-uniform), K a
multiple of 8 (or 16 for FP8) most of the time and anything otherwise, leading
dimensions padded at random (multiples of 8 most of the time), now and then a
base address off its 16-byte alignment, and random alpha, beta, bias and
activation.  Whichever kernel the library picks for a case, the result must
be within the tolerance; the case line names the kernel.
"""
from __future__ import annotations

import numpy as np
import pytest

from tests.test_gpu_parity import check_fp8, check_full, check_q8

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

EPIS = ("none", "gelu_tanh", "relu")


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _dim(rng, hi=2100):
    lo = 64 if rng.random() < 0.7 else 1  # mostly tile-sized, sometimes a few rows or columns
    return int(np.exp(rng.uniform(np.log(lo), np.log(hi))))


def _k(rng, multiple):
    k = _dim(rng, 3000)
    if rng.random() < 0.9:
        k = max(multiple, k // multiple * multiple)
    return max(k, 1)


def _ld(rng, base, multiple):
    pad = int(rng.integers(0, 5)) * multiple if rng.random() < 0.9 else int(rng.integers(1, 40))
    return base + pad


def _case(seed, multiple):
    rng = np.random.default_rng(seed)
    M, N, K = _dim(rng), _dim(rng), _k(rng, multiple)
    while M * N * K > 1.2e9:  # keeps the oracle's share of a case under a second
        K = max(1, K // 2)
    lda, ldb, ldc = _ld(rng, K, multiple), _ld(rng, K, multiple), _ld(rng, M, 8)
    offsets = tuple(int(rng.integers(0, 2)) if rng.random() < 0.05 else 0 for _ in range(3))
    beta = float(rng.choice([0.0, 0.5, -1.0]))
    return dict(M=M, N=N, K=K, lda=lda, ldb=ldb, ldc=ldc, offsets=offsets, alpha=float(rng.uniform(0.5, 1.5)),
                beta=beta, use_bias=bool(rng.random() < 0.5), epilogue=str(rng.choice(EPIS)), seed=seed)


@pytest.mark.parametrize("seed", range(64))
def test_random_bf16(seed):
    c = _case(1000 + seed, 8)
    check_full(f"random bf16 #{seed}", c["M"], c["N"], c["K"], lda=c["lda"], ldb=c["ldb"], ldc=c["ldc"],
               alpha=c["alpha"], beta=c["beta"], use_bias=c["use_bias"], epilogue=c["epilogue"],
               offsets=c["offsets"], seed=c["seed"], poison_pad=True)


@pytest.mark.parametrize("seed", range(24))
def test_random_int8_output(seed):
    c = _case(2000 + seed, 8)
    rng = np.random.default_rng(seed)
    ldq = c["M"] + int(rng.integers(0, 3)) * 8
    check_q8(f"random q8 #{seed}", c["M"], c["N"], c["K"], ldq=ldq, ldc=c["ldc"], alpha=c["alpha"],
             beta=c["beta"], use_bias=c["use_bias"], epilogue=c["epilogue"], zp=int(rng.integers(-20, 21)),
             q_offset=int(rng.integers(0, 2)) if rng.random() < 0.2 else 0, seed=c["seed"])


@pytest.mark.parametrize("seed", range(24))
def test_random_fp8(seed):
    c = _case(3000 + seed, 16)
    check_fp8(f"random fp8 #{seed}", c["M"], c["N"], c["K"], lda=c["lda"], ldb=c["ldb"], ldc=c["ldc"],
              alpha=c["alpha"], beta=c["beta"], use_bias=c["use_bias"], epilogue=c["epilogue"],
              scales=bool(seed % 4 != 3), offsets=c["offsets"], seed=c["seed"], poison_pad=True)
