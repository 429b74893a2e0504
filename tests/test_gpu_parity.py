"""GPU parity: the HIP library (called through its C ABI) against the CPU
oracle on the same seeded inputs, element by element, within
|gpu - oracle| <= 2 ulp_bf16(oracle) + 1e-3 sqrt(K).

Small and medium shapes are compared in full (several tiles and ragged
tails); the five benchmark workloads run at full size, in the launch
configuration the benchmark times, and are compared on sampled elements
(whole tiles at the corners plus random elements) that the oracle evaluates
one by one.
"""
from __future__ import annotations

import os

import numpy as np
import pytest

import oracle
from bf16_gemm_fp32_amd import inputs
from tests.tolerance import assert_q8_within_tolerance, assert_within_tolerance, bits_to_f64

torch = pytest.importorskip("torch")
gb = pytest.importorskip("bf16_gemm_fp32_amd")

pytestmark = pytest.mark.gpu

NAN_BF16 = 0x7FC0
EPI = {"none": 0, "gelu_tanh": 1, "relu": 2}
Q8_POISON = 0x55  # int8 padding rows must keep it


def _threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gb.library()
    yield


def to_dev(bits: np.ndarray, offset: int = 0):
    """Device copy of a uint16 buffer, optionally starting `offset` elements
    into a larger allocation (to break 16-byte alignment).  Returns the full
    tensor and the pointer of the data start."""
    full = torch.zeros(bits.size + offset + 8, dtype=torch.int16, device="cuda")
    full[offset:offset + bits.size] = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()
    return full, full.data_ptr() + 2 * offset


def from_dev(t, offset, n):
    return t[offset:offset + n].cpu().numpy().view(np.uint16).copy()


def run_gpu(M, N, K, A, lda, B, ldb, C_init, ldc, alpha, beta, bias, epilogue, offsets=(0, 0, 0)):
    a_t, a_p = to_dev(A, offsets[0])
    b_t, b_p = to_dev(B, offsets[1])
    c_t, c_p = to_dev(C_init, offsets[2])
    bias_p = 0
    if bias is not None:
        bias_t, bias_p = to_dev(bias)
    stream = torch.cuda.current_stream().cuda_stream
    st = gb.gemm_bf16(M, N, K, a_p, lda, b_p, ldb, c_p, ldc, alpha, beta, bias_p, EPI[epilogue], stream)
    assert st == 0, gb.gemm_bf16_status_string(st)
    torch.cuda.synchronize()
    return from_dev(c_t, offsets[2], C_init.size)


def check_full(tag, M, N, K, lda=None, ldb=None, ldc=None, alpha=1.0, beta=0.0, use_bias=False,
               epilogue="none", offsets=(0, 0, 0), seed=0, expect_kernel=None, poison_pad=False):
    lda = max(K, 1) if lda is None else lda
    ldb = max(K, 1) if ldb is None else ldb
    ldc = max(M, 1) if ldc is None else ldc
    case = inputs.random_case(seed, M, N, K, lda, ldb, ldc, with_c0=True, with_bias=use_bias)
    if poison_pad:
        # operand padding (k >= K within a row of A / a column of B) is NaN:
        # a kernel that reads it produces NaN
        for key, ld, rows in (("A", lda, M), ("B", ldb, N)):
            if ld > K:
                case[key].reshape(rows, ld)[:, K:] = NAN_BF16
    C0 = case["C0"]
    # beta == 0: C starts as NaN everywhere, which must not leak
    C_init = C0 if beta != 0.0 else np.full_like(C0, NAN_BF16)
    bias = case.get("bias") if use_bias else None
    # the selection only looks at alignment: an aligned stand-in base plus the offsets
    kname = gb.gemm_bf16_kernel_name(M, N, K, 4096 + 2 * offsets[0], lda, 4096 + 2 * offsets[1], ldb,
                                     4096 + 2 * offsets[2], ldc)
    say(f"[parity] {tag}: M={M} N={N} K={K} lda={lda} ldb={ldb} ldc={ldc} alpha={alpha} beta={beta} "
        f"bias={use_bias} epi={epilogue} offsets={offsets} kernel={kname}")
    if expect_kernel is not None:
        assert kname == expect_kernel
    got = run_gpu(M, N, K, case["A"], lda, case["B"], ldb, C_init, ldc, alpha, beta, bias, epilogue, offsets)
    ref = oracle.gemm(M, N, K, case["A"], lda, case["B"], ldb, C0, ldc, alpha, beta, bias, epilogue,
                      nthreads=_threads())
    g2 = got.reshape(N, ldc)
    r2 = ref.reshape(N, ldc)
    rep = assert_within_tolerance(g2[:, :M], r2[:, :M], K, tag)
    # rows M..ldc-1 of every column are not part of C: untouched
    if ldc > M:
        assert np.array_equal(g2[:, M:], C_init.reshape(N, ldc)[:, M:]), f"{tag}: padding written"
    say(f"[parity] {tag}: ok max_err/tol={rep['max_err_over_tol']:.3f} mean_err/tol={rep['mean_err_over_tol']:.4f} "
        f"exact={rep['exact']}/{rep['n']}")
    return rep


# ------------------------------------------------------- tile-path shapes ---

@pytest.mark.parametrize("M,N,K,kernel", [
    (256, 256, 256, "tile128x128x64_s4"),
    (512, 384, 192, "tile128x128x64_s4"),     # 3 K-slices (odd)
    (512, 384, 256, "tile128x128x64_s4"),     # 4 K-slices (even)
    (4608, 2048, 320, "ring256x256x64"),      # 144 tiles of 256, 5 slices of 64
    (4608, 2048, 64, "ring256x256x64"),       # a single K-slice
    (4096, 2048, 320, "tile128x128x64_s4"),   # 128 ring tiles, half the CUs: 128x128 tiles, two per CU
    (4608, 2048, 352, "ring256x256x64_masked"),  # K % 64 == 32: a half-empty last slice
    (4608, 2048, 32, "ring256x256x64_masked"),   # a single half-empty K-slice
    (4096, 2048, 352, "tile128x128x64_s4_masked"),  # half the CUs in ring tiles, with a K tail: 128x128 masked
    (4096, 4608, 256, "tile128x128x64_s4"),   # 288 ring tiles, just over one round: 1152 128x128 tiles, 4.5 per CU
])
def test_tile_paths_full(M, N, K, kernel):
    check_full(f"tile {M}x{N}x{K}", M, N, K, seed=M + N + K, expect_kernel=kernel)


def test_tile_path_epilogue_full():
    check_full("ring256 epilogue", 4608, 2048, 192, alpha=1.0, beta=0.5, use_bias=True,
               epilogue="gelu_tanh", seed=11, expect_kernel="ring256x256x64")
    check_full("masked ring epilogue", 4608, 2048, 160, alpha=1.0, beta=0.5, use_bias=True,
               epilogue="gelu_tanh", seed=16, expect_kernel="ring256x256x64_masked")
    check_full("tile128 epilogue", 512, 512, 128, alpha=-0.75, beta=-1.5, use_bias=True,
               epilogue="none", seed=12, expect_kernel="tile128x128x64_s4")
    check_full("tile128 gelu only", 384, 256, 320, alpha=2.0, epilogue="gelu_tanh", seed=13,
               expect_kernel="tile128x128x64_s4")


def test_tile_path_padded_leading_dims():
    check_full("tile128 padded ld", 512, 256, 256, lda=264, ldb=272, ldc=520, beta=0.25, use_bias=True,
               seed=14, expect_kernel="tile128x128x64_s4")
    check_full("ring256 padded ld", 4608, 2048, 128, lda=136, ldb=192, ldc=4616, seed=15,
               expect_kernel="ring256x256x64")
    check_full("masked ring padded ld", 4608, 2048, 96, lda=104, ldb=136, ldc=4616, seed=17,
               expect_kernel="ring256x256x64_masked")


# Split-K on the 128x128 tiles (small grids): the K-slices are cut into
# ranges whose fp32 partials a second kernel adds in range order, then runs
# the epilogue.  Shapes with 2, 3 (uneven: 9, 9, 7 slices), 4, 8 and 16
# ranges, padded leading dimensions, every epilogue combination, forced
# split counts, and run-to-run bit equality.
SPLITK = "splitk128x128x64"


@pytest.mark.parametrize("M,N,K", [
    (1536, 1024, 4096),  # 96 tiles, 64 slices: 2 ranges
    (256, 256, 1600),    # 4 tiles, 25 slices: 3 ranges of 9, 9, 7
    (512, 512, 2048),    # 16 tiles, 32 slices: 4 ranges
    (256, 384, 2048),    # 6 tiles: 4 ranges
    (512, 256, 4096),    # 8 tiles: 8 ranges
    (128, 128, 8192),    # 1 tile: 16 ranges
])
def test_splitk_full(M, N, K):
    check_full(f"splitk {M}x{N}x{K}", M, N, K, seed=M + 3 * N + K, expect_kernel=SPLITK)


@pytest.mark.parametrize("beta,use_bias,epi", [(b, u, e) for b in (0.0, -0.75) for u in (False, True)
                                               for e in ("none", "gelu_tanh", "relu")])
def test_splitk_epilogue_combinations(beta, use_bias, epi):
    check_full(f"splitk beta={beta} bias={use_bias} {epi}", 256, 384, 2048, alpha=1.25, beta=beta,
               use_bias=use_bias, epilogue=epi, seed=40 + int(abs(beta) * 4) + 2 * use_bias + len(epi),
               expect_kernel=SPLITK)


def test_splitk_padded_leading_dims():
    check_full("splitk padded ld", 512, 256, 2048, lda=2056, ldb=2064, ldc=520, beta=0.5, use_bias=True,
               epilogue="gelu_tanh", seed=51, expect_kernel=SPLITK)


@pytest.mark.parametrize("splits", [2, 3, 5, 7])
def test_splitk_forced_split_counts(splits, monkeypatch):
    monkeypatch.setenv("GEMM_BF16_SPLITK_SPLITS", str(splits))
    check_full(f"splitk forced {splits} ranges", 384, 256, 3840, beta=0.25, use_bias=True, seed=60 + splits,
               expect_kernel=SPLITK)


@pytest.mark.parametrize("M,N,K", [(1024, 1024, 1024), (512, 512, 1024), (256, 384, 1024)])
def test_short_k_small_grids_stay_unsplit(M, N, K):
    check_full(f"unsplit {M}x{N}x{K}", M, N, K, beta=0.5, use_bias=True, epilogue="gelu_tanh", seed=M + N + K,
               expect_kernel="tile128x128x64_s4")


def test_splitk_deterministic():
    M, N, K = 512, 256, 4096
    case = inputs.random_case(70, M, N, K, with_c0=False, with_bias=False)
    C_init = np.full(N * M, NAN_BF16, np.uint16)
    runs = [run_gpu(M, N, K, case["A"], K, case["B"], K, C_init, M, 1.0, 0.0, None, "none") for _ in range(3)]
    assert np.array_equal(runs[0], runs[1]) and np.array_equal(runs[0], runs[2]), "split-K results vary"


# Every tile kernel forced onto shapes whose K-slice count walks through the
# pipeline's prologue and tail cases (1 .. 10 slices, fewer and more slices
# than LDS stages, odd and even counts).
FORCEABLE = {"tile256x256x32_s5": 32, "tile128x128x64_s4": 64, "ring256x256x64": 64,
             "ring256x256x64_mfma32": 64, "ring256x256x64_w8": 64, "ring256x256x64_masked": 8,
             "generic64x64x32": 1, "tile128x128x64_s4_masked": 8}


@pytest.mark.parametrize("kernel", list(FORCEABLE))
@pytest.mark.parametrize("K", [32, 64, 96, 128, 160, 192, 256, 320, 448, 640])
def test_forced_kernels_all_slice_counts(kernel, K, monkeypatch):
    M, N = 1024, 512
    bk = FORCEABLE[kernel]
    if K % bk:
        pytest.skip(f"{kernel} needs K % {bk} == 0")
    monkeypatch.setenv("GEMM_BF16_FORCE_KERNEL", kernel)
    check_full(f"forced {kernel} K={K}", M, N, K, beta=0.5 if K % 64 else 0.0, use_bias=K == 96,
               seed=K + len(kernel), expect_kernel=kernel)


# Tails on small and mid-sized grids: the masked 128x128 kernel (whole K)
# and its split-K (whole tiles into a padded workspace; the reduction writes
# a chunk that straddles M element by element).
T128M = "tile128x128x64_s4_masked"
SPLITKM = "splitk128x128x64_masked"


@pytest.mark.parametrize("M,N,K,lda,ldb,ldc,kernel", [
    (1000, 1000, 1000, 1000, 1000, 1000, T128M),   # 64 tiles, K tail in the last slice
    (2000, 2000, 2000, 2000, 2000, 2000, T128M),   # 256 tiles
    (1001, 999, 1000, 1008, 1000, 1008, T128M),    # M % 8 == 1, N tail, padded lda / ldc
    (130, 70, 520, 520, 528, 136, T128M),          # one row / one column past a tile
    (1000, 1000, 4096, 4096, 4096, 1000, SPLITKM),  # 64 tiles: split K
    (1001, 520, 8200, 8200, 8208, 1008, SPLITKM),  # M % 8 == 1 in the reduction, K tail
    (250, 130, 3000, 3000, 3000, 256, SPLITKM),    # 4 tiles, a K tail in the last range
    (1500, 700, 1000, 1000, 1000, 1500, T128M),    # ldc % 8 != 0: element-wise C
    (1001, 777, 4000, 4000, 4000, 1003, SPLITKM),  # ldc % 8 != 0 in the reduction
])
def test_masked_small_grid_shapes(M, N, K, lda, ldb, ldc, kernel):
    check_full(f"masked small grid {M}x{N}x{K}", M, N, K, lda=lda, ldb=ldb, ldc=ldc, beta=0.5, use_bias=True,
               epilogue="gelu_tanh", seed=M + N + K + 300, expect_kernel=kernel, poison_pad=True)


@pytest.mark.parametrize("beta,use_bias,epi", [(b, u, e) for b in (0.0, -0.75) for u in (False, True)
                                               for e in ("none", "gelu_tanh", "relu")])
@pytest.mark.parametrize("M,N,K,ldc,kernel", [(999, 555, 320, 1000, T128M), (1000, 500, 4000, 1000, SPLITKM)])
def test_masked_small_grid_epilogue_combinations(M, N, K, ldc, kernel, beta, use_bias, epi):
    check_full(f"{kernel} beta={beta} bias={use_bias} {epi}", M, N, K, ldc=ldc, alpha=1.25, beta=beta,
               use_bias=use_bias, epilogue=epi, seed=310 + int(abs(beta) * 4) + 2 * use_bias + len(epi),
               expect_kernel=kernel)


def test_masked_small_grid_unaligned_c():
    check_full("masked medium unaligned C", 520, 300, 640, ldc=521, offsets=(0, 0, 3), beta=0.5, use_bias=True,
               epilogue="relu", seed=340, expect_kernel=T128M)
    check_full("masked splitk unaligned C", 520, 300, 4000, ldc=523, offsets=(0, 0, 5), beta=-0.5, use_bias=True,
               epilogue="gelu_tanh", seed=341, expect_kernel=SPLITKM)


@pytest.mark.parametrize("splits", [2, 3, 5])
def test_masked_splitk_forced_split_counts(splits, monkeypatch):
    monkeypatch.setenv("GEMM_BF16_SPLITK_SPLITS", str(splits))
    check_full(f"masked splitk forced {splits}", 377, 250, 2000, ldc=384, beta=0.25, use_bias=True,
               seed=330 + splits, expect_kernel=SPLITKM)


# The tile kernels are compiled once per epilogue combination (beta, bias,
# GELU): every combination on every tile configuration.
@pytest.mark.parametrize("kernel,M,N,K", [("tile256x256x32_s5", 2048, 1024, 160),
                                          ("tile128x128x64_s4", 512, 384, 192),
                                          ("ring256x256x64", 2048, 1024, 192),
                                          ("ring256x256x64_mfma32", 2048, 1024, 192),
                                          ("ring256x256x64_w8", 2048, 1024, 192)])
@pytest.mark.parametrize("beta,use_bias,epi", [(b, u, e) for b in (0.0, -0.75) for u in (False, True)
                                               for e in ("none", "gelu_tanh", "relu")])
def test_tile_epilogue_combinations(kernel, M, N, K, beta, use_bias, epi, monkeypatch):
    monkeypatch.setenv("GEMM_BF16_FORCE_KERNEL", kernel)
    check_full(f"{kernel} beta={beta} bias={use_bias} {epi}", M, N, K, alpha=1.25, beta=beta,
               use_bias=use_bias, epilogue=epi, seed=int(abs(beta) * 4) + 2 * use_bias + len(epi),
               expect_kernel=kernel)


# The masked ring kernel (shapes with tails): M and N tails of every size
# class (1 row/column, less than a wave's 128, straddling 8-row chunks), K
# tails down to a single 8-wide chunk, padded leading dimensions whose
# padding is NaN, and every epilogue combination.
MASKED = "ring256x256x64_masked"


@pytest.mark.parametrize("M,N,K,lda,ldb,ldc", [
    (300, 260, 72, 72, 72, 304),      # one full + one 8-wide K chunk past a slice
    (257, 513, 8, 16, 24, 264),        # a single 8-wide K chunk, 1-row / 1-column tails
    (1000, 600, 1000, 1000, 1008, 1000),
    (1001, 777, 200, 208, 200, 1008),  # M % 8 == 1: the last 8-row chunk straddles M
    (255, 1, 136, 136, 144, 256),      # N = 1
    (1, 255, 64, 64, 64, 8),           # M = 1
    (520, 264, 4040, 4048, 4040, 528), # 63 full slices and a 8-wide K tail
    (512, 512, 4096, 4096, 4096, 512), # no tails at all through the masked path
])
def test_masked_ring_tails(M, N, K, lda, ldb, ldc, monkeypatch):
    monkeypatch.setenv("GEMM_BF16_FORCE_KERNEL", MASKED)
    check_full(f"masked {M}x{N}x{K}", M, N, K, lda=lda, ldb=ldb, ldc=ldc, beta=0.0, seed=M + N + K,
               expect_kernel=MASKED, poison_pad=True)


@pytest.mark.parametrize("beta,use_bias,epi", [(b, u, e) for b in (0.0, -0.75) for u in (False, True)
                                               for e in ("none", "gelu_tanh", "relu")])
def test_masked_ring_epilogue_combinations(beta, use_bias, epi, monkeypatch):
    monkeypatch.setenv("GEMM_BF16_FORCE_KERNEL", MASKED)
    check_full(f"masked beta={beta} bias={use_bias} {epi}", 777, 300, 200, ldc=784, alpha=1.25, beta=beta,
               use_bias=use_bias, epilogue=epi, seed=7 + int(abs(beta) * 4) + 2 * use_bias + len(epi),
               expect_kernel=MASKED, poison_pad=True)


def test_masked_ring_any_ldc_and_c_alignment():
    check_full("masked ring odd ldc", 4500, 2000, 320, ldc=4501, beta=0.5, use_bias=True, epilogue="gelu_tanh",
               seed=350, expect_kernel="ring256x256x64_masked")
    check_full("masked ring unaligned C", 4096, 2304, 256, ldc=4104, offsets=(0, 0, 3), beta=-0.5, seed=351,
               expect_kernel="ring256x256x64_masked")


def test_q8_exact_ring_unaligned_c0_takes_the_masked_instance():
    check_q8("q8 ring unaligned C0", 4096, 2048, 192, ldc=4100, beta=0.5, use_bias=True, epilogue="relu", zp=2,
             seed=352, expect_kernel="ring256x256x64_q8_masked")


def test_masked_ring_is_the_default_for_large_ragged_shapes():
    check_full("ragged default", 4500, 2000, 1000, beta=0.5, use_bias=True, epilogue="gelu_tanh", seed=51,
               expect_kernel=MASKED)


# The streaming kernel for at most 64 rows: slice counts through its ring
# prologue and tail, every strip width, K splits (the split-K reduction),
# row / column / K tails, epilogue combinations, padding.
SK = "skinny"


@pytest.mark.parametrize("M", [64, 32])
@pytest.mark.parametrize("K", [256, 512, 768, 1024, 1280, 2560])
def test_skinny_slice_counts(M, K, monkeypatch):
    monkeypatch.setenv("GEMM_BF16_SKINNY_SPLITS", "1")
    check_full(f"skinny M={M} K={K}", M, 1024, K, seed=M + K, expect_kernel=SK)


@pytest.mark.parametrize("cols", ["32", "64", "128"])
@pytest.mark.parametrize("splits", ["1", "2", "3", "7"])
def test_skinny_widths_and_splits(cols, splits, monkeypatch):
    monkeypatch.setenv("GEMM_BF16_SKINNY_COLS", cols)
    monkeypatch.setenv("GEMM_BF16_SKINNY_SPLITS", splits)
    check_full(f"skinny cols={cols} splits={splits}", 64, 1024, 4096, beta=0.5, use_bias=True, epilogue="gelu_tanh",
               seed=int(cols) + int(splits), expect_kernel=SK)
    check_full(f"skinny M=32 cols={cols} splits={splits}", 32, 512, 2048, seed=3 * int(cols) + int(splits),
               expect_kernel=SK)


@pytest.mark.parametrize("M,N,K,lda,ldb,ldc", [
    (1, 4096, 4096, 4096, 4096, 8),      # decode: one row
    (7, 1000, 1032, 1032, 1040, 8),      # 7 rows, N and K tails
    (16, 333, 8, 8, 8, 16),              # a single 8-wide K chunk
    (33, 96, 520, 528, 520, 40),         # just over one 32-row block
    (48, 4096, 1024, 1024, 1024, 48),
    (63, 129, 4104, 4104, 4112, 64),     # every tail at once
    (64, 1, 256, 256, 256, 64),          # one column
    (1, 4096, 4096, 4096, 4096, 1),      # decode with the natural ldc = 1
    (7, 512, 2048, 2048, 2048, 7),       # ldc not a multiple of 8
    (12, 300, 1024, 1024, 1032, 13),
])
@pytest.mark.parametrize("splits", ["1", "3"])
def test_skinny_tails(M, N, K, lda, ldb, ldc, splits, monkeypatch):
    monkeypatch.setenv("GEMM_BF16_SKINNY_SPLITS", splits)
    monkeypatch.setenv("GEMM_BF16_FORCE_KERNEL", SK)  # M <= 4 would take the matrix-vector kernel
    check_full(f"skinny tails {M}x{N}x{K} splits={splits}", M, N, K, lda=lda, ldb=ldb, ldc=ldc, beta=0.0,
               seed=M + N + K, expect_kernel=SK, poison_pad=True)


# The matrix-vector kernel (1 to 4 rows): several K blocks with tails, N
# tails inside a wave's columns, NaN padding, any ldc and C alignment,
# every epilogue combination.
GV = "gemv"


@pytest.mark.parametrize("M,N,K,lda,ldb,ldc", [
    (1, 4096, 4096, 4096, 4096, 1),      # decode: one full K block
    (2, 1000, 1032, 1032, 1040, 2),      # N % 4 == 0, K tail inside the block
    (3, 333, 8, 8, 8, 3),                # a single 8-wide K chunk; an odd N leaves a 1-column wave
    (4, 129, 4104, 4104, 4112, 4),       # whole blocks and an 8-wide last block
    (1, 1, 8, 8, 8, 1),                  # the smallest product
    (4, 4097, 8200, 8200, 8200, 8),      # two blocks and a tail; a 1-column last wave
    (1, 5, 12296, 12304, 12296, 1),      # three blocks and a tail
    (3, 2050, 4096, 4096, 4104, 5),      # ldc > M
])
def test_gemv_shapes(M, N, K, lda, ldb, ldc):
    check_full(f"gemv {M}x{N}x{K}", M, N, K, lda=lda, ldb=ldb, ldc=ldc, beta=0.0, seed=M + N + K + 5,
               expect_kernel=GV, poison_pad=True)


@pytest.mark.parametrize("beta,use_bias,epi", [(b, u, e) for b in (0.0, -0.75) for u in (False, True)
                                               for e in ("none", "gelu_tanh", "relu")])
def test_gemv_epilogue_combinations(beta, use_bias, epi):
    check_full(f"gemv beta={beta} bias={use_bias} {epi}", 3, 515, 1000, ldc=3, alpha=1.25, beta=beta,
               use_bias=use_bias, epilogue=epi, seed=80 + int(abs(beta) * 4) + 2 * use_bias + len(epi),
               expect_kernel=GV)


@pytest.mark.parametrize("M,N,K,ldc", [(3, 8192, 8192, 3), (4, 16384, 8192, 8)])
def test_three_and_four_rows_on_large_b_take_the_streaming_kernel(M, N, K, ldc):
    check_full(f"rows {M} large B", M, N, K, ldc=ldc, beta=0.5, use_bias=True, epilogue="gelu_tanh",
               seed=M * 7 + 3, expect_kernel="skinny")


def test_gemv_unaligned_c_with_beta():
    check_full("gemv unaligned C", 2, 777, 520, ldc=3, beta=0.5, use_bias=True, epilogue="gelu_tanh",
               offsets=(0, 0, 1), seed=93, expect_kernel=GV)


def test_skinny_unaligned_c_with_beta():
    check_full("skinny unaligned C", 40, 1000, 1024, ldc=41, beta=-0.5, use_bias=True, epilogue="relu",
               offsets=(0, 0, 3), seed=92, expect_kernel=SK)


@pytest.mark.parametrize("beta,use_bias,epi", [(0.5, True, "gelu_tanh"), (0.0, True, "none"),
                                               (-1.0, False, "gelu_tanh"), (0.25, True, "relu")])
@pytest.mark.parametrize("splits", ["1", "4"])
def test_skinny_epilogues_and_padding(beta, use_bias, epi, splits, monkeypatch):
    monkeypatch.setenv("GEMM_BF16_SKINNY_SPLITS", splits)
    check_full(f"skinny epilogue beta={beta} bias={use_bias} {epi}", 64, 2048, 4096, alpha=0.5, beta=beta,
               use_bias=use_bias, epilogue=epi, seed=41, expect_kernel=SK)
    check_full("skinny padded", 61, 512, 4096, lda=4104, ldb=4160, ldc=72, beta=beta, use_bias=use_bias,
               epilogue=epi, seed=42, expect_kernel=SK, poison_pad=True)


def test_skinny_split_k_is_deterministic_across_launches(monkeypatch):
    """Split-K: the last unit adds the partials in split order, whichever
    unit arrives last, and resets the strip counters -- repeated launches on
    one stream are bit-identical and match the unsplit kernel within the
    tolerance."""
    M, N, K = 64, 2048, 16384  # 32 strips of 64 columns, 8 splits of 8 slices
    case = inputs.random_case(91, M, N, K)
    C_init = np.zeros(M * N, np.uint16)
    monkeypatch.setenv("GEMM_BF16_SKINNY_COLS", "64")
    monkeypatch.setenv("GEMM_BF16_SKINNY_SPLITS", "8")
    runs = [run_gpu(M, N, K, case["A"], K, case["B"], K, C_init, M, 1.0, 0.0, None, "none") for _ in range(4)]
    for r in runs[1:]:
        assert np.array_equal(runs[0], r)
    monkeypatch.setenv("GEMM_BF16_SKINNY_SPLITS", "1")
    single = run_gpu(M, N, K, case["A"], K, case["B"], K, C_init, M, 1.0, 0.0, None, "none")
    assert_within_tolerance(runs[0], single, K, "split vs unsplit")
    ref = oracle.gemm(M, N, K, case["A"], K, case["B"], K, nthreads=_threads())
    assert_within_tolerance(runs[0], ref, K, "split vs oracle")


# Split K within one XCD: when a strip's splits share an XCD (the strips a
# multiple of 8, one workgroup per unit) the partials are plain stores read
# back through that XCD's L2; otherwise (GEMM_BF16_SKINNY_COLOCATE=0) they
# cross XCDs as device-wide atomics.  (The two place strips differently, so
# each unit walks its K range from a different rotated start: their sums
# round differently and both are checked against the oracle.)  Three
# colocated calls in a row must agree bit for bit -- the handoff records
# return to zero after every call -- and so must a call that takes the
# handoff's fallback, the agent-scope release/acquire fences, although the
# placement check passes (GEMM_BF16_SKINNY_COLOCATE=fence).
@pytest.mark.parametrize("M,N,K,ldc,cols", [
    (64, 2048, 4096, 64, "32"),    # 64 strips of 32 columns, 4 splits
    (64, 4096, 8192, 64, "64"),    # 64 strips of 64 columns, 4 splits (the default there)
    (40, 1000, 4096, 41, "32"),    # N tail, odd ldc, 32 strips, 4 splits
    (17, 2048, 8192, 17, "32"),    # 32-row block, 64 strips, 4 splits
    (64, 512, 16384, 64, "32"),    # 16 strips, 8 splits
])
def test_skinny_colocated_and_crossing_splits(M, N, K, ldc, cols, monkeypatch):
    case = inputs.random_case(M + N + K, M, N, K, ldc=ldc, with_c0=True, with_bias=True)
    monkeypatch.setenv("GEMM_BF16_SKINNY_COLS", cols)
    assert gb.gemm_bf16_kernel_name(M, N, K, 4096, K, 4096, K, 4096, ldc) == SK
    say(f"[skinny-colocated] {M}x{N}x{K} ldc={ldc} cols={cols}")
    run = lambda: run_gpu(M, N, K, case["A"], K, case["B"], K, case["C0"], ldc, 1.25, -0.5, case["bias"], "relu")
    coloc = [run() for _ in range(3)]
    for r in coloc[1:]:
        assert np.array_equal(coloc[0], r), "colocated skinny split varies between calls"
    monkeypatch.setenv("GEMM_BF16_SKINNY_COLOCATE", "fence")
    assert np.array_equal(coloc[0], run()), "the fenced handoff differs from the L2 handoff"
    monkeypatch.setenv("GEMM_BF16_SKINNY_COLOCATE", "0")
    cross = run()
    ref = oracle.gemm(M, N, K, case["A"], K, case["B"], K, case["C0"], ldc, 1.25, -0.5, case["bias"], "relu",
                      nthreads=_threads())
    r2 = ref.reshape(N, ldc)
    for tag, got in (("colocated", coloc[0]), ("crossing", cross)):
        g2 = got.reshape(N, ldc)
        assert_within_tolerance(g2[:, :M], r2[:, :M], K, f"{tag} skinny split vs oracle")
        assert np.array_equal(g2[:, M:], case["C0"].reshape(N, ldc)[:, M:]), f"{tag}: padding rows of C written"


@pytest.mark.parametrize("M,N,K,ldq", [(40, 512, 4096, 48), (64, 1024, 8192, 64)])
def test_skinny_colocated_split_int8_output(M, N, K, ldq):
    """The int8-output instance takes the same colocated handoff (16 or 32
    strips of 32 columns, 4 splits)."""
    check_q8(f"q8 skinny colocated {M}x{N}x{K}", M, N, K, ldq=ldq, alpha=1.25, beta=0.5, use_bias=True,
             epilogue="gelu_tanh", zp=2, seed=M + N, expect_kernel=SQ8K)


@pytest.mark.parametrize("M,N,K", [(16, 2048, 8192), (40, 1024, 16384)])
def test_skinny_colocated_split_fp8(M, N, K):
    """The FP8 instance takes the same colocated handoff (64 or 32 strips,
    4 splits of 512-value slices)."""
    check_fp8(f"fp8 skinny colocated {M}x{N}x{K}", M, N, K, beta=-0.25, use_bias=True, epilogue="relu",
              seed=M + K, expect_kernel=SKF)


# At most 64 columns (and more than 64 rows): the streaming kernel runs on
# the transposed product C^T = B^T A^T, whose rows are C's columns, and
# writes each 8-wide chunk of a row of C^T as 8 consecutive rows of one
# column of C.  The bias belongs to C's columns, i.e. to the rows of C^T.
SKT = "skinny_t"


@pytest.mark.parametrize("M,N,K,lda,ldb,ldc", [
    (8192, 64, 1024, 1024, 1024, 8192),  # 64 columns: 256 strips of 32 rows of C
    (4096, 1, 2048, 2048, 2048, 4096),   # a single column
    (1000, 17, 3000, 3000, 3000, 1001),  # M tail inside a chunk, odd ldc: element-wise stores
    (777, 33, 1032, 1040, 1032, 784),    # 33 columns: the 64-row block; padded A
    (130, 5, 520, 528, 536, 131),        # a few strips, padded A and B
    (65, 64, 1024, 1024, 1024, 72),      # one row past the streaming kernel's own limit
    (2048, 32, 16384, 16384, 16384, 2048),  # long K: split within an XCD
])
def test_skinny_transposed_shapes(M, N, K, lda, ldb, ldc):
    check_full(f"skinny_t {M}x{N}x{K}", M, N, K, lda=lda, ldb=ldb, ldc=ldc, beta=0.0, seed=M + 3 * N + K,
               expect_kernel=SKT, poison_pad=True)


@pytest.mark.parametrize("beta,use_bias,epi", [(0.5, True, "gelu_tanh"), (0.0, True, "none"),
                                               (-1.0, False, "gelu_tanh"), (0.25, True, "relu")])
@pytest.mark.parametrize("splits", ["1", "4"])
def test_skinny_transposed_epilogues(beta, use_bias, epi, splits, monkeypatch):
    monkeypatch.setenv("GEMM_BF16_SKINNY_SPLITS", splits)
    check_full(f"skinny_t epilogue beta={beta} bias={use_bias} {epi}", 3000, 48, 2048, ldc=3000, alpha=0.5,
               beta=beta, use_bias=use_bias, epilogue=epi, seed=43, expect_kernel=SKT)
    check_full("skinny_t unaligned C", 999, 40, 1024, ldc=1003, alpha=1.5, beta=beta, use_bias=use_bias,
               epilogue=epi, offsets=(0, 0, 3), seed=44, expect_kernel=SKT)


@pytest.mark.parametrize("cols", ["32", "64", "128"])
@pytest.mark.parametrize("splits", ["1", "3", "7"])
def test_skinny_transposed_widths_and_splits(cols, splits, monkeypatch):
    monkeypatch.setenv("GEMM_BF16_SKINNY_COLS", cols)
    monkeypatch.setenv("GEMM_BF16_SKINNY_SPLITS", splits)
    check_full(f"skinny_t cols={cols} splits={splits}", 1024, 64, 4096, beta=0.5, use_bias=True,
               epilogue="gelu_tanh", seed=5 * int(cols) + int(splits), expect_kernel=SKT)
    check_full(f"skinny_t N=20 cols={cols} splits={splits}", 520, 20, 2048, ldc=528,
               seed=7 * int(cols) + int(splits), expect_kernel=SKT)


@pytest.mark.parametrize("M,N,K,cols", [(2048, 64, 8192, "32"), (4096, 64, 8192, "64"), (1000, 40, 4096, "32")])
def test_skinny_transposed_equals_the_direct_kernel_on_swapped_operands(M, N, K, cols, monkeypatch):
    """C^T = B^T A^T: the direct streaming kernel on the swapped operands
    (N x M x K, A' = B read row-major, B' = A read column-major) computes
    the same sums in the same order, so without bias the two outputs are
    bit-identical transposes (colocated split, fenced handoff and crossing
    split alike); both also match the oracle."""
    monkeypatch.setenv("GEMM_BF16_SKINNY_COLS", cols)
    case = inputs.random_case(M + N + K, M, N, K, with_c0=True)
    assert gb.gemm_bf16_kernel_name(M, N, K, 4096, K, 4096, K, 4096, M) == SKT
    assert gb.gemm_bf16_kernel_name(N, M, K, 4096, K, 4096, K, 4096, N) == SK
    say(f"[skinny_t] {M}x{N}x{K} cols={cols} vs direct {N}x{M}x{K}")
    trans = [run_gpu(M, N, K, case["A"], K, case["B"], K, case["C0"], M, 1.25, -0.5, None, "relu")
             for _ in range(2)]
    assert np.array_equal(trans[0], trans[1]), "transposed skinny varies between calls"
    C0_t = np.ascontiguousarray(case["C0"].reshape(N, M).T).reshape(-1)
    direct = run_gpu(N, M, K, case["B"], K, case["A"], K, C0_t, N, 1.25, -0.5, None, "relu")
    assert np.array_equal(trans[0].reshape(N, M), direct.reshape(M, N).T), "transposed != direct kernel"
    for mode in ("fence", "0"):
        monkeypatch.setenv("GEMM_BF16_SKINNY_COLOCATE", mode)
        other = run_gpu(M, N, K, case["A"], K, case["B"], K, case["C0"], M, 1.25, -0.5, None, "relu")
        if mode == "fence":
            assert np.array_equal(trans[0], other), "the fenced handoff differs from the L2 handoff"
        ref = oracle.gemm(M, N, K, case["A"], K, case["B"], K, case["C0"], M, 1.25, -0.5, None, "relu",
                          nthreads=_threads())
        assert_within_tolerance(other, ref, K, f"skinny_t colocate={mode} vs oracle")
    ref = oracle.gemm(M, N, K, case["A"], K, case["B"], K, case["C0"], M, 1.25, -0.5, None, "relu",
                      nthreads=_threads())
    assert_within_tolerance(trans[0], ref, K, "skinny_t vs oracle")


@pytest.mark.parametrize("M,N,K,ldq,q_offset", [
    (8192, 64, 2048, 8192, 0),     # 64 columns: 256 strips of 32 rows of Q, 8-byte stores
    (1000, 17, 3000, 1001, 0),     # row tail inside a chunk, odd ldq: element-wise stores
    (4096, 1, 2048, 4096, 0),      # a single column
    (999, 40, 1024, 1000, 1),      # Q not 8-byte aligned
    (2048, 32, 16384, 2048, 0),    # long K: split within an XCD
])
def test_skinny_transposed_int8_output(M, N, K, ldq, q_offset):
    """The int8-output instance on the transposed product: the scale of C's
    row m quantizes column m of C^T, and Q is written back transposed."""
    check_q8(f"q8 skinny_t {M}x{N}x{K}", M, N, K, ldq=ldq, ldc=ldq, alpha=1.25, beta=0.5, use_bias=True,
             epilogue="gelu_tanh", zp=3, q_offset=q_offset, seed=M + 2 * N + K, expect_kernel="skinny_q8_t")
    check_q8(f"q8 skinny_t beta=0 {M}x{N}x{K}", M, N, K, ldq=ldq, epilogue="relu", zp=-7, q_offset=q_offset,
             seed=M + 3 * N + K, expect_kernel="skinny_q8_t")


@pytest.mark.parametrize("M,N,K,ldc,scales", [
    (8192, 64, 1024, 8192, True),   # 64 columns: 256 strips
    (1000, 17, 3008, 1001, True),   # row tail, odd ldc
    (4096, 1, 2048, 4096, True),    # a single column
    (2048, 32, 16384, 2048, True),  # long K: split within an XCD
    (777, 33, 1024, 784, False),    # no scales
])
def test_skinny_transposed_fp8(M, N, K, ldc, scales):
    """The FP8 instance on the transposed product: the row and column scales
    trade places with the operands."""
    check_fp8(f"fp8 skinny_t {M}x{N}x{K}", M, N, K, ldc=ldc, alpha=0.75, beta=-0.25, use_bias=True,
              epilogue="relu", scales=scales, seed=M + N + K, expect_kernel="skinny_fp8_t")


@pytest.mark.parametrize("M,N,K,ldc", [(40, 10000, 512, 41), (9000, 24, 1024, 9000)])
def test_many_strips_over_a_short_k_take_the_masked_tiles(M, N, K, ldc):
    """More 32-wide strips than compute units over a short K: the masked
    128x128 tiles, their rows (or columns) mostly past the matrix."""
    check_full(f"many strips short K {M}x{N}x{K}", M, N, K, ldc=ldc, beta=0.5, use_bias=True,
               epilogue="gelu_tanh", seed=M + N + K, expect_kernel="tile128x128x64_s4_masked")


@pytest.mark.parametrize("M,N,K,ldc", [(40, 20000, 1024, 41), (20000, 24, 512, 20000)])
def test_fp8_many_strips_over_a_short_k_take_the_masked_tiles(M, N, K, ldc):
    check_fp8(f"fp8 many strips short K {M}x{N}x{K}", M, N, K, ldc=ldc, beta=0.5, use_bias=True,
              epilogue="gelu_tanh", seed=M + N + K, expect_kernel="fp8_128x128x128_masked")


# ---------------------------------------------------- bounds-checked path ---

@pytest.mark.parametrize("M,N,K", [
    (1, 1, 1), (33, 65, 97), (257, 257, 257), (1000, 1000, 1000), (64, 64, 4097), (1, 4096, 512),
    (300, 1, 70), (130, 70, 8),
])
def test_generic_ragged_full(M, N, K, monkeypatch):
    # forced: some of these shapes have a fast path (1 x 4096 x 512 streams)
    monkeypatch.setenv("GEMM_BF16_FORCE_KERNEL", "generic64x64x32")
    check_full(f"generic {M}x{N}x{K}", M, N, K, seed=3 * M + N + K, expect_kernel="generic64x64x32")


def test_generic_unaligned_and_odd_leading_dims():
    check_full("unaligned A", 256, 256, 256, offsets=(1, 0, 0), seed=21, expect_kernel="generic64x64x32")
    check_full("unaligned B C", 128, 192, 64, offsets=(0, 3, 5), beta=0.5, use_bias=True, seed=22,
               expect_kernel="generic64x64x32")
    check_full("odd lds", 100, 90, 77, lda=81, ldb=79, ldc=103, beta=2.0, use_bias=True,
               epilogue="gelu_tanh", seed=23, expect_kernel="generic64x64x32")
    check_full("odd lds relu", 100, 90, 77, lda=81, ldb=79, ldc=103, beta=-0.5, use_bias=True,
               epilogue="relu", seed=26, expect_kernel="generic64x64x32")


def test_k_zero_is_epilogue_only():
    check_full("K=0 beta bias gelu", 200, 150, 0, beta=0.5, use_bias=True, epilogue="gelu_tanh", seed=24,
               expect_kernel="generic64x64x32")
    check_full("K=0 beta=0", 64, 64, 0, seed=25, expect_kernel="generic64x64x32")


def test_empty_output_touches_nothing():
    c_t, c_p = to_dev(np.full(16, NAN_BF16, np.uint16))
    st = gb.gemm_bf16(0, 4, 4, 0, 4, c_p, 4, c_p, 1, 1.0, 0.0, 0, 0, torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    assert np.all(from_dev(c_t, 0, 16) == NAN_BF16)


def test_repeat_launches_bit_identical_and_paths_agree():
    """Repeated launches of the tile kernel are bit-identical (no race in the
    LDS ring), and the bounds-checked kernel forced on the same inputs agrees
    with it within the tolerance."""
    M, N, K = 512, 512, 512
    case = inputs.random_case(31, M, N, K)
    C_init = np.zeros(M * N, np.uint16)
    r1 = run_gpu(M, N, K, case["A"], K, case["B"], K, C_init, M, 1.0, 0.0, None, "none")
    r2 = run_gpu(M, N, K, case["A"], K, case["B"], K, C_init, M, 1.0, 0.0, None, "none")
    assert np.array_equal(r1, r2)
    os.environ["GEMM_BF16_FORCE_KERNEL"] = "generic64x64x32"
    try:
        assert gb.gemm_bf16_kernel_name(M, N, K, 4096, K, 4096, K, 4096, M) == "generic64x64x32"
        r3 = run_gpu(M, N, K, case["A"], K, case["B"], K, C_init, M, 1.0, 0.0, None, "none")
    finally:
        del os.environ["GEMM_BF16_FORCE_KERNEL"]
    assert_within_tolerance(r3, r1, K, "generic vs tile")


def test_kernels_with_one_accumulation_order_agree_bit_for_bit(monkeypatch):
    """Every kernel built on v_mfma_f32_32x32x16_bf16 that walks K in order
    gives each output element the same MFMAs on the same operands in the same
    order, whatever its tile, its ring (a five-slot unit ring, five and four
    stages, a plain double buffer) and its epilogue staging -- so their
    results must agree bit for bit.  A race in any of those pipelines would
    show up as a difference.  The epilogue is alpha * sum alone (one
    rounding), so the compiler's contraction of longer epilogues cannot make
    the kernels differ."""
    M, N, K = 1024, 512, 640
    case = inputs.random_case(32, M, N, K, with_c0=False, with_bias=False)
    C_init = np.full(N * M, NAN_BF16, np.uint16)
    outs = {}
    for kernel in ("ring256x256x64_mfma32", "tile256x256x32_s5", "tile128x128x64_s4", "generic64x64x32"):
        monkeypatch.setenv("GEMM_BF16_FORCE_KERNEL", kernel)
        assert gb.gemm_bf16_kernel_name(M, N, K, 4096, K, 4096, K, 4096, M) == kernel
        outs[kernel] = run_gpu(M, N, K, case["A"], K, case["B"], K, C_init, M, 1.25, 0.0, None, "none")
    ref = outs.pop("ring256x256x64_mfma32")
    for kernel, got in outs.items():
        assert np.array_equal(got, ref), f"{kernel} differs from ring256x256x64_mfma32"
    exp = oracle.gemm(M, N, K, case["A"], K, case["B"], K, None, M, 1.25, 0.0, None, "none", nthreads=_threads())
    assert_within_tolerance(ref, exp, K, "32x32x16 kernels vs oracle")


# ------------------------------------------------------- int8 output ---

def run_gpu_q8(M, N, K, A, lda, B, ldb, C0, ldc, Q_init, ldq, alpha, beta, bias, epilogue, scale, zp,
               q_offset=0):
    a_t, a_p = to_dev(A)
    b_t, b_p = to_dev(B)
    c_p = 0
    if beta != 0.0:
        c_t, c_p = to_dev(C0)
    q_t = torch.zeros(Q_init.size + q_offset + 16, dtype=torch.int8, device="cuda")
    q_t[q_offset:q_offset + Q_init.size] = torch.from_numpy(np.ascontiguousarray(Q_init)).cuda()
    s_t = torch.from_numpy(np.ascontiguousarray(scale, dtype=np.float32)).cuda()
    bias_p = 0
    if bias is not None:
        bias_t, bias_p = to_dev(bias)
    stream = torch.cuda.current_stream().cuda_stream
    st = gb.gemm_bf16_q8(M, N, K, a_p, lda, b_p, ldb, c_p, ldc, q_t.data_ptr() + q_offset, ldq, alpha, beta,
                         bias_p, EPI[epilogue], s_t.data_ptr(), zp, stream)
    assert st == 0, gb.gemm_bf16_status_string(st)
    torch.cuda.synchronize()
    return q_t[q_offset:q_offset + Q_init.size].cpu().numpy().copy()


def check_q8(tag, M, N, K, ldq=None, ldc=None, alpha=1.0, beta=0.0, use_bias=False, epilogue="none", zp=0,
             scale_range=(0.25, 0.75), q_offset=0, seed=0, expect_kernel=None):
    ldq = max(M, 1) if ldq is None else ldq
    ldc = max(M, 1) if ldc is None else ldc
    case = inputs.random_case(seed, M, N, K, ldc=ldc, with_c0=True, with_bias=use_bias)
    scale = inputs.uniform_f32(seed + 5, M, *scale_range)
    bias = case.get("bias") if use_bias else None
    Q_init = np.full(N * ldq, Q8_POISON, np.int8)
    kld = max(K, 1)
    kname = gb.gemm_bf16_q8_kernel_name(M, N, K, 4096, kld, 4096, kld, 4096 if beta != 0.0 else 0, ldc,
                                        4096 + q_offset, ldq, beta, 4096, EPI[epilogue])
    say(f"[parity-q8] {tag}: M={M} N={N} K={K} ldc={ldc} ldq={ldq} alpha={alpha} beta={beta} bias={use_bias} "
        f"epi={epilogue} zp={zp} scales={scale_range} q_offset={q_offset} kernel={kname}")
    if expect_kernel is not None:
        assert kname == expect_kernel
    got = run_gpu_q8(M, N, K, case["A"], kld, case["B"], kld, case["C0"], ldc, Q_init, ldq, alpha, beta, bias,
                     epilogue, scale, zp, q_offset)
    ref, t = oracle.gemm_q8(M, N, K, case["A"], kld, case["B"], kld, scale, zp, C_in=case["C0"], ldc=ldc, ldq=ldq,
                            alpha=alpha, beta=beta, bias=bias, epilogue=epilogue, nthreads=_threads())
    g2, r2 = got.reshape(N, ldq), ref.reshape(N, ldq)
    rep = assert_q8_within_tolerance(g2[:, :M], r2[:, :M], t, np.broadcast_to(scale[None, :], (N, M)), zp, K,
                                     tag)
    if ldq > M:
        assert np.all(g2[:, M:] == Q8_POISON), f"{tag}: padding rows written"
    say(f"[parity-q8] {tag}: ok exact={rep['exact']}/{rep['n']} near_boundary={rep['near_boundary']} "
        f"saturated={int(np.count_nonzero(np.abs(r2[:, :M].astype(np.int64) + 0.5) > 127))}")
    return rep


RQ8 = "ring256x256x64_q8"
RQ8M = "ring256x256x64_q8_masked"
SQ8 = "splitk128x128x64_q8"


# Small grids: split-K on 128x128 tiles, the reduction quantizing per row.
@pytest.mark.parametrize("M,N,K,ldq,beta,use_bias,epi,zp", [
    (1024, 512, 2048, 1024, 0.0, True, "relu", -20),   # 32 tiles, 4 ranges
    (256, 256, 4096, 264, 0.5, True, "gelu_tanh", 3),  # 4 tiles, 8 ranges, padded ldq, C0 read
    (512, 384, 1600, 520, -0.75, False, "none", 0),    # uneven ranges
])
def test_q8_splitk(M, N, K, ldq, beta, use_bias, epi, zp):
    check_q8(f"q8 splitk {M}x{N}x{K}", M, N, K, ldq=ldq, alpha=1.25, beta=beta, use_bias=use_bias, epilogue=epi,
             zp=zp, seed=M + N + K, expect_kernel=SQ8)


def test_q8_ring_is_the_default_for_large_shapes():
    check_q8("q8 ring default", 4096, 2048, 192, use_bias=True, epilogue="relu", zp=-20, seed=61,
             expect_kernel=RQ8)


# Grids too large to split but whose 128x128 tiles all fit the workspace:
# whole K through the split kernels with one range, the reduction running
# the epilogue and quantizing.
@pytest.mark.parametrize("M,N,K,ldq,beta,use_bias,epi,zp,kernel", [
    (2048, 1024, 1024, 2048, 0.5, True, "gelu_tanh", 3, "tile128x128x64_q8"),     # 128 tiles
    (2048, 2048, 512, 2056, 0.0, False, "relu", -9, "tile128x128x64_q8"),         # 256 tiles, padded ldq
    (1500, 1400, 1024, 1504, -0.75, True, "none", 0, "tile128x128x64_q8_masked"),  # tails in M and N
    (1504, 1504, 600, 1504, 0.5, True, "relu", 5, "tile128x128x64_q8_masked"),    # K tail
])
def test_q8_whole_k_tiles(M, N, K, ldq, beta, use_bias, epi, zp, kernel):
    check_q8(f"q8 whole-K tiles {M}x{N}x{K}", M, N, K, ldq=ldq, ldc=ldq, alpha=1.25, beta=beta, use_bias=use_bias,
             epilogue=epi, zp=zp, seed=M + N + K + 7, expect_kernel=kernel)


@pytest.mark.parametrize("M,N,K,ldq,kernel", [
    (2048, 2048, 256, 2048, RQ8),                # 64 ring tiles, 256 128x128 tiles: too many to split
    (1500, 1500, 320, 1504, RQ8M),               # 36 ring tiles, with tails
    (2048, 1024, 256, 2048, "generic64x64x32"),  # 32 ring tiles: the bounds-checked kernel is faster
])
def test_q8_mid_sized_grids(M, N, K, ldq, kernel):
    check_q8(f"q8 mid {M}x{N}x{K}", M, N, K, ldq=ldq, ldc=ldq, beta=0.5, use_bias=True, epilogue="gelu_tanh", zp=5,
             seed=M + N + K, expect_kernel=kernel)


SQ8M = "splitk128x128x64_q8_masked"


# Small grids with tails: split-K on the masked 128x128 tiles, the reduction
# quantizing 8-row chunks (element by element where a chunk straddles M).
@pytest.mark.parametrize("M,N,K,ldq,beta,use_bias,epi,zp", [
    (1000, 1000, 4096, 1000, 0.5, True, "relu", -7),      # 64 tiles, 3 ranges
    (1001, 777, 2048, 1008, 0.0, True, "gelu_tanh", 3),    # M % 8 == 1: the last chunk straddles M
    (1000, 1000, 1000, 1000, -0.75, False, "none", 0),     # 16 slices in 2 ranges
])
def test_q8_masked_splitk(M, N, K, ldq, beta, use_bias, epi, zp):
    check_q8(f"q8 masked splitk {M}x{N}x{K}", M, N, K, ldq=ldq, ldc=ldq, alpha=1.25, beta=beta,
             use_bias=use_bias, epilogue=epi, zp=zp, seed=M + N + K, expect_kernel=SQ8M)


@pytest.mark.parametrize("M,N,K,ldq", [
    (1001, 777, 200, 1008), (257, 513, 8, 264), (1, 255, 64, 8), (300, 260, 72, 304), (512, 512, 256, 512),
])
def test_q8_ring_tails(M, N, K, ldq, monkeypatch):
    monkeypatch.setenv("GEMM_BF16_FORCE_KERNEL", RQ8M)
    check_q8(f"q8 ring {M}x{N}x{K}", M, N, K, ldq=ldq, zp=3, seed=M + N, expect_kernel=RQ8M)


@pytest.mark.parametrize("beta,use_bias,epi", [(b, u, e) for b in (0.0, -0.75) for u in (False, True)
                                               for e in ("none", "gelu_tanh", "relu")])
def test_q8_ring_epilogue_combinations(beta, use_bias, epi, monkeypatch):
    monkeypatch.setenv("GEMM_BF16_FORCE_KERNEL", RQ8M)
    check_q8(f"q8 ring beta={beta} bias={use_bias} {epi}", 777, 300, 200, ldq=784, ldc=792, alpha=1.25, beta=beta,
             use_bias=use_bias, epilogue=epi, zp=-5, seed=70 + int(abs(beta) * 4) + 2 * use_bias + len(epi),
             expect_kernel=RQ8M)


# The unmasked int8 instance (exact tile multiples): every epilogue
# combination, padded leading dimensions, several tiles per compute unit.
@pytest.mark.parametrize("beta,use_bias,epi", [(b, u, e) for b in (0.0, -0.75) for u in (False, True)
                                               for e in ("none", "gelu_tanh", "relu")])
def test_q8_exact_ring_epilogue_combinations(beta, use_bias, epi, monkeypatch):
    monkeypatch.setenv("GEMM_BF16_FORCE_KERNEL", RQ8)
    check_q8(f"q8 exact ring beta={beta} bias={use_bias} {epi}", 768, 512, 320, ldq=776, ldc=784, alpha=0.75,
             beta=beta, use_bias=use_bias, epilogue=epi, zp=4,
             seed=170 + int(abs(beta) * 4) + 2 * use_bias + len(epi), expect_kernel=RQ8)


def test_q8_exact_ring_many_tiles():
    check_q8("q8 exact ring 4608x2048", 4608, 2048, 256, beta=0.5, use_bias=True, epilogue="gelu_tanh", zp=-3,
             seed=190, expect_kernel=RQ8)


def test_q8_saturation_both_paths(monkeypatch):
    # scales of 4..8 on values of std ~16: most codes saturate at -128 / 127
    check_q8("q8 saturating generic", 200, 150, 256, scale_range=(4.0, 8.0), zp=7, seed=81,
             expect_kernel="generic64x64x32")
    monkeypatch.setenv("GEMM_BF16_FORCE_KERNEL", RQ8)
    check_q8("q8 saturating ring", 512, 256, 256, scale_range=(4.0, 8.0), zp=7, seed=82, expect_kernel=RQ8)


# Int8 output on the streaming kernel (1 to 64 rows): row tails inside the
# 32- and 64-row blocks, K tails, padded and unaligned Q (element-wise
# stores), the split-K path (few strips), every epilogue combination.
SQ8K = "skinny_q8"


@pytest.mark.parametrize("M,N,K,ldq,ldc,q_offset", [
    (1, 4096, 4096, 1, 1, 0),        # decode
    (3, 1000, 520, 3, 3, 0),         # a K tail inside the last slice
    (17, 777, 1032, 24, 17, 0),      # padded ldq
    (32, 2048, 2048, 32, 32, 0),     # a full 32-row block
    (33, 515, 264, 40, 40, 3),       # 64-row block, unaligned Q
    (64, 8192, 2048, 64, 64, 0),     # 256 strips, no split
    (64, 256, 8192, 64, 64, 0),      # 8 strips: split K
])
def test_q8_skinny_shapes(M, N, K, ldq, ldc, q_offset):
    check_q8(f"q8 skinny {M}x{N}x{K}", M, N, K, ldq=ldq, ldc=ldc, use_bias=True, epilogue="relu", zp=-7,
             q_offset=q_offset, seed=200 + M + K, expect_kernel=SQ8K)


@pytest.mark.parametrize("beta,use_bias,epi", [(b, u, e) for b in (0.0, -0.75) for u in (False, True)
                                               for e in ("none", "gelu_tanh", "relu")])
def test_q8_skinny_epilogue_combinations(beta, use_bias, epi):
    check_q8(f"q8 skinny beta={beta} bias={use_bias} {epi}", 48, 640, 768, ldq=56, ldc=52, alpha=1.25, beta=beta,
             use_bias=use_bias, epilogue=epi, zp=3, seed=220 + int(abs(beta) * 4) + 2 * use_bias + len(epi),
             expect_kernel=SQ8K)


@pytest.mark.parametrize("splits", ["2", "3", "7"])
def test_q8_skinny_forced_splits(splits, monkeypatch):
    monkeypatch.setenv("GEMM_BF16_SKINNY_SPLITS", splits)
    check_q8(f"q8 skinny {splits} splits", 40, 512, 4096, beta=0.5, use_bias=True, epilogue="gelu_tanh", zp=1,
             seed=240 + int(splits), expect_kernel=SQ8K)


def test_q8_generic_paths():
    check_q8("q8 generic odd ldq", 100, 90, 77, ldq=103, beta=0.5, use_bias=True, epilogue="gelu_tanh", seed=83,
             expect_kernel="generic64x64x32")
    check_q8("q8 generic unaligned Q", 4096, 512, 64, q_offset=3, zp=-1, seed=84, expect_kernel="generic64x64x32")
    check_q8("q8 K=0", 70, 50, 0, beta=2.0, use_bias=True, epilogue="relu", zp=1, seed=85,
             expect_kernel="generic64x64x32")


# ----------------------------------------------------------- fp8 inputs ---

FP8R = "fp8_256x256x128"


def to_dev_u8(bits: np.ndarray, offset: int = 0):
    full = torch.zeros(bits.size + offset + 16, dtype=torch.uint8, device="cuda")
    full[offset:offset + bits.size] = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint8)).cuda()
    return full, full.data_ptr() + offset


FP8_NAN = 0x7F  # E4M3: S.1111.111


def check_fp8(tag, M, N, K, lda=None, ldb=None, ldc=None, alpha=1.0, beta=0.0, use_bias=False,
              epilogue="none", scales=True, offsets=(0, 0, 0), seed=0, expect_kernel=None, poison_pad=False):
    lda = max(K, 1) if lda is None else lda
    ldb = max(K, 1) if ldb is None else ldb
    ldc = max(M, 1) if ldc is None else ldc
    A = inputs.normal_fp8(seed + 1, M * lda)
    B = inputs.normal_fp8(seed + 2, N * ldb)
    if poison_pad:
        # operand padding (k >= K) is NaN: a kernel that reads it produces NaN
        for X, ld, rows in ((A, lda, M), (B, ldb, N)):
            if ld > K:
                X.reshape(rows, ld)[:, K:] = FP8_NAN
    C0 = inputs.normal_bf16(seed + 3, N * ldc)
    bias = inputs.normal_bf16(seed + 4, N, scale=0.1) if use_bias else None
    sa = inputs.uniform_f32(seed + 6, M, 0.5, 2.0) if scales else None
    sb = inputs.uniform_f32(seed + 7, N, 0.5, 2.0) if scales else None
    C_init = C0 if beta != 0.0 else np.full_like(C0, NAN_BF16)
    kname = gb.gemm_fp8_kernel_name(M, N, K, 4096 + offsets[0], lda, 4096 + offsets[1], ldb,
                                    4096 + 2 * offsets[2], ldc, EPI[epilogue])
    say(f"[parity-fp8] {tag}: M={M} N={N} K={K} lda={lda} ldb={ldb} ldc={ldc} alpha={alpha} beta={beta} "
        f"bias={use_bias} epi={epilogue} scales={scales} offsets={offsets} kernel={kname}")
    if expect_kernel is not None:
        assert kname == expect_kernel
    a_t, a_p = to_dev_u8(A, offsets[0])
    b_t, b_p = to_dev_u8(B, offsets[1])
    c_t, c_p = to_dev(C_init, offsets[2])
    bias_p = 0
    if bias is not None:
        bias_t, bias_p = to_dev(bias)
    sa_t = torch.from_numpy(sa).cuda() if scales else None
    sb_t = torch.from_numpy(sb).cuda() if scales else None
    st = gb.gemm_fp8(M, N, K, a_p, lda, b_p, ldb, c_p, ldc, alpha, beta, sa_t.data_ptr() if scales else 0,
                     sb_t.data_ptr() if scales else 0, bias_p, EPI[epilogue], torch.cuda.current_stream().cuda_stream)
    assert st == 0, gb.gemm_bf16_status_string(st)
    torch.cuda.synchronize()
    got = from_dev(c_t, offsets[2], C_init.size)
    ref = oracle.gemm_fp8(M, N, K, A, lda, B, ldb, C0, ldc, alpha, beta, sa, sb, bias, epilogue,
                          nthreads=_threads())
    g2, r2 = got.reshape(N, ldc), ref.reshape(N, ldc)
    rep = assert_within_tolerance(g2[:, :M], r2[:, :M], K, tag)
    if ldc > M:
        assert np.array_equal(g2[:, M:], C_init.reshape(N, ldc)[:, M:]), f"{tag}: padding written"
    say(f"[parity-fp8] {tag}: ok max_err/tol={rep['max_err_over_tol']:.3f} mean_err/tol={rep['mean_err_over_tol']:.4f} "
        f"exact={rep['exact']}/{rep['n']}")
    return rep


@pytest.mark.parametrize("M,N,K", [(512, 512, 128), (512, 256, 256), (1024, 512, 640), (4096, 2048, 1280)])
def test_fp8_ring_slice_counts(M, N, K, monkeypatch):
    monkeypatch.setenv("GEMM_BF16_FORCE_KERNEL", FP8R)  # small grids default to the 128x128 tiles
    check_fp8(f"fp8 ring {M}x{N}x{K}", M, N, K, seed=M + N + K, expect_kernel=FP8R)


@pytest.mark.parametrize("beta,use_bias,epi,scales", [(b, u, e, sc) for b in (0.0, -0.75) for u in (False, True)
                                                      for e in ("none", "gelu_tanh", "relu") for sc in (True, False)
                                                      if not (u and not sc and e == "relu")])
def test_fp8_ring_epilogue_combinations(beta, use_bias, epi, scales, monkeypatch):
    monkeypatch.setenv("GEMM_BF16_FORCE_KERNEL", FP8R)
    check_fp8(f"fp8 ring beta={beta} bias={use_bias} {epi} scales={scales}", 1024, 512, 384, alpha=1.25,
              beta=beta, use_bias=use_bias, epilogue=epi, scales=scales,
              seed=int(abs(beta) * 4) + 2 * use_bias + len(epi) + 7 * scales, expect_kernel=FP8R)


def test_fp8_ring_padded_leading_dims(monkeypatch):
    monkeypatch.setenv("GEMM_BF16_FORCE_KERNEL", FP8R)
    check_fp8("fp8 ring padded", 512, 768, 512, lda=528, ldb=640, ldc=520, beta=0.5, use_bias=True, seed=95,
              expect_kernel=FP8R)


@pytest.mark.parametrize("M,N,K,ldc", [(3, 8192, 8192, 3), (4, 16384, 4096, 8)])
def test_fp8_three_and_four_rows_on_large_b_take_the_streaming_kernel(M, N, K, ldc):
    check_fp8(f"fp8 rows {M} large B", M, N, K, ldc=ldc, beta=0.5, use_bias=True, epilogue="gelu_tanh",
              seed=M * 11 + 5, expect_kernel="skinny_fp8")


# Split-K on the 256x256 FP8 tiles (forced: on small grids the 128x128 tiles
# are the default): ranges of unequal length, the scales applied by the
# reduction, every epilogue combination, forced range counts, run-to-run
# bit equality.
FP8S = "splitk_fp8_256x256x128"


@pytest.fixture
def force_fp8_split256(monkeypatch):
    monkeypatch.setenv("GEMM_BF16_FORCE_KERNEL", FP8S)


@pytest.mark.parametrize("M,N,K", [
    (1024, 1024, 4096),   # 16 tiles, 32 slices: 4 ranges
    (512, 512, 8192),     # 4 tiles, 64 slices: 8 ranges
    (256, 768, 1664),     # 3 tiles, 13 slices: ranges of 5, 5, 3
    (512, 256, 2048),     # 2 tiles, 16 slices: 4 ranges
])
def test_fp8_splitk_shapes(M, N, K, force_fp8_split256):
    check_fp8(f"fp8 splitk {M}x{N}x{K}", M, N, K, beta=0.5, use_bias=True, epilogue="gelu_tanh",
              seed=M + 2 * N + K, expect_kernel=FP8S)


@pytest.mark.parametrize("beta,use_bias,epi,scales", [(b, u, e, sc) for b in (0.0, -0.75) for u in (False, True)
                                                      for e in ("none", "gelu_tanh", "relu") for sc in (True, False)
                                                      if not (u and not sc and e == "relu")])
def test_fp8_splitk_epilogue_combinations(beta, use_bias, epi, scales, force_fp8_split256):
    check_fp8(f"fp8 splitk beta={beta} bias={use_bias} {epi} scales={scales}", 512, 256, 2048, alpha=1.25,
              beta=beta, use_bias=use_bias, epilogue=epi, scales=scales,
              seed=100 + int(abs(beta) * 4) + 2 * use_bias + len(epi) + 7 * scales, expect_kernel=FP8S)


def test_fp8_splitk_padded_leading_dims(force_fp8_split256):
    check_fp8("fp8 splitk padded", 512, 512, 2048, lda=2064, ldb=2080, ldc=520, beta=0.5, use_bias=True,
              seed=131, expect_kernel=FP8S)


@pytest.mark.parametrize("splits", ["2", "3", "5"])
def test_fp8_splitk_forced_range_counts(splits, monkeypatch, force_fp8_split256):
    monkeypatch.setenv("GEMM_BF16_FP8_SPLITS", splits)
    check_fp8(f"fp8 splitk {splits} ranges", 256, 512, 2560, beta=0.25, use_bias=True, seed=140 + int(splits),
              expect_kernel=FP8S)


@pytest.mark.parametrize("kernel", [FP8S, "splitk_fp8_128x128x128"])
def test_fp8_splitk_deterministic(kernel, monkeypatch):
    monkeypatch.setenv("GEMM_BF16_FORCE_KERNEL", kernel)
    M, N, K = 512, 512, 4096
    A, B = inputs.normal_fp8(150, M * K), inputs.normal_fp8(151, N * K)
    a_t, a_p = to_dev_u8(A)
    b_t, b_p = to_dev_u8(B)
    assert gb.gemm_fp8_kernel_name(M, N, K, a_p, K, b_p, K, a_p, M) == kernel
    outs = []
    for _ in range(3):
        c = torch.full((M * N,), -1, dtype=torch.int16, device="cuda")
        st = gb.gemm_fp8(M, N, K, a_p, K, b_p, K, c.data_ptr(), M, 1.0, 0.0, 0, 0, 0, 0,
                         torch.cuda.current_stream().cuda_stream)
        assert st == 0
        torch.cuda.synchronize()
        outs.append(c.cpu().numpy())
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2]), "fp8 split-K results vary"


# FP8 on the 128x128 tiles (32x32x64 MFMAs, K-slices of 128 values, the
# bf16 128x128 kernel's rows and ring): whole K over 1 to 10 slices, split-K
# (ranges of unequal length, the reduction applying the scales), tails of
# every kind with NaN operand padding, every epilogue combination with
# scales on and off.
F8T128 = "fp8_128x128x128"
F8T128M = "fp8_128x128x128_masked"
F8T128S = "splitk_fp8_128x128x128"
F8T128SM = "splitk_fp8_128x128x128_masked"


@pytest.mark.parametrize("M,N,K", [(128, 128, 128), (256, 128, 256), (512, 384, 384), (384, 512, 512),
                                   (1024, 512, 640), (256, 768, 1152), (2048, 2048, 1280), (4096, 2048, 768)])
def test_fp8_medium_slice_counts(M, N, K, monkeypatch):
    monkeypatch.setenv("GEMM_BF16_FORCE_KERNEL", F8T128)
    check_fp8(f"fp8 128x128 {M}x{N}x{K}", M, N, K, seed=M + N + K + 600, expect_kernel=F8T128)


@pytest.mark.parametrize("beta,use_bias,epi,scales", [(b, u, e, sc) for b in (0.0, -0.75) for u in (False, True)
                                                      for e in ("none", "gelu_tanh", "relu") for sc in (True, False)
                                                      if not (u and not sc and e == "relu")])
@pytest.mark.parametrize("kernel", [F8T128, F8T128S])
def test_fp8_medium_epilogue_combinations(kernel, beta, use_bias, epi, scales, monkeypatch):
    monkeypatch.setenv("GEMM_BF16_FORCE_KERNEL", kernel)
    K = 384 if kernel == F8T128 else 2048
    check_fp8(f"{kernel} beta={beta} bias={use_bias} {epi} scales={scales}", 512, 384, K, alpha=1.25,
              beta=beta, use_bias=use_bias, epilogue=epi, scales=scales,
              seed=610 + int(abs(beta) * 4) + 2 * use_bias + len(epi) + 7 * scales, expect_kernel=kernel)


@pytest.mark.parametrize("M,N,K", [
    (1024, 1024, 4096),  # 64 tiles, 32 slices: 4 ranges
    (512, 512, 8192),    # 16 tiles, 64 slices: 8 ranges of 8
    (256, 384, 2048),    # 6 tiles, 16 slices: 2 ranges
    (128, 128, 16384),   # 1 tile, 128 slices: 16 ranges
    (384, 256, 3200),    # 6 tiles, 25 slices: 3 ranges of 9, 9, 7
])
def test_fp8_medium_splitk_shapes(M, N, K, monkeypatch):
    monkeypatch.setenv("GEMM_BF16_FORCE_KERNEL", F8T128S)
    check_fp8(f"fp8 128x128 splitk {M}x{N}x{K}", M, N, K, beta=0.5, use_bias=True, epilogue="gelu_tanh",
              seed=M + 2 * N + K + 620, expect_kernel=F8T128S)


@pytest.mark.parametrize("splits", ["2", "3", "5"])
def test_fp8_medium_splitk_forced_range_counts(splits, monkeypatch):
    monkeypatch.setenv("GEMM_BF16_FORCE_KERNEL", F8T128S)
    monkeypatch.setenv("GEMM_BF16_SPLITK_SPLITS", splits)
    check_fp8(f"fp8 128x128 splitk {splits} ranges", 256, 384, 5120, beta=0.25, use_bias=True,
              seed=630 + int(splits), expect_kernel=F8T128S)


# The masked kernels load the last K-slice through a peeled iteration: walk
# the slice count through 1 .. 7 with a K tail in the last slice, on both
# masked FP8 tile kernels (the bf16 ones are walked by the forced-kernel
# slice counts above).
@pytest.mark.parametrize("kernel", ["fp8_256x256x128_masked", "fp8_256x256x128_mfma16_masked", F8T128M])
@pytest.mark.parametrize("nk", [1, 2, 3, 4, 5, 7])
def test_fp8_masked_slice_counts_with_k_tail(kernel, nk, monkeypatch):
    monkeypatch.setenv("GEMM_BF16_FORCE_KERNEL", kernel)
    K = 128 * nk - 48
    check_fp8(f"{kernel} nk={nk}", 520, 264, K, lda=K + 16, ldb=K + 32, ldc=528, beta=0.5, use_bias=True,
              seed=700 + nk, expect_kernel=kernel, poison_pad=True)


@pytest.mark.parametrize("M,N,K,lda,ldb,ldc,kernel", [
    (1000, 1000, 1008, 1008, 1024, 1000, F8T128M),   # M, N tails; K tail of 112 in the last slice
    (130, 70, 528, 544, 528, 136, F8T128M),          # one row / one column past a tile
    (1001, 777, 400, 416, 400, 1003, F8T128M),       # M % 8 == 1, ldc % 8 != 0: element-wise C
    (100, 300, 16, 16, 32, 104, F8T128M),            # a single 16-value K chunk
    (1000, 1000, 4096, 4096, 4112, 1000, F8T128SM),  # split K with M, N tails
    (1001, 520, 8208, 8224, 8208, 1008, F8T128SM),   # M % 8 == 1 in the reduction, K tail
    (250, 130, 3008, 3008, 3024, 256, F8T128SM),     # 4 tiles, a K tail in the last range
])
def test_fp8_medium_masked_shapes(M, N, K, lda, ldb, ldc, kernel, monkeypatch):
    monkeypatch.setenv("GEMM_BF16_FORCE_KERNEL", kernel)
    check_fp8(f"{kernel} {M}x{N}x{K}", M, N, K, lda=lda, ldb=ldb, ldc=ldc, beta=0.5, use_bias=True,
              epilogue="gelu_tanh", seed=M + N + K + 640, expect_kernel=kernel, poison_pad=True)


@pytest.mark.parametrize("M,N,K,ldc,kernel", [
    (1024, 1024, 4096, 1024, F8T128),     # 64 tiles, 32 slices: unsplit
    (512, 512, 8192, 512, F8T128S),      # 16 tiles, 64 slices: split
    (1000, 1000, 4096, 1000, F8T128M),
    (500, 500, 8192, 504, F8T128SM),
])
def test_fp8_small_grid_defaults(M, N, K, ldc, kernel):
    """Without forcing, small FP8 grids take the 128x128 tiles."""
    check_fp8(f"fp8 default {M}x{N}x{K}", M, N, K, ldc=ldc, beta=0.5, use_bias=True, epilogue="gelu_tanh",
              seed=M + N + K + 660, expect_kernel=kernel)


def test_fp8_medium_masked_unaligned_c(monkeypatch):
    monkeypatch.setenv("GEMM_BF16_FORCE_KERNEL", F8T128M)
    check_fp8("fp8 128x128 masked unaligned C", 520, 300, 640, ldc=521, offsets=(0, 0, 3), beta=0.5,
              use_bias=True, epilogue="relu", seed=650, expect_kernel=F8T128M)
    monkeypatch.setenv("GEMM_BF16_FORCE_KERNEL", F8T128SM)
    check_fp8("fp8 128x128 splitk masked unaligned C", 520, 300, 4000, ldc=523, offsets=(0, 0, 5), beta=-0.5,
              use_bias=True, epilogue="gelu_tanh", seed=651, expect_kernel=F8T128SM)


def test_fp8_kernels_with_one_accumulation_order_agree_bit_for_bit(monkeypatch):
    """The FP8 kernels on 32x32x64 MFMAs (256x256 tiles exact and masked,
    128x128 tiles exact and masked) give each output element the same MFMAs
    on the same operand bytes in the same k order, and scale and round it
    the same way (the sum times scale_a[m], times scale_b[n], times alpha:
    no additions to contract), so on exact tile multiples they must agree
    bit for bit."""
    M, N, K = 1024, 512, 640
    A, B = inputs.normal_fp8(720, M * K), inputs.normal_fp8(721, N * K)
    sa, sb = inputs.uniform_f32(722, M, 0.5, 2.0), inputs.uniform_f32(723, N, 0.5, 2.0)
    a_t, a_p = to_dev_u8(A)
    b_t, b_p = to_dev_u8(B)
    sa_t, sb_t = torch.from_numpy(sa).cuda(), torch.from_numpy(sb).cuda()
    outs = {}
    for kernel in ("fp8_256x256x128_mfma32", "fp8_256x256x128_masked", F8T128, F8T128M):
        monkeypatch.setenv("GEMM_BF16_FORCE_KERNEL", kernel)
        assert gb.gemm_fp8_kernel_name(M, N, K, a_p, K, b_p, K, a_p, M) == kernel
        c = torch.full((M * N,), -1, dtype=torch.int16, device="cuda")
        st = gb.gemm_fp8(M, N, K, a_p, K, b_p, K, c.data_ptr(), M, 1.25, 0.0, sa_t.data_ptr(), sb_t.data_ptr(), 0,
                         0, torch.cuda.current_stream().cuda_stream)
        assert st == 0, gb.gemm_bf16_status_string(st)
        torch.cuda.synchronize()
        outs[kernel] = c.cpu().numpy().view(np.uint16)
    ref = outs.pop("fp8_256x256x128_mfma32")
    for kernel, got in outs.items():
        assert np.array_equal(got, ref), f"{kernel} differs from fp8_256x256x128_mfma32"
    exp = oracle.gemm_fp8(M, N, K, A, K, B, K, None, M, 1.25, 0.0, sa, sb, None, "none", nthreads=_threads())
    assert_within_tolerance(ref, exp, K, "32x32x64 FP8 kernels vs oracle")


# The FP8 tile kernel on 32x32x64 MFMAs forced onto exact tiles (its masked
# instance is the default for tails, its split mode serves split-K): 1 to
# 10 K-slices, two tiles per CU, epilogue combinations with scales on and
# off, padded leading dimensions; and the masked instance of the 16x16x128
# kernel (forced) on tails.
FP8R32 = "fp8_256x256x128_mfma32"
FP8R16M = "fp8_256x256x128_mfma16_masked"


@pytest.mark.parametrize("M,N,K", [(256, 256, 128), (512, 256, 256), (512, 512, 384), (256, 512, 512),
                                   (1024, 512, 640), (256, 768, 1152), (4096, 2048, 1280), (8192, 4096, 128)])
def test_fp8_mfma32_slice_counts(M, N, K, monkeypatch):
    monkeypatch.setenv("GEMM_BF16_FORCE_KERNEL", FP8R32)
    check_fp8(f"fp8 mfma32 {M}x{N}x{K}", M, N, K, seed=M + N + K + 500, expect_kernel=FP8R32)


@pytest.mark.parametrize("beta,use_bias,epi,scales", [(b, u, e, sc) for b in (0.0, -0.75) for u in (False, True)
                                                      for e in ("none", "gelu_tanh", "relu") for sc in (True, False)
                                                      if not (u and not sc and e == "relu")])
def test_fp8_mfma32_epilogue_combinations(beta, use_bias, epi, scales, monkeypatch):
    monkeypatch.setenv("GEMM_BF16_FORCE_KERNEL", FP8R32)
    check_fp8(f"fp8 mfma32 beta={beta} bias={use_bias} {epi} scales={scales}", 1024, 512, 384, alpha=1.25,
              beta=beta, use_bias=use_bias, epilogue=epi, scales=scales,
              seed=510 + int(abs(beta) * 4) + 2 * use_bias + len(epi) + 7 * scales, expect_kernel=FP8R32)


def test_fp8_mfma32_padded_leading_dims(monkeypatch):
    monkeypatch.setenv("GEMM_BF16_FORCE_KERNEL", FP8R32)
    check_fp8("fp8 mfma32 padded", 512, 768, 512, lda=528, ldb=640, ldc=520, beta=0.5, use_bias=True, seed=530,
              expect_kernel=FP8R32)


@pytest.mark.parametrize("M,N,K,lda,ldb,ldc", [
    (300, 260, 144, 144, 144, 304),      # one full slice and a 16-wide K chunk
    (257, 513, 16, 32, 48, 264),         # a single 16-wide K chunk, 1-row / 1-column tails
    (1001, 777, 208, 224, 208, 1008),    # M % 8 == 1: the last 8-row chunk straddles M
    (255, 1, 128, 128, 144, 256),        # N = 1
    (520, 264, 4048, 4064, 4048, 528),   # 31 full slices and a 80-wide K tail
    (1001, 777, 400, 400, 416, 1003),    # ldc % 8 != 0: element-wise C
])
def test_fp8_mfma16_masked_tails(M, N, K, lda, ldb, ldc, monkeypatch):
    monkeypatch.setenv("GEMM_BF16_FORCE_KERNEL", FP8R16M)
    check_fp8(f"fp8 mfma16 masked {M}x{N}x{K}", M, N, K, lda=lda, ldb=ldb, ldc=ldc, beta=0.5, use_bias=True,
              epilogue="relu", seed=M + N + K + 540, expect_kernel=FP8R16M)


@pytest.mark.parametrize("beta,use_bias,epi,scales", [(0.0, False, "none", True), (-0.75, True, "gelu_tanh", False),
                                                      (0.5, False, "relu", True), (0.0, True, "none", False)])
def test_fp8_mfma16_masked_epilogue_combinations(beta, use_bias, epi, scales, monkeypatch):
    monkeypatch.setenv("GEMM_BF16_FORCE_KERNEL", FP8R16M)
    check_fp8(f"fp8 mfma16 masked beta={beta} bias={use_bias} {epi} scales={scales}", 777, 300, 208, ldc=784,
              alpha=1.25, beta=beta, use_bias=use_bias, epilogue=epi, scales=scales,
              seed=560 + int(abs(beta) * 4) + 2 * use_bias + len(epi) + 7 * scales, expect_kernel=FP8R16M)


# The masked 256x256 FP8 instance (forced: small grids take the 128x128
# tiles): M and N tails of every size class, K tails down to a single
# 16-byte chunk, padded leading dimensions, epilogue combinations, and exact
# tile multiples forced through it.
FP8M = "fp8_256x256x128_masked"


def test_fp8_masked_odd_ldc(monkeypatch):
    monkeypatch.setenv("GEMM_BF16_FORCE_KERNEL", FP8M)
    check_fp8("fp8 masked odd ldc", 1001, 777, 208, lda=224, ldb=208, ldc=1003, beta=0.5, use_bias=True,
              epilogue="relu", seed=420, expect_kernel=FP8M)
    check_fp8("fp8 masked unaligned C", 512, 512, 256, ldc=520, offsets=(0, 0, 3), beta=-0.5, seed=421,
              expect_kernel=FP8M)


@pytest.mark.parametrize("M,N,K,lda,ldb,ldc", [
    (300, 260, 144, 144, 144, 304),      # one full slice and a 16-wide K chunk
    (257, 513, 16, 32, 48, 264),         # a single 16-wide K chunk, 1-row / 1-column tails
    (1001, 777, 208, 224, 208, 1008),    # M % 8 == 1: the last 8-row chunk straddles M
    (255, 1, 128, 128, 144, 256),        # N = 1
    (65, 255, 64, 64, 64, 72),           # M = 65 (up to 64 rows take the streaming kernels)
    (520, 264, 4048, 4064, 4048, 528),   # 31 full slices and a 80-wide K tail (forced unsplit)
])
def test_fp8_masked_tails(M, N, K, lda, ldb, ldc, monkeypatch):
    monkeypatch.setenv("GEMM_BF16_FORCE_KERNEL", FP8M)
    check_fp8(f"fp8 masked {M}x{N}x{K}", M, N, K, lda=lda, ldb=ldb, ldc=ldc, seed=M + N + K + 11,
              expect_kernel=FP8M)


# Split-K on the masked 256x256 FP8 kernel (forced): whole tiles into a
# padded workspace, K tails in the last range, M % 8 != 0 in the reduction.
FP8SM = "splitk_fp8_256x256x128_masked"


@pytest.mark.parametrize("M,N,K,lda,ldb,ldc", [
    (520, 264, 4048, 4064, 4048, 528),   # 6 tiles, 32 slices: 8 ranges, an 80-wide K tail
    (1001, 777, 4000, 4000, 4016, 1008), # M % 8 == 1, N tail
    (300, 260, 2064, 2064, 2064, 304),   # 4 tiles, 17 slices: 4 ranges, a 16-wide K tail
    (1001, 777, 4000, 4000, 4000, 1001), # ldc % 8 != 0: element-wise C in the reduction
])
def test_fp8_masked_splitk_shapes(M, N, K, lda, ldb, ldc, monkeypatch):
    monkeypatch.setenv("GEMM_BF16_FORCE_KERNEL", FP8SM)
    check_fp8(f"fp8 masked splitk {M}x{N}x{K}", M, N, K, lda=lda, ldb=ldb, ldc=ldc, beta=0.5, use_bias=True,
              epilogue="gelu_tanh", seed=M + N + K + 400, expect_kernel=FP8SM)


@pytest.mark.parametrize("beta,use_bias,epi,scales", [(b, u, e, sc) for b in (0.0, -0.75) for u in (False, True)
                                                      for e in ("none", "gelu_tanh", "relu") for sc in (True, False)
                                                      if not (u and not sc and e == "relu")])
def test_fp8_masked_splitk_epilogue_combinations(beta, use_bias, epi, scales, monkeypatch):
    monkeypatch.setenv("GEMM_BF16_FORCE_KERNEL", FP8SM)
    check_fp8(f"fp8 masked splitk beta={beta} bias={use_bias} {epi} scales={scales}", 777, 300, 2000, ldc=784,
              alpha=1.25, beta=beta, use_bias=use_bias, epilogue=epi, scales=scales,
              seed=410 + int(abs(beta) * 4) + 2 * use_bias + len(epi) + 7 * scales, expect_kernel=FP8SM)


@pytest.mark.parametrize("beta,use_bias,epi", [(b, u, e) for b in (0.0, -0.75) for u in (False, True)
                                               for e in ("none", "gelu_tanh", "relu")])
def test_fp8_masked_epilogue_combinations(beta, use_bias, epi, monkeypatch):
    monkeypatch.setenv("GEMM_BF16_FORCE_KERNEL", FP8M)
    check_fp8(f"fp8 masked beta={beta} bias={use_bias} {epi}", 777, 300, 208, ldc=784, alpha=1.25, beta=beta,
              use_bias=use_bias, epilogue=epi, seed=17 + int(abs(beta) * 4) + 2 * use_bias + len(epi),
              expect_kernel=FP8M)


# FP8 on the matrix-vector kernel (1 to 4 rows): 16 values per 16-byte
# chunk, K blocks of 4096 with tails, N tails, scales on and off.
GVF = "gemv_fp8"


@pytest.mark.parametrize("M,N,K,lda,ldb,ldc", [
    (1, 4096, 4096, 4096, 4096, 1),      # decode: one full K block
    (2, 1000, 1040, 1040, 1056, 2),      # K tail inside the block
    (3, 333, 16, 16, 16, 3),             # a single 16-wide K chunk
    (4, 129, 4112, 4112, 4128, 4),       # a full block and a 16-wide second block
    (1, 5, 12304, 12304, 12304, 1),      # three blocks and a tail
    (4, 4097, 8208, 8208, 8224, 8),      # a 1-column last wave
])
def test_fp8_gemv_shapes(M, N, K, lda, ldb, ldc):
    check_fp8(f"fp8 gemv {M}x{N}x{K}", M, N, K, lda=lda, ldb=ldb, ldc=ldc, seed=M + N + K + 23,
              expect_kernel=GVF)


@pytest.mark.parametrize("beta,use_bias,epi,scales", [(b, u, e, sc) for b in (0.0, -0.75) for u in (False, True)
                                                      for e in ("none", "gelu_tanh", "relu") for sc in (True, False)
                                                      if not (u and not sc and e == "relu")])
def test_fp8_gemv_epilogue_combinations(beta, use_bias, epi, scales):
    check_fp8(f"fp8 gemv beta={beta} bias={use_bias} {epi} scales={scales}", 3, 515, 1008, ldc=3, alpha=1.25,
              beta=beta, use_bias=use_bias, epilogue=epi, scales=scales,
              seed=29 + int(abs(beta) * 4) + 2 * use_bias + len(epi) + 7 * scales, expect_kernel=GVF)


# FP8 on the streaming kernel (5 to 64 rows): 512-value slices with K
# tails, row / column tails, split-K, epilogue combinations with scales.
SKF = "skinny_fp8"


@pytest.mark.parametrize("M,N,K,lda,ldb,ldc", [
    (64, 1024, 4096, 4096, 4096, 64),    # 8 slices
    (33, 96, 528, 544, 528, 40),         # just over one 32-row block, a 16-wide K tail
    (7, 1000, 1040, 1040, 1056, 8),      # 7 rows, N and K tails
    (48, 4096, 1024, 1024, 1024, 48),
    (63, 129, 4112, 4112, 4128, 64),     # every tail at once
    (64, 1, 512, 512, 512, 64),          # one column, one slice
    (5, 300, 16, 16, 16, 5),             # a single 16-wide K chunk, ldc not a multiple of 8
])
@pytest.mark.parametrize("splits", ["1", "3"])
def test_fp8_skinny_shapes(M, N, K, lda, ldb, ldc, splits, monkeypatch):
    monkeypatch.setenv("GEMM_BF16_SKINNY_SPLITS", splits)
    check_fp8(f"fp8 skinny {M}x{N}x{K} splits={splits}", M, N, K, lda=lda, ldb=ldb, ldc=ldc,
              seed=M + N + K + 31, expect_kernel=SKF)


@pytest.mark.parametrize("beta,use_bias,epi,scales", [(b, u, e, sc) for b in (0.0, -0.75) for u in (False, True)
                                                      for e in ("none", "gelu_tanh", "relu") for sc in (True, False)
                                                      if not (u and not sc and e == "relu")])
def test_fp8_skinny_epilogue_combinations(beta, use_bias, epi, scales):
    check_fp8(f"fp8 skinny beta={beta} bias={use_bias} {epi} scales={scales}", 40, 515, 2048, ldc=41, alpha=1.25,
              beta=beta, use_bias=use_bias, epilogue=epi, scales=scales,
              seed=37 + int(abs(beta) * 4) + 2 * use_bias + len(epi) + 7 * scales, expect_kernel=SKF)


def test_fp8_masked_forced_on_tile_multiples(monkeypatch):
    monkeypatch.setenv("GEMM_BF16_FORCE_KERNEL", FP8M)
    check_fp8("fp8 masked forced", 512, 512, 384, beta=0.5, use_bias=True, seed=18, expect_kernel=FP8M)


def test_fp8_generic_paths(monkeypatch):
    check_fp8("fp8 generic ragged", 300, 200, 77, beta=0.5, use_bias=True, epilogue="gelu_tanh", seed=96,
              expect_kernel="generic64x64x32")
    check_fp8("fp8 generic unaligned", 256, 256, 256, offsets=(3, 5, 1), lda=259, ldb=261, ldc=257, seed=97,
              expect_kernel="generic64x64x32")
    check_fp8("fp8 K=0", 70, 50, 0, beta=2.0, use_bias=True, epilogue="relu", seed=98,
              expect_kernel="generic64x64x32")
    monkeypatch.setenv("GEMM_BF16_FORCE_KERNEL", "generic64x64x32")
    check_fp8("fp8 generic forced on a tile shape", 512, 512, 256, seed=99, expect_kernel="generic64x64x32")


# ------------------------------------------- the five workloads, full size ---

def sample_coords(M, N, tile, rng, n_random):
    ms, ns = [], []
    for (m0, n0) in [(0, 0), (max(M - tile, 0), max(N - tile, 0))]:
        mm, nn = np.meshgrid(np.arange(m0, min(m0 + tile, M)), np.arange(n0, min(n0 + tile, N)), indexing="ij")
        ms.append(mm.ravel())
        ns.append(nn.ravel())
    ms.append(rng.integers(0, M, n_random))
    ns.append(rng.integers(0, N, n_random))
    return np.concatenate(ms), np.concatenate(ns)


@pytest.mark.parametrize("name", list(inputs.WORKLOADS))
def test_workload_full_size_sampled(name):
    w = inputs.WORKLOADS[name]
    d = inputs.make_inputs(w)
    if w.out == "int8":
        return _workload_q8_sampled(w, d)
    if w.inp == "fp8":
        return _workload_fp8_sampled(w, d)
    M, N, K = w.M, w.N, w.K
    C0 = d.get("C0")
    C_init = C0 if C0 is not None else np.full(N * M, NAN_BF16, np.uint16)
    bias = d.get("bias")
    kname = gb.gemm_bf16_kernel_name(M, N, K, 4096, K, 4096, K, 4096, M)
    say(f"[parity] workload {name}: M={M} N={N} K={K} kernel={kname}")
    got = run_gpu(M, N, K, d["A"], K, d["B"], K, C_init, M, w.alpha, w.beta, bias, w.epilogue)
    assert not np.isnan(bits_to_f64(got)).any(), "NaN in the output"
    if M * N <= 256 * 256:
        ref = oracle.gemm(M, N, K, d["A"], K, d["B"], K, C0, M, w.alpha, w.beta, bias, w.epilogue,
                          nthreads=_threads())
        rep = assert_within_tolerance(got, ref, K, name)
    else:
        rng = np.random.Generator(np.random.PCG64(7 + w.index))
        ms, ns = sample_coords(M, N, 64 if M <= 64 else 256, rng, 20000)
        ref = oracle.gemm_elems(M, N, K, d["A"], K, d["B"], K, ms, ns, C0, M, w.alpha, w.beta, bias,
                                w.epilogue, nthreads=_threads())
        rep = assert_within_tolerance(got[ms + ns * M], ref, K, name)
    say(f"[parity] workload {name}: ok n={rep['n']} max_err/tol={rep['max_err_over_tol']:.3f} "
        f"mean_err/tol={rep['mean_err_over_tol']:.4f} exact={rep['exact']}")


def _workload_q8_sampled(w, d):
    M, N, K = w.M, w.N, w.K
    C0, bias, scale = d.get("C0"), d.get("bias"), d["scale"]
    kname = gb.gemm_bf16_q8_kernel_name(M, N, K, 4096, K, 4096, K, 4096 if C0 is not None else 0, M, 4096, M,
                                        w.beta, 4096, EPI[w.epilogue])
    say(f"[parity-q8] workload {w.name}: M={M} N={N} K={K} kernel={kname}")
    Q_init = np.full(N * M, Q8_POISON, np.int8)
    got = run_gpu_q8(M, N, K, d["A"], K, d["B"], K, C0, M, Q_init, M, w.alpha, w.beta, bias, w.epilogue, scale,
                     w.zero_point)
    rng = np.random.Generator(np.random.PCG64(7 + w.index))
    ms, ns = sample_coords(M, N, 256, rng, 20000)
    _, y = oracle.gemm_elems(M, N, K, d["A"], K, d["B"], K, ms, ns, C0, M, w.alpha, w.beta, bias, w.epilogue,
                             nthreads=_threads(), return_pre=True)
    ref, t = oracle.quantize_i8_array(y, scale[ms], w.zero_point)
    rep = assert_q8_within_tolerance(got[ms + ns * M], ref, t, scale[ms], w.zero_point, K, w.name)
    say(f"[parity-q8] workload {w.name}: ok exact={rep['exact']}/{rep['n']} near_boundary={rep['near_boundary']}")


def _workload_fp8_sampled(w, d):
    M, N, K = w.M, w.N, w.K
    kname = gb.gemm_fp8_kernel_name(M, N, K, 4096, K, 4096, K, 4096, M, EPI[w.epilogue])
    say(f"[parity-fp8] workload {w.name}: M={M} N={N} K={K} kernel={kname}")
    a_t, a_p = to_dev_u8(d["A"])
    b_t, b_p = to_dev_u8(d["B"])
    c_t, c_p = to_dev(np.full(N * M, NAN_BF16, np.uint16))
    sa_t = torch.from_numpy(d["scale_a"]).cuda()
    sb_t = torch.from_numpy(d["scale_b"]).cuda()
    st = gb.gemm_fp8(M, N, K, a_p, K, b_p, K, c_p, M, w.alpha, w.beta, sa_t.data_ptr(), sb_t.data_ptr(), 0,
                     EPI[w.epilogue], torch.cuda.current_stream().cuda_stream)
    assert st == 0, gb.gemm_bf16_status_string(st)
    torch.cuda.synchronize()
    got = from_dev(c_t, 0, N * M)
    rng = np.random.Generator(np.random.PCG64(7 + w.index))
    ms, ns = sample_coords(M, N, 256, rng, 20000)
    ref_bits = oracle.gemm_fp8_elems(M, N, K, d["A"], K, d["B"], K, ms, ns, scale_a=d["scale_a"],
                                     scale_b=d["scale_b"], epilogue=w.epilogue, nthreads=_threads())
    rep = assert_within_tolerance(got[ms + ns * M], ref_bits, K, w.name)
    say(f"[parity-fp8] workload {w.name}: ok n={rep['n']} max_err/tol={rep['max_err_over_tol']:.3f} exact={rep['exact']}")
