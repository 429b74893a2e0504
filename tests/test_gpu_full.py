"""GPU parity on the persistent multi-tile path, compared element by element.

The DeepGEMM-style article (section 4.1) checks a kernel by diffing its whole
fixed-seed result against a reference, and (section 4.2) names boundaries and
indexing as the places kernels go wrong.  The tile kernels here are
persistent: a workgroup takes tiles t, t + G, t + 2G, ... (G = number of
compute units), and the second and later tiles of a workgroup reuse the LDS
ring and the epilogue's staging area that the previous tile left behind.  So
these tests run grids of several tiles per compute unit and compare EVERY
output element against the CPU oracle:

* short K (256) keeps the oracle to seconds at 1024 to 1792 tiles (4 and 7
  per compute unit), with and without the full fused epilogue;
* the 4096^3 headline product and the 64-row streaming product at full size;
* at 8192^3 and 8192 x 14336 x 4096 (1.1 and 0.96 TFLOP, too slow for the
  oracle in full) one element of every 8-row chunk of every column -- the
  unit one lane stores -- so every store of every tile is checked;
* the int8 output with a whole-Q check: two runs from different initial Q
  contents must agree bit for bit (every code was written) and match the
  oracle everywhere;
* Inf and NaN operands and products that overflow bf16, on every kernel
  family;
* kernels with the same accumulation order (the ring, its masked instance
  on exact tile multiples, and the eight-wave ring) must agree bit for bit.

Tolerance: |gpu - oracle| <= 2 ulp_bf16(oracle) + 1e-3 sqrt(K); infinities
must match exactly and NaN only passes against NaN.
"""
from __future__ import annotations


import numpy as np
import pytest

import oracle
from bf16_gemm_fp32_amd import inputs
from tests.tolerance import assert_q8_within_tolerance, assert_within_tolerance, bits_to_f64
from tests.test_gpu_parity import (EPI, NAN_BF16, Q8_POISON, _threads, check_fp8, check_full, from_dev,
                                   run_gpu, run_gpu_q8, say, to_dev)

torch = pytest.importorskip("torch")
gb = pytest.importorskip("bf16_gemm_fp32_amd")

pytestmark = pytest.mark.gpu

RING = "ring256x256x64"
RINGM = "ring256x256x64_masked"
RINGW8 = "ring256x256x64_w8"
FP8 = "fp8_256x256x128"
RQ8 = "ring256x256x64_q8"

INF_BF16 = 0x7F80
NINF_BF16 = 0xFF80


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gb.library()
    yield


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


# ------------------------------------------- several tiles per compute unit ---

def test_ring_four_tiles_per_cu_full():
    """8192 x 8192 x 256: 1024 tiles of 256x256, four per compute unit on 256
    CUs; C starts as NaN (beta = 0), so an element never written fails."""
    tiles = (8192 // 256) ** 2
    assert tiles >= 4 * _cus()
    check_full("ring 8192x8192x256", 8192, 8192, 256, seed=901, expect_kernel=RING)


def test_ring_seven_tiles_per_cu_epilogue_full():
    """8192 x 14336 x 256 with the fused epilogue of the 8192 x 14336 x 4096
    workload (alpha 1, beta 0.5, bias[n], GELU-tanh): 1792 tiles, seven per
    compute unit.  C starts as C0, which differs from the result almost
    everywhere, and every element is compared."""
    check_full("ring 8192x14336x256 gelu", 8192, 14336, 256, alpha=1.0, beta=0.5, use_bias=True,
               epilogue="gelu_tanh", seed=902, expect_kernel=RING)


def test_fp8_ring_two_tiles_per_cu_full():
    """The default FP8 tile kernel (16x16x128 MFMAs) on 512 tiles, two per CU."""
    check_fp8("fp8 8192x4096x256", 8192, 4096, 256, seed=903, expect_kernel=FP8)


def test_fp8_ring_seven_tiles_per_cu_epilogue_full():
    check_fp8("fp8 8192x14336x256 gelu", 8192, 14336, 256, beta=0.5, use_bias=True, epilogue="gelu_tanh",
              seed=904, expect_kernel=FP8)


def test_q8_ring_seven_tiles_per_cu_whole_q():
    """Int8 output on 1792 tiles (ReLU, bias, zero point -20): every code is
    compared with the oracle, and a second run from a different initial Q
    must give the same bytes, so no code was left unwritten."""
    M, N, K, zp = 8192, 14336, 256, -20
    case = inputs.random_case(905, M, N, K, with_c0=False, with_bias=True)
    scale = inputs.uniform_f32(910, M, 0.25, 0.75)
    kname = gb.gemm_bf16_q8_kernel_name(M, N, K, 4096, K, 4096, K, 0, M, 4096, M, 0.0, 4096, EPI["relu"])
    say(f"[full-q8] {M}x{N}x{K} relu zp={zp} kernel={kname}")
    assert kname == RQ8
    runs = []
    for poison in (Q8_POISON, -Q8_POISON):
        Q_init = np.full(N * M, poison, np.int8)
        runs.append(run_gpu_q8(M, N, K, case["A"], K, case["B"], K, None, M, Q_init, M, 1.0, 0.0, case["bias"],
                               "relu", scale, zp))
    assert np.array_equal(runs[0], runs[1]), "int8 output depends on the initial Q: some codes not written"
    ref, t = oracle.gemm_q8(M, N, K, case["A"], K, case["B"], K, scale, zp, bias=case["bias"], epilogue="relu",
                            nthreads=_threads())
    rep = assert_q8_within_tolerance(runs[0].reshape(N, M), ref.reshape(N, M), t,
                                     np.broadcast_to(scale[None, :], (N, M)), zp, K, "q8 whole")
    say(f"[full-q8] ok exact={rep['exact']}/{rep['n']} near_boundary={rep['near_boundary']}")


def test_ring_variants_bit_identical_on_many_tiles(monkeypatch):
    """The masked ring instance and the eight-wave ring run, for every output
    element, the same MFMAs on the same operands in the same k order as the
    unmasked four-wave ring, so on exact tile multiples (where the masked one
    loads no zeros) all three must agree bit for bit -- on 512 tiles, two per
    CU, with the full epilogue.  A race in any LDS ring, or in the eight-wave
    kernel's hand-over from one tile's epilogue to the next tile's loads,
    would show up as a difference."""
    M, N, K = 8192, 4096, 512
    case = inputs.random_case(906, M, N, K, with_c0=True, with_bias=True)
    outs = []
    for kernel in (RING, RINGM, RINGW8):
        monkeypatch.setenv("GEMM_BF16_FORCE_KERNEL", kernel)
        assert gb.gemm_bf16_kernel_name(M, N, K, 4096, K, 4096, K, 4096, M) == kernel
        say(f"[full] bit-identity {M}x{N}x{K} kernel={kernel}")
        outs.append(run_gpu(M, N, K, case["A"], K, case["B"], K, case["C0"], M, 1.0, 0.5, case["bias"],
                            "gelu_tanh"))
    monkeypatch.delenv("GEMM_BF16_FORCE_KERNEL")
    assert np.array_equal(outs[0], outs[1]), "ring and masked ring differ on exact tile multiples"
    assert np.array_equal(outs[0], outs[2]), "four-wave and eight-wave rings differ"
    idx = np.random.Generator(np.random.PCG64(906)).integers(0, M * N, 4096)
    ref = oracle.gemm_elems(M, N, K, case["A"], K, case["B"], K, idx % M, idx // M, case["C0"], M, 1.0, 0.5,
                            case["bias"], "gelu_tanh", nthreads=_threads())
    assert_within_tolerance(outs[0][idx], ref, K, "ring vs oracle (sampled)")


# ------------------------------------------------ the workloads at full size ---

def _run_workload(w, d):
    M, N, K = w.M, w.N, w.K
    C0 = d.get("C0")
    C_init = C0 if C0 is not None else np.full(N * M, NAN_BF16, np.uint16)
    kname = gb.gemm_bf16_kernel_name(M, N, K, 4096, K, 4096, K, 4096, M)
    say(f"[full] workload {w.name}: M={M} N={N} K={K} kernel={kname}")
    return run_gpu(M, N, K, d["A"], K, d["B"], K, C_init, M, w.alpha, w.beta, d.get("bias"), w.epilogue)


@pytest.mark.parametrize("name", ["square_4096", "skinny_64x8192x8192", "ragged_4000x4000x4000",
                                  "mid_1024x1024x4096", "decode_1x4096x4096"])
def test_workload_every_element(name):
    """The whole output of the workload, in the launch configuration the
    benchmark times, against the whole oracle product."""
    w = inputs.WORKLOADS[name]
    d = inputs.make_inputs(w)
    got = _run_workload(w, d)
    ref = oracle.gemm(w.M, w.N, w.K, d["A"], w.K, d["B"], w.K, d.get("C0"), w.M, w.alpha, w.beta, d.get("bias"),
                      w.epilogue, nthreads=_threads())
    rep = assert_within_tolerance(got, ref, w.K, name)
    say(f"[full] workload {name}: ok n={rep['n']} max_err/tol={rep['max_err_over_tol']:.3f} exact={rep['exact']}")


@pytest.mark.parametrize("name", ["fp8_4096", "fp8_mid_1024x1024x4096"])
def test_fp8_workload_every_element(name):
    w = inputs.WORKLOADS[name]
    d = inputs.make_inputs(w)
    M, N, K = w.M, w.N, w.K
    kname = gb.gemm_fp8_kernel_name(M, N, K, 4096, K, 4096, K, 4096, M, EPI[w.epilogue])
    say(f"[full-fp8] workload {w.name}: kernel={kname}")
    a_t = torch.from_numpy(d["A"]).cuda()
    b_t = torch.from_numpy(d["B"]).cuda()
    c_t, c_p = to_dev(np.full(N * M, NAN_BF16, np.uint16))
    sa_t = torch.from_numpy(d["scale_a"]).cuda()
    sb_t = torch.from_numpy(d["scale_b"]).cuda()
    st = gb.gemm_fp8(M, N, K, a_t.data_ptr(), K, b_t.data_ptr(), K, c_p, M, w.alpha, w.beta, sa_t.data_ptr(),
                     sb_t.data_ptr(), 0, EPI[w.epilogue], torch.cuda.current_stream().cuda_stream)
    assert st == 0, gb.gemm_bf16_status_string(st)
    torch.cuda.synchronize()
    got = from_dev(c_t, 0, N * M)
    ref = oracle.gemm_fp8(M, N, K, d["A"], K, d["B"], K, scale_a=d["scale_a"], scale_b=d["scale_b"],
                          epilogue=w.epilogue, nthreads=_threads())
    rep = assert_within_tolerance(got, ref, K, w.name)
    say(f"[full-fp8] ok n={rep['n']} max_err/tol={rep['max_err_over_tol']:.3f} exact={rep['exact']}")


def _chunk_coords(M, N, seed):
    """One random row inside every 8-row chunk of every column: the unit a
    lane of the tile epilogue stores, so every store of every tile is
    checked once."""
    rng = np.random.Generator(np.random.PCG64(seed))
    chunks = (M + 7) // 8
    base = np.arange(chunks, dtype=np.int64) * 8
    ms = (base[None, :] + rng.integers(0, 8, (N, chunks))).ravel()
    ns = np.repeat(np.arange(N, dtype=np.int64), chunks)
    keep = ms < M
    return ms[keep], ns[keep]


@pytest.mark.parametrize("name", ["square_8192", "gelu_8192x14336x4096"])
def test_workload_every_store(name):
    w = inputs.WORKLOADS[name]
    d = inputs.make_inputs(w)
    got = _run_workload(w, d)
    assert not np.isnan(bits_to_f64(got)).any(), "NaN in the output"
    ms, ns = _chunk_coords(w.M, w.N, 17 + w.index)
    ref = oracle.gemm_elems(w.M, w.N, w.K, d["A"], w.K, d["B"], w.K, ms, ns, d.get("C0"), w.M, w.alpha, w.beta,
                            d.get("bias"), w.epilogue, nthreads=_threads())
    rep = assert_within_tolerance(got[ms + ns * w.M], ref, w.K, name)
    say(f"[full] workload {name}: ok n={rep['n']} (every 8-row chunk) "
        f"max_err/tol={rep['max_err_over_tol']:.3f} exact={rep['exact']}")


def test_q8_workload_every_store():
    w = inputs.WORKLOADS["q8relu_8192x14336x4096"]
    d = inputs.make_inputs(w)
    M, N, K = w.M, w.N, w.K
    runs = []
    for poison in (Q8_POISON, -Q8_POISON):
        Q_init = np.full(N * M, poison, np.int8)
        runs.append(run_gpu_q8(M, N, K, d["A"], K, d["B"], K, d.get("C0"), M, Q_init, M, w.alpha, w.beta,
                               d.get("bias"), w.epilogue, d["scale"], w.zero_point))
    assert np.array_equal(runs[0], runs[1]), "int8 output depends on the initial Q: some codes not written"
    ms, ns = _chunk_coords(M, N, 17 + w.index)
    _, y = oracle.gemm_elems(M, N, K, d["A"], K, d["B"], K, ms, ns, d.get("C0"), M, w.alpha, w.beta,
                             d.get("bias"), w.epilogue, nthreads=_threads(), return_pre=True)
    ref, t = oracle.quantize_i8_array(y, d["scale"][ms], w.zero_point)
    rep = assert_q8_within_tolerance(runs[0][ms + ns * M], ref, t, d["scale"][ms], w.zero_point, K, w.name)
    say(f"[full-q8] workload {w.name}: ok exact={rep['exact']}/{rep['n']}")


# ----------------------------------------------- Inf, NaN and bf16 overflow ---

def _special_case(M, N, K, seed):
    """N(0,1) operands with planted specials: row 1 of A has +Inf at k0 (its
    outputs are +-Inf by the sign of B[k0, n]); row 2 has +Inf at k0 and -Inf
    at k1 (NaN where B[k0, n] and B[k1, n] have the same sign, +-Inf where
    they differ); row 3 has a NaN (its row of C is NaN); column 2 of B has a
    NaN (its column of C is NaN)."""
    case = inputs.random_case(seed, M, N, K, with_c0=True, with_bias=True)
    A = case["A"].reshape(M, K)
    B = case["B"].reshape(N, K)
    k0, k1 = K // 3, (2 * K) // 3
    A[1, k0] = INF_BF16
    A[2, k0] = INF_BF16
    A[2, k1] = NINF_BF16
    A[3, k1] = NAN_BF16
    B[2, k0 + 1] = NAN_BF16
    return case


@pytest.mark.parametrize("M,N,K,kernel", [
    (4608, 2048, 256, RING),
    (1000, 700, 264, "tile128x128x64_s4_masked"),
    (1024, 1024, 4096, "splitk128x128x64"),
    (64, 2048, 1024, "skinny"),
    (4, 4096, 4096, "gemv"),
    (300, 200, 77, "generic64x64x32"),
])
@pytest.mark.parametrize("epi", ["none", "gelu_tanh"])
def test_inf_nan_operands(M, N, K, kernel, epi):
    case = _special_case(M, N, K, seed=M + N + K)
    kname = gb.gemm_bf16_kernel_name(M, N, K, 4096, K, 4096, K, 4096, M)
    say(f"[special] {M}x{N}x{K} epi={epi} kernel={kname}")
    assert kname == kernel
    got = run_gpu(M, N, K, case["A"], K, case["B"], K, np.full(N * M, NAN_BF16, np.uint16), M, 1.0, 0.0,
                  case["bias"], epi)
    ref = oracle.gemm(M, N, K, case["A"], K, case["B"], K, None, M, 1.0, 0.0, case["bias"], epi,
                      nthreads=_threads())
    r = bits_to_f64(ref).reshape(N, M)
    # the plants took effect: row 1 non-finite (infinite, or NaN where GELU
    # meets -Inf and in NaN column 2), column 2 and row 3 NaN
    assert (~np.isfinite(r[:, 1])).all() and np.isnan(r[2, :]).all() and np.isnan(r[:, 3]).all()
    rep = assert_within_tolerance(got, ref, K, f"specials {kernel} {epi}")
    say(f"[special] ok inf={int(np.isinf(r).sum())} nan={int(np.isnan(r).sum())} n={rep['n']}")


@pytest.mark.parametrize("M,N,K,kernel", [
    (4608, 2048, 256, RING),
    (512, 512, 256, "tile128x128x64_s4"),
    (64, 2048, 256, "skinny"),
])
def test_bf16_overflow(M, N, K, kernel):
    """Non-negative operands scaled by powers of two so that rows of A with
    exponent >= 64 give sums above 2^131 (beyond fp32, Inf in both) and rows
    with exponent <= 52 give sums below 2^123 (finite); no row lands near the
    bf16 overflow threshold, and with non-negative terms no partial sum of a
    finite row overflows in any order."""
    rng = np.random.Generator(np.random.PCG64(M + K))
    a = np.abs(rng.standard_normal((M, K), dtype=np.float32)) + np.float32(0.5)
    b = np.abs(rng.standard_normal((N, K), dtype=np.float32)) + np.float32(0.5)
    exps = np.where(np.arange(M) % 2 == 0, 40 + (np.arange(M) % 13), 64 + (np.arange(M) % 11)).astype(np.float32)
    a = a * np.exp2(exps)[:, None]
    b = b * np.float32(2.0 ** 60)
    A = inputs.f32_to_bf16_bits(a.ravel())
    B = inputs.f32_to_bf16_bits(b.ravel())
    kname = gb.gemm_bf16_kernel_name(M, N, K, 4096, K, 4096, K, 4096, M)
    say(f"[overflow] {M}x{N}x{K} kernel={kname}")
    assert kname == kernel
    got = run_gpu(M, N, K, A, K, B, K, np.full(N * M, NAN_BF16, np.uint16), M, 1.0, 0.0, None, "none")
    ref = oracle.gemm(M, N, K, A, K, B, K, None, M, 1.0, 0.0, None, "none", nthreads=_threads())
    r = bits_to_f64(ref).reshape(N, M)
    assert np.isinf(r[:, 1::2]).all() and np.isfinite(r[:, 0::2]).all()
    assert_within_tolerance(got, ref, K, f"overflow {kernel}")
