"""Pins for the CPU oracle: every check here compares it with something other
than itself -- exhaustive library decoding, exact rational arithmetic on tiny
inputs, a library double-precision matmul, closed forms (identity and
permutation matrices, exact scalings) and invariants (linearity, thread-count
independence).  A dropped term, a wrong sign or index, or a transposed
operand anywhere in the oracle makes at least one of them fail.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from bf16_gemm_fp32_amd import inputs
from tests.tolerance import bits_to_f64, tolerance_report, ulp_bf16

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# ---------------------------------------------------------------- helpers ---

def torch_decode(bits: np.ndarray) -> np.ndarray:
    """bf16 bits -> float64 through torch's own bfloat16 type."""
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).double().numpy()


_ALL_BITS = np.arange(65536, dtype=np.uint32).astype(np.uint16)
_ALL_VALS = torch_decode(_ALL_BITS)
_FIN = np.isfinite(_ALL_VALS) & (_ALL_BITS != 0x8000)       # one zero only
_SORTED_IDX = np.argsort(_ALL_VALS[_FIN], kind="stable")
_SORTED_VALS = _ALL_VALS[_FIN][_SORTED_IDX]
_SORTED_BITS = _ALL_BITS[_FIN][_SORTED_IDX]


def round_fraction_to_bf16(q: Fraction) -> int:
    """Nearest finite bf16 to the exact rational q, ties to the even pattern.

    Brute force over the sorted table of all bf16 values; independent of the
    oracle's frexp/rint method.  (No overflow handling: inputs here are small.)
    """
    x = float(q)  # only used to locate the neighbours
    i = int(np.searchsorted(_SORTED_VALS, x))
    cands = [j for j in (i - 2, i - 1, i, i + 1) if 0 <= j < _SORTED_VALS.size]
    lo = max((j for j in cands if Fraction(_SORTED_VALS[j]) <= q), key=lambda j: _SORTED_VALS[j])
    hi = min((j for j in cands if Fraction(_SORTED_VALS[j]) >= q), key=lambda j: _SORTED_VALS[j])
    if lo == hi:
        return int(_SORTED_BITS[lo])
    dlo = q - Fraction(_SORTED_VALS[lo])
    dhi = Fraction(_SORTED_VALS[hi]) - q
    if dlo < dhi:
        return int(_SORTED_BITS[lo])
    if dhi < dlo:
        return int(_SORTED_BITS[hi])
    return int(_SORTED_BITS[lo] if (_SORTED_BITS[lo] & 1) == 0 else _SORTED_BITS[hi])


def same_value(a_bits, b_bits) -> np.ndarray:
    """Bit equality with +0 == -0."""
    a = np.asarray(a_bits, dtype=np.uint16)
    b = np.asarray(b_bits, dtype=np.uint16)
    zero = ((a & 0x7FFF) == 0) & ((b & 0x7FFF) == 0)
    return (a == b) | zero


def dense(case, M, N, K):
    """Decode a case's flat buffers into float64 matrices (A: MxK, B: KxN)."""
    A = bits_to_f64(case["A"]).reshape(M, case["lda"])[:, :K]
    B = bits_to_f64(case["B"]).reshape(N, case["ldb"])[:, :K].T
    return A, B


# ------------------------------------------------------------ P1, P2 bf16 ---

def test_p1_decode_exhaustive_matches_torch():
    got = oracle.bf16_to_f64(_ALL_BITS)
    ref = _ALL_VALS
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def _finite_positive_bits():
    b = _ALL_BITS[(_ALL_BITS < 0x7F80)]
    return b


def test_p2_exact_values_round_to_themselves():
    b = _ALL_BITS[np.isfinite(_ALL_VALS)]
    assert np.array_equal(oracle.bf16_from_f64(_ALL_VALS[np.isfinite(_ALL_VALS)]), b)


def test_p2_midpoints_round_to_even_and_offsets_to_nearer():
    lo = _finite_positive_bits()[:-1]              # 0 .. max finite - 1 step
    hi = lo + 1
    vlo, vhi = _ALL_VALS[lo], _ALL_VALS[hi]
    mid = (vlo + vhi) / 2                          # exact in float64
    even = np.where((lo & 1) == 0, lo, hi)
    assert np.array_equal(oracle.bf16_from_f64(mid), even)
    assert np.array_equal(oracle.bf16_from_f64(-mid), even | 0x8000)
    step = (vhi - vlo) * 2.0 ** -20
    assert np.array_equal(oracle.bf16_from_f64(mid - step), lo)
    assert np.array_equal(oracle.bf16_from_f64(mid + step), hi)


def test_p2_overflow_underflow_specials():
    maxf = _ALL_VALS[0x7F7F]
    half = 2.0 ** 127 * 2.0 ** -8                  # half a ulp at the top binade
    assert oracle.bf16_from_f64(np.array([maxf + half]))[0] == 0x7F80
    assert oracle.bf16_from_f64(np.array([maxf + half * (1 - 2.0 ** -20)]))[0] == 0x7F7F
    assert oracle.bf16_from_f64(np.array([-(maxf + half)]))[0] == 0xFF80
    assert oracle.bf16_from_f64(np.array([np.inf]))[0] == 0x7F80
    assert oracle.bf16_from_f64(np.array([-np.inf]))[0] == 0xFF80
    assert (oracle.bf16_from_f64(np.array([np.nan]))[0] & 0x7FFF) > 0x7F80
    tiny = 2.0 ** -133                             # smallest bf16 subnormal
    assert oracle.bf16_from_f64(np.array([tiny]))[0] == 0x0001
    assert oracle.bf16_from_f64(np.array([tiny / 2]))[0] == 0x0000     # tie -> even (0)
    assert oracle.bf16_from_f64(np.array([tiny * 0.75]))[0] == 0x0001
    assert oracle.bf16_from_f64(np.array([tiny * 1.5]))[0] == 0x0002   # tie -> even (2)
    assert oracle.bf16_from_f64(np.array([-0.0]))[0] == 0x8000
    assert oracle.bf16_from_f64(np.array([1e-300]))[0] == 0x0000


def test_p2_matches_torch_on_float32_inputs():
    """On float32-representable inputs torch's float->bfloat16 cast rounds once."""
    g = np.random.Generator(np.random.PCG64(7))
    x = np.concatenate([
        g.standard_normal(200_000).astype(np.float32),
        (g.standard_normal(50_000) * 1e30).astype(np.float32),
        (g.standard_normal(50_000) * 1e-39).astype(np.float32),   # float32 subnormals
        g.integers(0, 2 ** 32, 100_000, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ])
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_from_f64(x.astype(np.float64))
    assert np.array_equal(got, ref)


# ------------------------------------------------------------- P3 brute ---

@pytest.mark.parametrize("seed", range(12))
def test_p3_exact_rational_bruteforce_tiny(seed):
    g = np.random.Generator(np.random.PCG64(100 + seed))
    M, N, K = (int(v) for v in g.integers(1, 9, 3))
    lda, ldb, ldc = K + int(g.integers(0, 3)), K + int(g.integers(0, 3)), M + int(g.integers(0, 3))
    case = inputs.random_case(1000 * seed, M, N, K, lda, ldb, ldc, with_c0=True, with_bias=True)
    alpha = float(g.choice([1.0, 0.75, -2.0]))
    beta = float(g.choice([0.0, 0.5, -1.25]))
    use_bias = bool(g.integers(0, 2))
    bias = case["bias"] if use_bias else None
    got = oracle.gemm(M, N, K, case["A"], lda, case["B"], ldb, case["C0"], ldc,
                      alpha, beta, bias, "none")
    Af = [Fraction(float(v)) for v in bits_to_f64(case["A"])]
    Bf = [Fraction(float(v)) for v in bits_to_f64(case["B"])]
    Cf = [Fraction(float(v)) for v in bits_to_f64(case["C0"])]
    biasf = [Fraction(float(v)) for v in bits_to_f64(case["bias"])]
    for n in range(N):
        for m in range(M):
            s = sum((Af[m * lda + k] * Bf[k + n * ldb] for k in range(K)), Fraction(0))
            y = Fraction(alpha) * s
            if beta != 0.0:
                y += Fraction(beta) * Cf[m + n * ldc]
            if use_bias:
                y += biasf[n]
            want = round_fraction_to_bf16(y)
            assert same_value(got[m + n * ldc], want), (m, n, got[m + n * ldc], want)


def test_p3_k1_is_the_rounded_product():
    g = np.random.Generator(np.random.PCG64(5))
    M, N = 37, 29
    a = inputs.normal_bf16(11, M)
    b = inputs.normal_bf16(12, N)
    got = oracle.gemm(M, N, 1, a, 1, b, 1).reshape(N, M)
    prod = np.outer(bits_to_f64(b), bits_to_f64(a))   # (n, m), exact in float64
    want = np.vectorize(lambda v: round_fraction_to_bf16(Fraction(float(v))))(prod)
    assert np.all(same_value(got, want))
    del g


# ---------------------------------------------------------- P4 library ---

@pytest.mark.parametrize("M,N,K,pad", [(64, 48, 96, 0), (130, 70, 257, 3), (256, 256, 512, 0)])
def test_p4_matches_numpy_float64_matmul(M, N, K, pad):
    case = inputs.random_case(4242 + K, M, N, K, K + pad, K + 2 * pad, M + pad)
    got, pre = oracle.gemm(M, N, K, case["A"], case["lda"], case["B"], case["ldb"],
                           ldc=case["ldc"], return_pre=True)
    A, B = dense(case, M, N, K)
    ref = A @ B                                              # (M, N) float64 dgemm
    scale = np.abs(A) @ np.abs(B)
    assert np.all(np.abs(pre.T - ref) <= 1e-13 * scale + 1e-300)
    ref_bits = oracle.bf16_from_f64(ref)                     # pinned by P2
    got_mn = got.reshape(N, case["ldc"])[:, :M].T
    diff = ~same_value(got_mn, ref_bits)
    if diff.any():
        # only allowed where ref sits within 1e-12 (relative) of a rounding midpoint
        r = ref[diff]
        u = ulp_bf16(bits_to_f64(ref_bits[diff]))
        frac = np.abs(r) / u
        near_mid = np.abs(frac - np.floor(frac) - 0.5) * u <= 1e-12 * np.maximum(scale[diff], 1)
        assert near_mid.all()
    assert np.count_nonzero(diff) <= 2
    # padding rows of C are untouched (left at 0 by the oracle wrapper)
    if case["ldc"] > M:
        assert np.all(got.reshape(N, case["ldc"])[:, M:] == 0)


# -------------------------------------------------- P5 layout / indexing ---

def _identity_bits(n):
    eye = np.zeros((n, n), dtype=np.uint16)
    eye[np.arange(n), np.arange(n)] = 0x3F80
    return eye


def test_p5_identity_A_returns_B():
    M = K = 48
    N = 21
    case = inputs.random_case(77, M, N, K)
    A = _identity_bits(M).reshape(-1)
    got = oracle.gemm(M, N, K, A, K, case["B"], K)
    assert np.all(same_value(got.reshape(N, M), case["B"].reshape(N, K)))


def test_p5_identity_B_returns_A():
    M, K = 19, 40
    N = K
    case = inputs.random_case(78, M, N, K)
    B = _identity_bits(K).reshape(-1)                 # column-major identity
    got = oracle.gemm(M, N, K, case["A"], K, B, K).reshape(N, M)
    assert np.all(same_value(got.T, case["A"].reshape(M, K)))


def test_p5_permutations_rectangular_padded():
    g = np.random.Generator(np.random.PCG64(3))
    M = K = 33
    N = 17
    lda, ldb, ldc = K + 5, K + 2, M + 7
    perm = g.permutation(M)
    A = np.zeros((M, lda), dtype=np.uint16)
    A[np.arange(M), perm] = 0x3F80                    # A[m, perm[m]] = 1
    A[:, K:] = 0x7FC0                                 # NaN in the padding: must never be read
    case = inputs.random_case(79, M, N, K, ldb=ldb)
    Bmat = case["B"].reshape(N, ldb)
    Bmat[:, K:] = 0x7FC0
    got = oracle.gemm(M, N, K, A.reshape(-1), lda, Bmat.reshape(-1), ldb, ldc=ldc)
    got = got.reshape(N, ldc)[:, :M]                  # (n, m)
    want = Bmat[:, :K][:, perm]                       # C[m,n] = B[perm[m], n]
    assert np.all(same_value(got, want))
    # column permutation via B: B[k, n] = 1 iff k == q[n]  ->  C[m, n] = A[m, q[n]]
    M2, K2, N2 = 23, 31, 29
    q = g.integers(0, K2, N2)
    case2 = inputs.random_case(80, M2, N2, K2, lda=K2 + 1)
    B2 = np.zeros((N2, K2), dtype=np.uint16)
    B2[np.arange(N2), q] = 0x3F80
    got2 = oracle.gemm(M2, N2, K2, case2["A"], K2 + 1, B2.reshape(-1), K2).reshape(N2, M2)
    Amat = case2["A"].reshape(M2, K2 + 1)
    assert np.all(same_value(got2.T, Amat[:, q]))


# --------------------------------------------------------- P6 linearity ---

def test_p6_linearity_disjoint_split():
    M, N, K = 40, 36, 300
    case = inputs.random_case(91, M, N, K)
    g = np.random.Generator(np.random.PCG64(92))
    mask = g.integers(0, 2, case["B"].size).astype(bool)
    B1 = np.where(mask, case["B"], np.uint16(0))
    B2 = np.where(mask, np.uint16(0), case["B"])
    _, p = oracle.gemm(M, N, K, case["A"], K, case["B"], K, return_pre=True)
    _, p1 = oracle.gemm(M, N, K, case["A"], K, B1, K, return_pre=True)
    _, p2 = oracle.gemm(M, N, K, case["A"], K, B2, K, return_pre=True)
    A, B = dense(case, M, N, K)
    scale = (np.abs(A) @ np.abs(B)).T
    assert np.all(np.abs(p - (p1 + p2)) <= 1e-12 * scale)
    # and the split is not trivial: each part alone differs from the whole
    assert np.abs(p - p1).max() > 1.0 and np.abs(p - p2).max() > 1.0


def test_p6_power_of_two_scaling_exact():
    M, N, K = 24, 20, 128
    case = inputs.random_case(93, M, N, K)
    B2 = (case["B"].astype(np.uint32) + 0x80).astype(np.uint16)   # exponent + 1: 2*B
    assert np.array_equal(bits_to_f64(B2), 2 * bits_to_f64(case["B"]))
    c1 = oracle.gemm(M, N, K, case["A"], K, case["B"], K)
    c2 = oracle.gemm(M, N, K, case["A"], K, B2, K)
    assert np.array_equal(bits_to_f64(c2), 2 * bits_to_f64(c1))


# ------------------------------------------------ P7 alpha / beta / bias ---

def test_p7_zero_A_gives_beta_c0_plus_bias_closed_forms():
    M, N, K = 12, 9, 16                              # M != N catches bias[m] vs bias[n]
    case = inputs.random_case(95, M, N, K, with_c0=True, with_bias=True)
    zeroA = np.zeros_like(case["A"])
    # beta = 0.5, no bias: exactly half of C0
    got = oracle.gemm(M, N, K, zeroA, K, case["B"], K, case["C0"], M, 1.0, 0.5)
    assert np.array_equal(bits_to_f64(got), 0.5 * bits_to_f64(case["C0"]))
    # C0[m, n] = -bias[n] with beta = 1: every output is exactly zero
    c0 = np.tile(case["bias"] ^ np.uint16(0x8000), (M, 1)).T.reshape(-1).copy()
    got = oracle.gemm(M, N, K, zeroA, K, case["B"], K, c0, M, 1.0, 1.0, case["bias"])
    assert np.all(bits_to_f64(got) == 0)
    # K = 0 takes the same path: C = beta*C0 + bias, here with beta = -2 (exact)
    got = oracle.gemm(M, N, 0, np.zeros(0, np.uint16), 1, np.zeros(0, np.uint16), 1,
                      case["C0"], M, 1.0, -2.0, None)
    assert np.array_equal(bits_to_f64(got), -2 * bits_to_f64(case["C0"]))


def test_p7_alpha_two_doubles_exactly():
    M, N, K = 30, 26, 64
    case = inputs.random_case(96, M, N, K)
    c1 = oracle.gemm(M, N, K, case["A"], K, case["B"], K, alpha=1.0)
    c2 = oracle.gemm(M, N, K, case["A"], K, case["B"], K, alpha=2.0)
    assert np.array_equal(bits_to_f64(c2), 2 * bits_to_f64(c1))


def test_p7_beta_zero_never_reads_c():
    M, N, K = 16, 16, 32
    case = inputs.random_case(97, M, N, K, with_bias=True)
    nanC = np.full(M * N, 0x7FC0, dtype=np.uint16)
    c_nan = oracle.gemm(M, N, K, case["A"], K, case["B"], K, nanC, M, 1.0, 0.0, case["bias"])
    c_zero = oracle.gemm(M, N, K, case["A"], K, case["B"], K, None, M, 1.0, 0.0, case["bias"])
    assert not np.isnan(bits_to_f64(c_nan)).any()
    assert np.array_equal(c_nan, c_zero)


def test_worked_example_by_hand():
    """A = [[1,2],[3,4]], B = [[5,6],[7,8]]: A*B = [[19,22],[43,50]].
    With alpha = 0.5, beta = 2, C0 = I and bias = [1, -1]:
    y = [[9.5+2+1, 11+0-1], [21.5+0+1, 25+2-1]] = [[12.5, 10], [22.5, 26]],
    all exactly representable in bf16."""
    f = inputs.f32_to_bf16_bits
    A = f(np.array([1, 2, 3, 4], np.float32))            # row-major
    B = f(np.array([5, 7, 6, 8], np.float32))            # column-major: columns (5,7), (6,8)
    C0 = f(np.array([1, 0, 0, 1], np.float32))           # column-major identity
    bias = f(np.array([1, -1], np.float32))
    plain = oracle.gemm(2, 2, 2, A, 2, B, 2)
    assert bits_to_f64(plain).tolist() == [19, 43, 22, 50]
    got = oracle.gemm(2, 2, 2, A, 2, B, 2, C0, 2, 0.5, 2.0, bias)
    assert bits_to_f64(got).tolist() == [12.5, 22.5, 10, 26]


# ---------------------------------------------------------------- P8 GELU ---

def test_p8_gelu_identities_and_torch():
    x = np.concatenate([np.linspace(-12, 12, 4001), bits_to_f64(inputs.normal_bf16(1, 1000)) * 3])
    g = oracle.gelu_tanh(x)
    assert oracle.gelu_tanh(np.array([0.0]))[0] == 0.0
    assert np.all(np.abs((g - oracle.gelu_tanh(-x)) - x) <= 1e-15 * np.maximum(1, np.abs(x)))
    assert abs(oracle.gelu_tanh(np.array([10.0]))[0] - 10.0) <= 1e-14
    assert abs(oracle.gelu_tanh(np.array([-10.0]))[0]) <= 1e-15
    ref = torch.nn.functional.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    assert np.all(np.abs(g - ref) <= 2e-15 * np.maximum(1, np.abs(x)))


def test_p8_gelu_in_the_gemm_is_applied_after_bias():
    """K = 1: pre-activation is a*b + bias exactly (in double); the output is
    the rounded torch GELU of that value."""
    M, N = 21, 13
    a = inputs.normal_bf16(31, M)
    b = inputs.normal_bf16(32, N)
    bias = inputs.normal_bf16(33, N, scale=0.1)
    got = oracle.gemm(M, N, 1, a, 1, b, 1, bias=bias, epilogue="gelu_tanh").reshape(N, M)
    pre = np.outer(bits_to_f64(b), bits_to_f64(a)) + bits_to_f64(bias)[:, None]
    ref = torch.nn.functional.gelu(torch.from_numpy(pre), approximate="tanh").numpy()
    assert np.count_nonzero(~same_value(got, oracle.bf16_from_f64(ref))) <= 1


# ------------------------------------------------ P9 thread independence ---

def test_p9_thread_count_independent():
    M, N, K = 96, 80, 200
    case = inputs.random_case(99, M, N, K, with_c0=True, with_bias=True)
    args = (M, N, K, case["A"], K, case["B"], K, case["C0"], M, 1.5, -0.5, case["bias"], "gelu_tanh")
    c1 = oracle.gemm(*args, nthreads=1)
    c8 = oracle.gemm(*args, nthreads=8)
    assert np.array_equal(c1, c8)


def test_elems_agree_with_whole_product():
    M, N, K = 50, 60, 70
    case = inputs.random_case(101, M, N, K, with_c0=True, with_bias=True)
    full = oracle.gemm(M, N, K, case["A"], K, case["B"], K, case["C0"], M, 1.0, 0.5,
                       case["bias"], "gelu_tanh")
    g = np.random.Generator(np.random.PCG64(102))
    ms, ns = g.integers(0, M, 300), g.integers(0, N, 300)
    el = oracle.gemm_elems(M, N, K, case["A"], K, case["B"], K, ms, ns, case["C0"], M,
                           1.0, 0.5, case["bias"], "gelu_tanh")
    assert np.array_equal(el, full[ms + ns * M])


def test_oracle_rejects_bad_arguments():
    z = np.zeros(16, np.uint16)
    with pytest.raises(ValueError):
        oracle.gemm(4, 4, 4, z, 3, z, 4)                  # lda < K
    with pytest.raises(ValueError):
        oracle.gemm(4, 4, 4, z, 4, z, 4, None, 4, 1.0, 1.0)   # beta != 0 without C


# ---------------------------------------------------- P10 the tolerance ---

def test_p10_tolerance_hand_cases():
    f = inputs.f32_to_bf16_bits
    one = f(np.array([1.0], np.float32))
    assert tolerance_report(f(np.array([1.0078125], np.float32)), one, 4096)["fail"] == 0
    # 0 vs 0.05 at K=4096: the absolute slack 1e-3*64 = 0.064 covers it
    assert tolerance_report(f(np.array([0.05], np.float32)), f(np.array([0.0], np.float32)), 4096)["fail"] == 0
    assert tolerance_report(f(np.array([0.07], np.float32)), f(np.array([0.0], np.float32)), 4096)["fail"] == 1
    # at 256: ulp(256) = 2, so 2 ulps = 4 plus slack 0.064; 260 passes, 262 fails
    big = f(np.array([256.0], np.float32))
    assert tolerance_report(f(np.array([260.0], np.float32)), big, 4096)["fail"] == 0
    assert tolerance_report(f(np.array([262.0], np.float32)), big, 4096)["fail"] == 1
    # just below a binade boundary the ulp is the smaller one: ulp(255) = 1
    below = f(np.array([255.0], np.float32))
    assert tolerance_report(f(np.array([258.0], np.float32)), below, 0)["fail"] == 1
    assert tolerance_report(f(np.array([256.0], np.float32)), below, 0)["fail"] == 0
    nan = np.array([0x7FC0], np.uint16)
    assert tolerance_report(nan, nan, 1)["fail"] == 0
    assert tolerance_report(one, nan, 1)["fail"] == 1
    assert tolerance_report(nan, one, 1)["fail"] == 1


# ---------------------------------------------------------------- P11 ReLU ---

def test_p11_relu_in_the_gemm_matches_torch_after_bias():
    """K = 1: the pre-activation a*b + bias is exact in double; the output is
    torch's ReLU of it, rounded (the P2-pinned rounding)."""
    M, N = 23, 17
    a = inputs.normal_bf16(41, M)
    b = inputs.normal_bf16(42, N)
    bias = inputs.normal_bf16(43, N, scale=0.5)
    got, pre = oracle.gemm(M, N, 1, a, 1, b, 1, bias=bias, epilogue="relu", return_pre=True)
    y = np.outer(bits_to_f64(b), bits_to_f64(a)) + bits_to_f64(bias)[:, None]
    ref = torch.relu(torch.from_numpy(y)).numpy()
    assert np.array_equal(pre, ref)
    assert np.all(same_value(got.reshape(N, M), oracle.bf16_from_f64(ref)))
    assert np.count_nonzero(ref == 0) > 50 and np.count_nonzero(ref > 0) > 50


def test_p11_relu_odd_part_identity_and_nan():
    """relu(y) - relu(-y) = y: negating A and bias negates the pre-activation
    exactly.  NaN (inf * 0) passes through ReLU, as in torch."""
    M, N, K = 30, 22, 40
    case = inputs.random_case(44, M, N, K, with_bias=True)
    neg = lambda bits: (np.asarray(bits, np.uint16) ^ np.uint16(0x8000)).astype(np.uint16)
    _, p1 = oracle.gemm(M, N, K, case["A"], K, case["B"], K, bias=case["bias"], epilogue="relu", return_pre=True)
    _, p2 = oracle.gemm(M, N, K, neg(case["A"]), K, case["B"], K, bias=neg(case["bias"]), epilogue="relu",
                        return_pre=True)
    _, p0 = oracle.gemm(M, N, K, case["A"], K, case["B"], K, bias=case["bias"], return_pre=True)
    assert np.array_equal(p1 - p2, p0)
    inf, zero = np.array([0x7F80], np.uint16), np.array([0], np.uint16)
    out = oracle.gemm(1, 1, 1, inf, 1, zero, 1, epilogue="relu")
    assert np.isnan(bits_to_f64(out)[0]) and np.isnan(torch.relu(torch.tensor([np.nan])).item())


# ------------------------------------------------------- P12 int8 output ---

def round_fraction_to_f32(q: Fraction) -> Fraction:
    """Nearest binary32 value to the exact rational q, ties to even (normal
    range only; enough for the values here)."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    unit = Fraction(2) ** (e - 23)
    return sign * round(a / unit) * unit  # Python's round() on a Fraction ties to even


def q8_code_by_hand(y: Fraction, s: float, zp: int) -> int:
    """The decision the pages' formula describes, taken in fp32 exactly:
    x = f32(y), t = f32(x*s + zp) (one rounding), ties-to-even integer,
    saturated."""
    x = round_fraction_to_f32(y)
    t = round_fraction_to_f32(x * Fraction(s) + zp)
    return max(-128, min(127, round(t)))


def test_p12_quantize_hand_table():
    """Worked by hand: scale 1, zero point 0, exact K = 1 products."""
    f = inputs.f32_to_bf16_bits
    cases = [(2.5, 2), (3.5, 4), (-2.5, -2), (0.5, 0), (1.5, 2), (-0.5, 0), (126.5, 126), (127.5, 127),
             (300.0, 127), (-300.0, -128), (0.75, 1), (-0.75, -1)]
    vals = np.array([v for v, _ in cases], np.float32)
    A = f(vals)
    B = f(np.array([1.0], np.float32))
    Q, t = oracle.gemm_q8(len(cases), 1, 1, A, 1, B, 1, np.ones(len(cases), np.float32), 0)
    assert Q.tolist() == [c for _, c in cases]
    assert np.array_equal(t[0], vals.astype(np.float64))
    # zero point 10 and scale 1/4: 2.5*... -> rint(v/4 + 10)
    Q2, _ = oracle.gemm_q8(len(cases), 1, 1, A, 1, B, 1, np.full(len(cases), 0.25, np.float32), 10)
    assert Q2.tolist() == [max(-128, min(127, round(Fraction(float(v)) / 4 + 10))) for v in vals]
    # zero point -128: -128.5 -> -128 (even), -129.5 -> -130 -> saturates, -127.5 -> -128, -126.5 -> -126
    Q3, _ = oracle.gemm_q8(4, 1, 1, f(np.array([-0.5, -1.5, 0.5, 1.5], np.float32)), 1, B, 1,
                           np.ones(4, np.float32), -128)
    assert Q3.tolist() == [-128, -128, -128, -126]
    # NaN (inf * 0) gives 0
    Qn, tn = oracle.gemm_q8(1, 1, 1, np.array([0x7F80], np.uint16), 1, np.array([0], np.uint16), 1,
                            np.ones(1, np.float32), 5)
    assert Qn.tolist() == [0] and np.isnan(tn[0, 0])


@pytest.mark.parametrize("seed", range(8))
def test_p12_quantize_exact_rational_bruteforce(seed):
    """Tiny random products with per-row scales, a zero point, alpha, beta,
    bias and each activation but GELU: exact rational epilogue value, then the
    fp32 decision worked by hand -- identical codes."""
    g = np.random.Generator(np.random.PCG64(7000 + seed))
    M, N, K = (int(v) for v in g.integers(1, 9, 3))
    case = inputs.random_case(7100 + seed, M, N, K, with_c0=True, with_bias=True)
    scale = (g.random(M) * 8 + 0.5).astype(np.float32) * np.float32(g.choice([-1, 1]))
    zp = int(g.integers(-20, 21))
    alpha, beta = 1.25, -0.5
    epi = ["none", "relu"][seed % 2]
    Q, _ = oracle.gemm_q8(M, N, K, case["A"], K, case["B"], K, scale, zp, C_in=case["C0"], ldc=M,
                          alpha=alpha, beta=beta, bias=case["bias"], epilogue=epi)
    A, B = dense(case, M, N, K)
    C0 = bits_to_f64(case["C0"]).reshape(N, M)
    bias = bits_to_f64(case["bias"])
    for n in range(N):
        for m in range(M):
            s = sum(Fraction(A[m, k]) * Fraction(B[k, n]) for k in range(K))
            y = Fraction(alpha) * s + Fraction(beta) * Fraction(C0[n, m]) + Fraction(bias[n])
            if epi == "relu" and y < 0:
                y = Fraction(0)
            assert Q[m + n * M] == q8_code_by_hand(y, float(scale[m]), zp), (m, n)


def test_p12_quantize_rows_use_their_own_scale_and_layout():
    """M != N, padded ldq: row m uses scale[m] (indexing by n would fail),
    codes land at Q[m + n*ldq] and the padding stays 0."""
    M, N, K, ldq = 12, 7, 5, 16
    case = inputs.random_case(7200, M, N, K)
    scale = np.arange(1, M + 1, dtype=np.float32)
    Q, t = oracle.gemm_q8(M, N, K, case["A"], K, case["B"], K, scale, 3, ldq=ldq)
    _, pre = oracle.gemm(M, N, K, case["A"], K, case["B"], K, return_pre=True)
    assert np.allclose(t, pre * scale[None, :] + 3, rtol=0, atol=1e-12 * (1 + np.abs(t)).max())
    Q2 = Q.reshape(N, ldq)
    assert np.all(Q2[:, M:] == 0)
    for n in range(N):
        for m in range(M):
            assert Q2[n, m] == q8_code_by_hand(Fraction(pre[n, m]), float(scale[m]), 3)


def test_p13_q8_tolerance_hand_cases():
    from tests.tolerance import q8_report
    # exact agreement passes; a code one off passes only next to a boundary
    assert q8_report([3], [3], [3.2], [1.0], 0, 64)["fail"] == 0
    assert q8_report([4], [3], [3.2], [1.0], 0, 64)["fail"] == 1
    assert q8_report([4], [3], [3.4999], [1.0], 0, 64)["fail"] == 0   # delta = 0.008 covers 1e-4
    assert q8_report([5], [3], [3.4999], [1.0], 0, 64)["fail"] == 1
    assert q8_report([0], [0], [np.nan], [1.0], 0, 64)["fail"] == 0
    assert q8_report([1], [0], [np.nan], [1.0], 0, 64)["fail"] == 1


def test_p12_quantize_array_agrees_with_whole_product():
    """The sampled-element form (epilogue values, then codes) reproduces the
    whole-product codes at every coordinate."""
    M, N, K = 40, 30, 50
    case = inputs.random_case(7300, M, N, K, with_c0=True, with_bias=True)
    scale = inputs.uniform_f32(7305, M, 0.25, 4.0)
    Q, t = oracle.gemm_q8(M, N, K, case["A"], K, case["B"], K, scale, -7, C_in=case["C0"], ldc=M, alpha=0.75,
                          beta=0.5, bias=case["bias"], epilogue="gelu_tanh")
    g = np.random.Generator(np.random.PCG64(7306))
    ms, ns = g.integers(0, M, 400), g.integers(0, N, 400)
    _, y = oracle.gemm_elems(M, N, K, case["A"], K, case["B"], K, ms, ns, case["C0"], M, 0.75, 0.5,
                             case["bias"], "gelu_tanh", return_pre=True)
    q2, t2 = oracle.quantize_i8_array(y, scale[ms], -7)
    assert np.array_equal(q2, Q[ms + ns * M]) and np.array_equal(t2, t[ns, ms])


# ------------------------------------------------------ P14-P17 fp8 input ---

def test_p14_fp8_decode_exhaustive_matches_torch():
    bits = np.arange(256, dtype=np.uint16).astype(np.uint8)
    ours = oracle.fp8_to_f64(bits)
    ref = torch.from_numpy(bits.copy()).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan) and nan.sum() == 2     # 0x7F and 0xFF
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))  # -0 at 0x80
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6


@pytest.mark.parametrize("seed", range(10))
def test_p15_fp8_exact_rational_bruteforce_tiny(seed):
    """Tiny fp8 products (random bytes, subnormals included), per-row and
    per-column scales, alpha, beta, bias, ReLU: exact rational result rounded
    by brute force -- bit-identical."""
    g = np.random.Generator(np.random.PCG64(8000 + seed))
    M, N, K = (int(v) for v in g.integers(1, 9, 3))
    lda, ldb = K + int(g.integers(0, 3)), K + int(g.integers(0, 3))
    A = g.integers(0, 256, M * lda).astype(np.uint8)
    B = g.integers(0, 256, N * ldb).astype(np.uint8)
    A[(A & 0x7F) == 0x7F] = 0x3C   # no NaN operands here
    B[(B & 0x7F) == 0x7F] = 0xB4
    sa = (g.random(M) * 2 + 0.25).astype(np.float32)
    sb = (g.random(N) * 2 + 0.25).astype(np.float32)
    C0 = inputs.normal_bf16(8100 + seed, N * M)
    bias = inputs.normal_bf16(8200 + seed, N, scale=0.5)
    alpha, beta = 0.75, -1.5
    epi = ["none", "relu"][seed % 2]
    got = oracle.gemm_fp8(M, N, K, A, lda, B, ldb, C0, M, alpha, beta, sa, sb, bias, epi)
    dA = oracle.fp8_to_f64(A).reshape(M, lda)
    dB = oracle.fp8_to_f64(B).reshape(N, ldb)
    torch_a = torch.from_numpy(A.copy()).view(torch.float8_e4m3fn).double().numpy().reshape(M, lda)
    assert np.array_equal(dA, torch_a)
    c0 = bits_to_f64(C0).reshape(N, M)
    bb = bits_to_f64(bias)
    for n in range(N):
        for m in range(M):
            s = sum(Fraction(dA[m, k]) * Fraction(dB[n, k]) for k in range(K))
            y = Fraction(alpha) * Fraction(float(sa[m])) * Fraction(float(sb[n])) * s
            y += Fraction(beta) * Fraction(c0[n, m]) + Fraction(bb[n])
            if epi == "relu" and y < 0:
                y = Fraction(0)
            want = round_fraction_to_bf16(y)
            assert same_value(got[m + n * M], want), (m, n)


def test_p16_fp8_matches_numpy_float64_matmul():
    M, N, K = 96, 80, 1000
    A = inputs.normal_fp8(8301, M * K)
    B = inputs.normal_fp8(8302, N * K)
    sa = inputs.uniform_f32(8303, M, 0.5, 2.0)
    sb = inputs.uniform_f32(8304, N, 0.5, 2.0)
    _, pre = oracle.gemm_fp8(M, N, K, A, K, B, K, scale_a=sa, scale_b=sb, return_pre=True)
    dA = oracle.fp8_to_f64(A).reshape(M, K)
    dB = oracle.fp8_to_f64(B).reshape(N, K)
    ref = (dA @ dB.T) * sa.astype(np.float64)[:, None] * sb.astype(np.float64)[None, :]
    assert np.max(np.abs(pre.T - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_p17_fp8_identity_and_scale_axes():
    """A = I (fp8 1.0 is 0x38): C[m,n] = sa[m] * sb[n] * B[m,n] exactly after
    rounding (M != N, so swapped scale axes would fail)."""
    M, N = 24, 10
    A = np.zeros(M * M, np.uint8)
    A[np.arange(M) * M + np.arange(M)] = 0x38
    B = inputs.normal_fp8(8401, N * M)
    sa = np.exp2(np.arange(M) % 5 - 2).astype(np.float32)      # powers of two: exact products
    sb = np.exp2(np.arange(N) % 3 - 1).astype(np.float32)
    got = oracle.gemm_fp8(M, N, M, A, M, B, M, scale_a=sa, scale_b=sb).reshape(N, M)
    want = oracle.fp8_to_f64(B).reshape(N, M) * sa[None, :] * sb[:, None]
    assert np.all(same_value(got, oracle.bf16_from_f64(want)))
    assert oracle.fp8_to_f64(np.array([0x38], np.uint8))[0] == 1.0


def test_p16_fp8_elems_agree_with_whole_product():
    M, N, K = 40, 30, 300
    A = inputs.normal_fp8(8501, M * K)
    B = inputs.normal_fp8(8502, N * K)
    sa = inputs.uniform_f32(8503, M, 0.5, 2.0)
    sb = inputs.uniform_f32(8504, N, 0.5, 2.0)
    C0 = inputs.normal_bf16(8505, N * M)
    bias = inputs.normal_bf16(8506, N, scale=0.1)
    full = oracle.gemm_fp8(M, N, K, A, K, B, K, C0, M, 1.5, 0.25, sa, sb, bias, "gelu_tanh")
    g = np.random.Generator(np.random.PCG64(8507))
    ms, ns = g.integers(0, M, 300), g.integers(0, N, 300)
    el = oracle.gemm_fp8_elems(M, N, K, A, K, B, K, ms, ns, C0, M, 1.5, 0.25, sa, sb, bias, "gelu_tanh")
    assert np.array_equal(el, full[ms + ns * M])
