"""Concurrent calls through the C ABI: the split-K workspace is one buffer per
(device, stream), allocated by the first split call on a stream and shared
by the calls that stream orders, so split-K calls enqueued on several
streams at once, and from several host threads at once, must each produce
the result a lone call produces (bit for bit: the same kernels add the same
partials in the same order) and stay within the oracle's tolerance.
"""
from __future__ import annotations

import threading

import numpy as np
import pytest

import oracle
from bf16_gemm_fp32_amd import inputs
from tests.tolerance import assert_within_tolerance

torch = pytest.importorskip("torch")
gb = pytest.importorskip("bf16_gemm_fp32_amd")

pytestmark = pytest.mark.gpu

NAN_BF16 = 0x7FC0

# split-K on 128x128 tiles, the streaming kernel's split, and the masked split
SHAPES = [(1024, 1024, 4096, "splitk128x128x64"), (64, 1024, 16384, "skinny"),
          (1000, 1000, 4096, "splitk128x128x64_masked")]


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gb.library()
    yield


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()


def _cases(n):
    out = []
    for i in range(n):
        M, N, K, kernel = SHAPES[i % len(SHAPES)]
        case = inputs.random_case(8100 + i, M, N, K, with_c0=True, with_bias=True)
        out.append((M, N, K, kernel, case, 0.5 if i % 2 else 0.0, "gelu_tanh" if i % 3 == 0 else "none"))
    return out


def _buffers(M, N, K, case, beta):
    """Device copies of a case's operands and a fresh C (C0, or NaN when beta
    is 0); the caller synchronizes before any other stream uses them."""
    A, B, bias = _dev(case["A"]), _dev(case["B"]), _dev(case["bias"])
    C = _dev(case["C0"] if beta != 0.0 else np.full(N * M, NAN_BF16, np.uint16))
    return A, B, bias, C


def _call(M, N, K, bufs, beta, epi, stream_handle):
    A, B, bias, C = bufs
    st = gb.gemm_bf16(M, N, K, A.data_ptr(), K, B.data_ptr(), K, C.data_ptr(), M, 1.0, beta, bias.data_ptr(),
                      gb.EPILOGUES[epi], stream_handle)
    assert st == 0, gb.gemm_bf16_status_string(st)


def _alone(M, N, K, case, beta, epi):
    bufs = _buffers(M, N, K, case, beta)
    torch.cuda.synchronize()
    _call(M, N, K, bufs, beta, epi, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return bufs[3].cpu().numpy().view(np.uint16).copy()


def test_split_calls_on_many_streams_at_once():
    cases = _cases(6)
    for (M, N, K, kernel, *_rest) in cases:
        assert gb.gemm_bf16_kernel_name(M, N, K, 4096, K, 4096, K, 4096, M) == kernel
    want = [_alone(M, N, K, case, beta, epi) for (M, N, K, _, case, beta, epi) in cases]
    streams = [torch.cuda.Stream() for _ in cases]
    for rep in range(3):
        held = [_buffers(M, N, K, case, beta) for (M, N, K, _, case, beta, epi) in cases]
        torch.cuda.synchronize()
        for (M, N, K, _, case, beta, epi), bufs, s in zip(cases, held, streams):
            _call(M, N, K, bufs, beta, epi, s.cuda_stream)
        torch.cuda.synchronize()
        for i, h in enumerate(held):
            got = h[3].cpu().numpy().view(np.uint16)
            assert np.array_equal(got, want[i]), f"stream {i} (rep {rep}) differs from the lone call"
    print(f"[streams] {len(cases)} streams x 3 reps bit-identical to lone calls", flush=True)
    for i, (M, N, K, _, case, beta, epi) in enumerate(cases[:3]):
        ref = oracle.gemm(M, N, K, case["A"], K, case["B"], K, case["C0"], M, 1.0, beta, case["bias"], epi)
        assert_within_tolerance(want[i], ref, K, f"case {i} vs oracle")


def test_split_calls_from_many_threads_at_once():
    cases = _cases(4)
    want = [_alone(M, N, K, case, beta, epi) for (M, N, K, _, case, beta, epi) in cases]
    streams = [torch.cuda.Stream() for _ in cases]
    # four calls per thread, each with its own C; operands ready before any thread starts
    held = [[_buffers(M, N, K, case, beta) for _ in range(4)] for (M, N, K, _, case, beta, epi) in cases]
    torch.cuda.synchronize()
    handles = [s.cuda_stream for s in streams]
    errors = []
    start = threading.Barrier(len(cases))

    def worker(i):
        try:
            M, N, K, _, case, beta, epi = cases[i]
            start.wait()
            for bufs in held[i]:  # ordered on this thread's stream: they share its workspace
                _call(M, N, K, bufs, beta, epi, handles[i])
        except Exception as e:  # reported below
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not errors, errors
    torch.cuda.synchronize()
    for i in range(len(cases)):
        for r, bufs in enumerate(held[i]):
            got = bufs[3].cpu().numpy().view(np.uint16)
            assert np.array_equal(got, want[i]), f"thread {i} call {r} differs from the lone call"
    print(f"[threads] {len(cases)} threads x 4 calls bit-identical to lone calls", flush=True)
