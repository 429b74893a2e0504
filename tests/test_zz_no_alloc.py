"""gemm_bf16_noalloc (split-K scratch in the library's static device array)
against gemm_bf16 (per-stream workspace), through the C ABI.

Both entry points run the same kernels with the same split plans on a
256-CU device, so their outputs must agree bit for bit; both are also held
to the oracle's tolerance.  Two calls in a row, the second on a smaller
input, exercise the array keeping the previous call's contents: split-K
partials are overwritten before they are read, and the streaming kernel's
arrival counters must be back at zero after every call.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from bf16_gemm_fp32_amd import inputs
from tests.tolerance import assert_within_tolerance

torch = pytest.importorskip("torch")
gb = pytest.importorskip("bf16_gemm_fp32_amd")

pytestmark = pytest.mark.gpu

NAN_BF16 = 0x7FC0


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gb.library()
    yield


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()


def _run(entry, M, N, K, case, beta, epi):
    A, B, bias = _dev(case["A"]), _dev(case["B"]), _dev(case["bias"])
    C = _dev(case["C0"] if beta != 0.0 else np.full(N * M, NAN_BF16, np.uint16))
    stream = torch.cuda.current_stream().cuda_stream
    st = entry(M, N, K, A.data_ptr(), K, B.data_ptr(), K, C.data_ptr(), M, 1.0, beta, bias.data_ptr(),
               gb.EPILOGUES[epi], stream)
    assert st == 0, gb.gemm_bf16_status_string(st)
    torch.cuda.synchronize()
    return C.cpu().numpy().view(np.uint16).copy()


# (first call, second smaller call), each (M, N, K, beta, epilogue, expected kernel)
SEQUENCES = [
    [(1024, 1024, 4096, 0.0, "none", "splitk128x128x64"),        # 4 ranges: the whole 16 MiB of partials
     (512, 512, 2048, 0.5, "gelu_tanh", "splitk128x128x64")],
    [(64, 1024, 16384, 0.0, "none", "skinny"),                   # 32 strips x 8 splits: counters + partials
     (48, 512, 8192, -0.5, "relu", "skinny")],
    [(1000, 1000, 4096, 0.5, "gelu_tanh", "splitk128x128x64_masked"),
     (520, 300, 4000, 0.0, "none", "splitk128x128x64_masked")],
    [(2048, 32, 16384, 0.0, "none", "skinny_t"),                 # the transposed product, split in K
     (1000, 40, 8192, 0.5, "relu", "skinny_t")],
]


@pytest.mark.parametrize("seq", SEQUENCES, ids=["tile-split", "streaming-split", "masked-split",
                                                "transposed-split"])
def test_noalloc_matches_gemm_bf16_twice(seq):
    for i, (M, N, K, beta, epi, kernel) in enumerate(seq):
        kname = gb.gemm_bf16_kernel_name(M, N, K, 4096, K, 4096, K, 4096, M)
        print(f"[noalloc] call {i}: {M}x{N}x{K} beta={beta} epi={epi} kernel={kname}", flush=True)
        assert kname == kernel
        case = inputs.random_case(7000 + 10 * i + M, M, N, K, with_c0=True, with_bias=True)
        got = _run(gb.gemm_bf16_noalloc, M, N, K, case, beta, epi)
        want = _run(gb.gemm_bf16, M, N, K, case, beta, epi)
        assert np.array_equal(got, want), "gemm_bf16_noalloc differs from gemm_bf16"
        ref = oracle.gemm(M, N, K, case["A"], K, case["B"], K, case["C0"], M, 1.0, beta, case["bias"], epi)
        assert_within_tolerance(got, ref, K, f"noalloc {M}x{N}x{K}")
        # the static array keeps this call's contents; a repeat must not see them
        again = _run(gb.gemm_bf16_noalloc, M, N, K, case, beta, epi)
        assert np.array_equal(again, got), "a repeated gemm_bf16_noalloc call differs"


@pytest.mark.parametrize("M,N,K,kernel", [
    (1024, 1024, 4096, "splitk128x128x64"),
    (64, 1024, 16384, "skinny"),
    (2048, 32, 16384, "skinny_t"),
    (1000, 1000, 4096, "splitk128x128x64_masked"),
    (4608, 2048, 320, "ring256x256x64"),
])
def test_noalloc_replays_from_a_captured_graph(M, N, K, kernel):
    """A gemm_bf16_noalloc call captured into a HIP graph (stream capture
    through torch.cuda.graph) replays to the eager call's result bit for bit,
    replay after replay, with eager work and a synchronisation between
    replays: the split paths clear what they count in-kernel, so nothing in
    the graph depends on state a previous replay left behind."""
    assert gb.gemm_bf16_kernel_name(M, N, K, 4096, K, 4096, K, 4096, M) == kernel
    case = inputs.random_case(9100 + M + N, M, N, K, with_c0=True, with_bias=True)
    A, B, bias, C0 = _dev(case["A"]), _dev(case["B"]), _dev(case["bias"]), _dev(case["C0"])
    C = C0.clone()

    def call():
        st = gb.gemm_bf16_noalloc(M, N, K, A.data_ptr(), K, B.data_ptr(), K, C.data_ptr(), M, 1.25, 0.5,
                                  bias.data_ptr(), gb.EPILOGUES["gelu_tanh"], torch.cuda.current_stream().cuda_stream)
        assert st == 0, gb.gemm_bf16_status_string(st)

    print(f"[noalloc-graph] {M}x{N}x{K} kernel={kernel}", flush=True)
    call()  # eager: the reference, and the device's one-time set-up outside the capture
    torch.cuda.synchronize()
    want = C.cpu().numpy().view(np.uint16).copy()
    ref = oracle.gemm(M, N, K, case["A"], K, case["B"], K, case["C0"], M, 1.25, 0.5, case["bias"], "gelu_tanh")
    assert_within_tolerance(want, ref, K, f"eager {M}x{N}x{K}")
    C.copy_(C0)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for r in range(3):
        C.copy_(C0)  # beta != 0: every replay starts from C0 again
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = C.cpu().numpy().view(np.uint16)
        assert np.array_equal(got, want), f"replay {r} differs from the eager call"
