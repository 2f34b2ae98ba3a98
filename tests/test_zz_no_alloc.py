"""gemm_run_noalloc: the entry point that allocates nothing, for callers
that cannot (graph capture, serving loops).  It runs gemm_run's kernels with
the library's own static device scratch in place of a caller workspace, so
its results must equal gemm_run's with a caller workspace bit for bit; two
calls in a row, the second smaller, check that the scratch's leftover
contents from the first do not leak into the second."""
import ctypes

import numpy as np
import pytest
import torch

import gemm_inputs as gi
from _gpu_helpers import check_bf16, dev_bf16, host_values

import dense_gemm_05_amd as g5

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[noalloc] {msg}", flush=True)


@pytest.fixture(autouse=True)
def _no_forced_config(monkeypatch):
    monkeypatch.delenv("GEMM_FORCE_CONFIG", raising=False)
    monkeypatch.delenv("GEMM_FORCE_KSPLIT", raising=False)


def _args(M, N, K, dA, dB, C, batch=1, lda=None, sA=0, sB=0, sC=0):
    return (g5.GEMM_OP_BF16, batch, M, N, K, dA.data_ptr(), K if lda is None else lda, sA, dB.data_ptr(), N, sB,
            C.data_ptr(), N, sC, 0 if C.dtype == torch.bfloat16 else 1, 1.0, None, 0.0, None, None)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _pair(M, N, K, seed, out=torch.bfloat16):
    A, B = gi.small_case("bf16", M, N, K, seed=seed, scale_b=0.125)
    dA, dB = dev_bf16(A), dev_bf16(B)
    C_na = torch.full((M, N), float("nan"), dtype=out, device="cuda")
    C_ws = torch.full((M, N), float("nan"), dtype=out, device="cuda")
    return A, B, dA, dB, C_na, C_ws


@pytest.mark.parametrize("first,second,plan_name", [
    ((1, 12288, 4096), (4, 4096, 2048), b"decode_splitk"),          # split small-M path: partials + counters
    ((1024, 1536, 4096), (512, 512, 4096), b"bf16_128x128"),        # K split over workgroups
])
def test_noalloc_matches_gemm_run_twice(oracle_mod, first, second, plan_name):
    L = g5.lib()
    for i, (M, N, K) in enumerate((first, second)):
        _say(f"{M}x{N}x{K} call {i}")
        st, plan = g5.plan_query(g5.GEMM_OP_BF16, M, N, K)
        assert st == 0 and plan.name == plan_name and 0 < plan.workspace_bytes <= 16 << 20, plan.name
        assert plan_name != b"bf16_128x128" or plan.ksplit > 1
        A, B, dA, dB, C_na, C_ws = _pair(M, N, K, seed=300 + i)
        wsbuf = torch.zeros(plan.workspace_bytes, dtype=torch.uint8, device="cuda")
        st_na = L.gemm_run_noalloc(*_args(M, N, K, dA, dB, C_na), _stream())
        st_ws = L.gemm_run(*_args(M, N, K, dA, dB, C_ws), wsbuf.data_ptr(), wsbuf.numel(), _stream())
        torch.cuda.synchronize()
        assert st_na == 0 and st_ws == 0, (st_na, st_ws)
        assert torch.equal(C_na.view(torch.int16), C_ws.view(torch.int16)), "noalloc result differs from gemm_run"
        check_bf16(host_values(C_na), oracle_mod.gemm_bf16(A, B), K, f"noalloc {M}x{N}x{K}")


def test_noalloc_swiglu_e4m3_matches_gemm_run_twice():
    """The SwiGLU with E4M3FN output through the scratch: the first call's
    small-M plan pairs gate and up workgroups in exchange slots, the second
    (smaller) splits K over four slices with counters and partial sums; the
    codes equal gemm_run's with a caller workspace bit for bit, the range
    travelling in alpha."""
    L = g5.lib()
    amax = 6.0
    for i, (M, N, K, ks) in enumerate(((1, 12288, 4096, 1), (16, 4096, 2048, 4))):
        _say(f"swiglu e4m3 {M}x{N}x{K} call {i}")
        st, plan = g5.plan_query(g5.GEMM_OP_BF16_SWIGLU, M, N, K, c_type=g5.GEMM_OUT_E4M3)
        assert st == 0 and plan.name == b"decode_splitk" and 0 < plan.workspace_bytes <= 16 << 20
        assert plan.grid == (N // 128) * 2 * ks, plan.grid
        g = np.random.default_rng([gi.SEED_BASE + 3800, i])
        X = gi.to_bf16_bits(gi.normal(g, (M, K)))
        Wgu = gi.to_bf16_bits(gi.normal(g, (K, 2 * N), 0.125))
        dX, dW = dev_bf16(X), dev_bf16(Wgu)
        Q_na = torch.full((M, N), 0xAA, dtype=torch.uint8, device="cuda")
        Q_ws = torch.full((M, N), 0x55, dtype=torch.uint8, device="cuda")
        wsbuf = torch.zeros(plan.workspace_bytes, dtype=torch.uint8, device="cuda")
        args = lambda Q: (g5.GEMM_OP_BF16_SWIGLU, 1, M, N, K, dX.data_ptr(), K, 0, dW.data_ptr(), 2 * N, 0,
                          Q.data_ptr(), N, 0, g5.GEMM_OUT_E4M3, amax, None, 0.0, None, None)
        st_na = L.gemm_run_noalloc(*args(Q_na), _stream())
        st_ws = L.gemm_run(*args(Q_ws), wsbuf.data_ptr(), wsbuf.numel(), _stream())
        torch.cuda.synchronize()
        assert st_na == 0 and st_ws == 0, (st_na, st_ws)
        assert torch.equal(Q_na, Q_ws), "noalloc codes differ from gemm_run"
        assert int((Q_na == 0x7e).sum()) + int((Q_na == 0xfe).sum()) > 0   # the range saturates some outputs


def test_noalloc_rejects_calls_beyond_its_scratch():
    """A call whose plan needs more than the 16 MiB of scratch (here a
    realigned copy of 64 MiB of A rows) is refused before anything runs."""
    M, N, K, batch = 2048, 1024, 4100, 4
    st, plan = g5.plan_query(g5.GEMM_OP_BF16, M, N, K, batch=batch, c_type=1, lda=K, sA=M * K)
    assert st == 0 and plan.workspace_bytes > 16 << 20
    dA = torch.zeros((batch, M, K), dtype=torch.bfloat16, device="cuda")
    dB = torch.zeros((batch, K, N), dtype=torch.bfloat16, device="cuda")
    C = torch.full((batch, M, N), 7.0, dtype=torch.float32, device="cuda")
    st = g5.lib().gemm_run_noalloc(*_args(M, N, K, dA, dB, C, batch=batch, sA=M * K, sB=K * N, sC=M * N), _stream())
    torch.cuda.synchronize()
    assert st == g5.GEMM_ERR_WORKSPACE
    assert bool((C == 7.0).all()), "a refused call wrote C"


def test_noalloc_allocates_nothing():
    """Device free memory is unchanged across noalloc calls (after the first
    call on the device has loaded the library's code and scratch)."""
    M, N, K = 1, 12288, 4096
    A, B, dA, dB, C_na, _ = _pair(M, N, K, seed=310)
    L = g5.lib()
    assert L.gemm_run_noalloc(*_args(M, N, K, dA, dB, C_na), _stream()) == 0
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    for _ in range(3):
        assert L.gemm_run_noalloc(*_args(M, N, K, dA, dB, C_na), _stream()) == 0
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0
