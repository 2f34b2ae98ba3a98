"""GPU parity of the transposed-A ("TN") entry points, gemm_bf16_tn and
gemm_bf16_tn_batched, against the oracle, through the C ABI.

A is given as At [K, M]; the oracle multiplies by the plain definition
C[i][j] = sum_k A[i][k] B[k][j] with A = At^T materialised on the host.
The full-size case is the weight gradient of the FFN projection,
dW = X^T . dY, whose X is stored [tokens, features] as the forward pass
wrote it.
"""
import numpy as np
import pytest
import torch

import gemm_inputs as gi
from _gpu_helpers import amax_bf16, check_bf16, check_f32, dev_bf16, host_values, ws

import dense_gemm_05_amd as g5

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[tn] {msg}", flush=True)


@pytest.fixture(autouse=True)
def _no_forced_config(monkeypatch):
    monkeypatch.delenv("GEMM_FORCE_CONFIG", raising=False)
    monkeypatch.delenv("GEMM_FORCE_KSPLIT", raising=False)


def _case(M, N, K, pa, pb, seed, batch=None):
    g = np.random.default_rng([gi.SEED_BASE + 7000 + seed, M, N, K, pa, pb])
    shp = (lambda *s: s) if batch is None else (lambda *s: (batch,) + s)
    At = gi.to_bf16_bits(gi.normal(g, shp(K, M + pa)))
    B = gi.to_bf16_bits(gi.normal(g, shp(K, N + pb), 0.125))
    return At, B


def _ref(oracle_mod, At, B, M, N):
    return oracle_mod.gemm_bf16(np.ascontiguousarray(At[:, :M].T), np.ascontiguousarray(B[:, :N]))


@pytest.mark.parametrize("cfg", [None, "bf16_256x192", "bf16_256x256", "bf16_128x128"])
@pytest.mark.parametrize("M,N,K,pa,pb", [
    (300, 392, 262, 4, 8),      # M % 8 != 0 (At rows realigned, zero padded), K tail of 6
    (304, 392, 264, 8, 8),      # 16-byte rows with padded strides, partial tiles
    (264, 200, 1000, 0, 0),     # K tail of 8
    (512, 384, 128, 0, 0),      # whole tiles (aligned variant for 128x128)
    (17, 136, 96, 3, 0),        # small M on the tiled kernel, rows 2-byte aligned: realigned
])
def test_tn_ragged(oracle_mod, monkeypatch, cfg, M, N, K, pa, pb):
    """Every ring config with the transposed A (forced) and the selector's
    choice, FP32 and bf16 output; NaN in the ldc padding shows any stray
    write."""
    _say(f"tn {cfg} {M}x{N}x{K} pad {pa},{pb}")
    At, B = _case(M, N, K, pa, pb, 1)
    dA, dB = dev_bf16(At), dev_bf16(B)
    if cfg:
        monkeypatch.setenv("GEMM_FORCE_CONFIG", cfg)
    ref = _ref(oracle_mod, At, B, M, N)
    for od in (torch.float32, torch.bfloat16):
        Cfull = torch.full((M, N + 5), float("nan"), device="cuda", dtype=od)
        g5.gemm_bf16_tn(dA[:, :M], dB[:, :N], Cfull[:, :N], workspace=ws())
        host = host_values(Cfull)
        if od == torch.bfloat16:
            check_bf16(host[:, :N], ref, K, f"tn {cfg} bf16")
        else:
            check_f32(host[:, :N], ref, K, amax_bf16(At[:, :M]), amax_bf16(B[:, :N]), f"tn {cfg} f32")
        assert np.all(np.isnan(host[:, N:])), "ldc padding was written"


@pytest.mark.parametrize("S", [2, 3, 5])
def test_tn_ksplit(oracle_mod, monkeypatch, S):
    _say(f"tn ksplit {S}")
    M, N, K = 200, 264, 1000
    At, B = _case(M, N, K, 8, 8, 2)
    monkeypatch.setenv("GEMM_FORCE_CONFIG", "bf16_128x128")
    monkeypatch.setenv("GEMM_FORCE_KSPLIT", str(S))
    st, plan = g5.plan_query(g5.GEMM_OP_BF16_TN, M, N, K, lda=M + 8, ldb=N + 8, c_type=1)
    assert st == 0 and plan.ksplit == S
    C = g5.gemm_bf16_tn(dev_bf16(At)[:, :M], dev_bf16(B)[:, :N], out_dtype=torch.float32, workspace=ws())
    check_f32(host_values(C), _ref(oracle_mod, At, B, M, N), K, amax_bf16(At[:, :M]), amax_bf16(B[:, :N]),
              f"tn split {S}")


@pytest.mark.parametrize("cfg", ["bf16_256x192", "bf16_256x256", "bf16_128x128"])
def test_tn_matches_nn_bitwise(monkeypatch, cfg):
    """The same product through gemm_bf16 (A = At^T materialised) and
    gemm_bf16_tn gives the same bits on the same configuration: the
    transposing read hands the matrix core the same A fragments."""
    At, B = _case(512, 576, 640, 0, 0, 3)
    dAt, dB = dev_bf16(At), dev_bf16(B)
    dA = dAt.t().contiguous()
    monkeypatch.setenv("GEMM_FORCE_CONFIG", cfg)
    monkeypatch.setenv("GEMM_FORCE_KSPLIT", "1")
    c1 = g5.gemm_bf16(dA, dB, out_dtype=torch.float32, workspace=ws())
    c2 = g5.gemm_bf16_tn(dAt, dB, out_dtype=torch.float32, workspace=ws())
    assert torch.equal(c1.view(torch.int32), c2.view(torch.int32))


def test_tn_batched_broadcast(oracle_mod):
    """Batched entries with their own At and one shared B (batch stride 0)."""
    _say("tn batched")
    At, B = _case(136, 200, 300, 0, 0, 4, batch=3)
    dB = dev_bf16(B[0]).unsqueeze(0).expand(3, -1, -1)
    C = g5.gemm_bf16_tn_batched(dev_bf16(At), dB, out_dtype=torch.float32, workspace=ws())
    host = host_values(C)
    for b in range(3):
        ref = oracle_mod.gemm_bf16(np.ascontiguousarray(At[b].T), B[0])
        check_f32(host[b], ref, 300, amax_bf16(At[b]), amax_bf16(B[0]), f"tn batched {b}")


def test_tn_k_zero():
    C = torch.full((40, 64), float("nan"), device="cuda", dtype=torch.bfloat16)
    At = torch.zeros((0, 40), device="cuda", dtype=torch.bfloat16)
    B = torch.zeros((0, 64), device="cuda", dtype=torch.bfloat16)
    g5.gemm_bf16_tn(At, B, C, workspace=ws())
    assert torch.all(C == 0)


def test_tn_weight_gradient_full_size(oracle_mod):
    """dW [4096, 12288] = X^T . dY with X [1024, 4096] and dY [1024, 12288]
    (K = 1024 tokens): rows from every row tile, all columns."""
    _say("wgrad TN 4096x12288x1024")
    X, dY = gi.wgrad_inputs()
    st, plan = g5.plan_query(g5.GEMM_OP_BF16_TN, 4096, 12288, 1024)
    assert st == 0 and plan.variant == 1 and plan.workspace_bytes == 0
    C = g5.gemm_bf16_tn(dev_bf16(X), dev_bf16(dY), workspace=ws())
    rows = np.array([0, 1, 255, 256, 2047, 3000, 4095])
    ref = oracle_mod.gemm_bf16(np.ascontiguousarray(X[:, rows].T), dY)
    check_bf16(host_values(C)[rows], ref, 1024, "wgrad rows")
