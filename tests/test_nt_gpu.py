"""GPU parity of the transposed-B ("NT") entry points, gemm_bf16_nt and
gemm_bf16_nt_batched, against the oracle, through the C ABI.

B is given as Bt [N, K]; the oracle multiplies by the plain definition with
B = Bt^T materialised on the host.  The batched form is the attention-score
product Q . K^T of the multi-head attention case (page "4.1 Tối ưu hiệu năng
toán tử GEMM trên CUDA", §1.2) with K row-major, as attention stores it.
"""
import numpy as np
import pytest
import torch

import gemm_inputs as gi
from _gpu_helpers import amax_bf16, check_bf16, check_f32, dev_bf16, host_values, ws

import dense_gemm_05_amd as g5

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[nt] {msg}", flush=True)


@pytest.fixture(autouse=True)
def _no_forced_config(monkeypatch):
    monkeypatch.delenv("GEMM_FORCE_CONFIG", raising=False)
    monkeypatch.delenv("GEMM_FORCE_KSPLIT", raising=False)


def _case(M, N, K, pa, pb, seed, batch=None):
    g = np.random.default_rng([gi.SEED_BASE + 6000 + seed, M, N, K, pa, pb])
    shp = (lambda *s: s) if batch is None else (lambda *s: (batch,) + s)
    A = gi.to_bf16_bits(gi.normal(g, shp(M, K + pa)))
    Bt = gi.to_bf16_bits(gi.normal(g, shp(N, K + pb), 0.125))
    return A, Bt


def _ref(oracle_mod, A, Bt, K):
    return oracle_mod.gemm_bf16(np.ascontiguousarray(A[:, :K]), np.ascontiguousarray(Bt[:, :K].T))


@pytest.mark.parametrize("cfg", [None, "bf16_256x192", "bf16_256x256", "bf16_256x128", "bf16_128x128"])
@pytest.mark.parametrize("M,N,K,pa,pb", [
    (300, 392, 262, 0, 0),      # 4-byte A copies; Bt rows 4-byte aligned: realigned
    (300, 392, 264, 8, 8),      # 16-byte rows, padded strides
    (257, 190, 1000, 8, 8),     # N not a multiple of 8, K tail of 8
    (512, 384, 128, 0, 0),      # whole tiles (aligned variant for 128x128)
])
def test_nt_ragged(oracle_mod, monkeypatch, cfg, M, N, K, pa, pb):
    """Every ring config (forced) and the selector's choice, FP32 and bf16
    output; NaN in the ldc padding shows any stray write."""
    _say(f"nt {cfg} {M}x{N}x{K} pad {pa},{pb}")
    A, Bt = _case(M, N, K, pa, pb, 1)
    dA, dB = dev_bf16(A), dev_bf16(Bt)
    if cfg:
        monkeypatch.setenv("GEMM_FORCE_CONFIG", cfg)
    ref = _ref(oracle_mod, A, Bt, K)
    for od in (torch.float32, torch.bfloat16):
        Cfull = torch.full((M, N + 5), float("nan"), device="cuda", dtype=od)
        g5.gemm_bf16_nt(dA[:, :K], dB[:, :K], Cfull[:, :N], workspace=ws())
        host = host_values(Cfull)
        if od == torch.bfloat16:
            check_bf16(host[:, :N], ref, K, f"nt {cfg} bf16")
        else:
            check_f32(host[:, :N], ref, K, amax_bf16(A[:, :K]), amax_bf16(Bt[:, :K]), f"nt {cfg} f32")
        assert np.all(np.isnan(host[:, N:])), "ldc padding was written"


@pytest.mark.parametrize("S", [2, 3, 5])
def test_nt_ksplit(oracle_mod, monkeypatch, S):
    _say(f"nt ksplit {S}")
    M, N, K = 200, 264, 1000
    A, Bt = _case(M, N, K, 8, 8, 2)
    monkeypatch.setenv("GEMM_FORCE_CONFIG", "bf16_128x128")
    monkeypatch.setenv("GEMM_FORCE_KSPLIT", str(S))
    C = g5.gemm_bf16_nt(dev_bf16(A)[:, :K], dev_bf16(Bt)[:, :K], out_dtype=torch.float32, workspace=ws())
    check_f32(host_values(C), _ref(oracle_mod, A, Bt, K), K, amax_bf16(A[:, :K]), amax_bf16(Bt[:, :K]),
              f"nt split {S}")


def test_nt_matches_nn_bitwise():
    """The same product through gemm_bf16 (B = Bt^T materialised) and
    gemm_bf16_nt gives the same bits: same tiles, same MFMA order."""
    A, Bt = _case(512, 576, 640, 0, 0, 3)
    dA, dBt = dev_bf16(A), dev_bf16(Bt)
    dB = dBt.t().contiguous()
    c1 = g5.gemm_bf16(dA, dB, out_dtype=torch.float32, workspace=ws())
    c2 = g5.gemm_bf16_nt(dA, dBt, out_dtype=torch.float32, workspace=ws())
    assert torch.equal(c1.view(torch.int32), c2.view(torch.int32))


def test_attention_scores_nt_full_size(oracle_mod):
    """32 x (Q[1024,128] . K^T) with K [32,1024,128] row-major (no
    transposed copy), FP32 out: 4 entries in full, sampled rows of all."""
    _say("attention scores NT 32x1024x1024x128")
    Q, KT = gi.batched_inputs()
    Km = np.ascontiguousarray(np.transpose(KT, (0, 2, 1)))      # [32, 1024, 128], as drawn
    st, plan = g5.plan_query(g5.GEMM_OP_BF16_NT, 1024, 1024, 128, batch=32, c_type=1)
    assert st == 0 and plan.name == b"bf16_128x128" and plan.variant == 1 and plan.workspace_bytes == 0
    C = g5.gemm_bf16_nt_batched(dev_bf16(Q), dev_bf16(Km), out_dtype=torch.float32, workspace=ws())
    host = host_values(C)
    for b in (0, 5, 31):
        ref = oracle_mod.gemm_bf16(Q[b], KT[b])
        check_f32(host[b], ref, 128, amax_bf16(Q[b]), amax_bf16(KT[b]), f"scores entry {b}")
    rows = np.array([0, 127, 128, 600, 1023])
    for b in range(32):
        ref = oracle_mod.gemm_bf16(np.ascontiguousarray(Q[b][rows]), KT[b])
        check_f32(host[b][rows], ref, 128, amax_bf16(Q[b]), amax_bf16(KT[b]), f"scores {b} rows")


def test_nt_linear_weight_full_size(oracle_mod):
    """The FFN projection with its weight stored as a linear layer's
    [12288, 4096]: sampled rows, all columns."""
    _say("FFN NT 1024x12288x4096")
    X, W = gi.ffn_inputs()
    Wt = np.ascontiguousarray(W.T)
    st, plan = g5.plan_query(g5.GEMM_OP_BF16_NT, 1024, 12288, 4096)
    assert st == 0 and plan.name == b"bf16_256x192" and plan.variant == 1
    C = g5.gemm_bf16_nt(dev_bf16(X), dev_bf16(Wt), workspace=ws())
    rows = np.array([0, 255, 256, 511, 700, 1023])
    ref = oracle_mod.gemm_bf16(np.ascontiguousarray(X[rows]), W)
    check_bf16(host_values(C)[rows], ref, 4096, "FFN NT rows")


@pytest.mark.parametrize("M,N,K,batch", [(1, 12288, 4096, 1), (4, 1000, 1000, 1), (16, 264, 4104, 1), (7, 100, 72, 3),
                                         (3, 40, 8, 1)])
def test_nt_small_m(oracle_mod, M, N, K, batch):
    """Small M with B transposed runs as a GEMV over the rows of Bt
    (decode_nt): ragged N, K tails (K % 32 != 0), batched, both outputs."""
    _say(f"nt small-M {batch}x{M}x{N}x{K}")
    st, plan = g5.plan_query(g5.GEMM_OP_BF16_NT, M, N, K, batch=batch)
    assert st == 0 and plan.name == b"decode_nt"
    g = np.random.default_rng([gi.SEED_BASE + 6100, M, N, K, batch])
    A = gi.to_bf16_bits(gi.normal(g, (batch, M, K)))
    Bt = gi.to_bf16_bits(gi.normal(g, (batch, N, K), 0.125))
    for od in (torch.float32, torch.bfloat16):
        Cfull = torch.full((batch, M, N + 3), float("nan"), device="cuda", dtype=od)
        if batch == 1:
            g5.gemm_bf16_nt(dev_bf16(A[0]), dev_bf16(Bt[0]), Cfull[0, :, :N], workspace=ws())
        else:
            g5.gemm_bf16_nt_batched(dev_bf16(A), dev_bf16(Bt), Cfull[:, :, :N], workspace=ws())
        host = host_values(Cfull)
        for b in range(batch):
            ref = oracle_mod.gemm_bf16(A[b], np.ascontiguousarray(Bt[b].T))
            if od == torch.bfloat16:
                check_bf16(host[b, :, :N], ref, K, f"nt small-M bf16 {b}")
            else:
                check_f32(host[b, :, :N], ref, K, amax_bf16(A[b]), amax_bf16(Bt[b]), f"nt small-M f32 {b}")
        assert np.all(np.isnan(host[:, :, N:])), "ldc padding was written"


def test_nt_small_m_batch_invariance():
    """Rows of an M = 1, 4, 9 call equal the same rows of an M = 16 call bit
    for bit (the K partition does not depend on M)."""
    X, W = gi.decode_inputs(16)
    dW = dev_bf16(np.ascontiguousarray(W.T))
    dX = dev_bf16(X)
    c16 = g5.gemm_bf16_nt(dX, dW, workspace=ws()).view(torch.int16)
    for M in (1, 4, 9):
        cm = g5.gemm_bf16_nt(dX[:M], dW, workspace=ws()).view(torch.int16)
        assert torch.equal(cm, c16[:M]), f"M={M} differs from the M=16 rows"
