"""GPU parity: the HIP kernels, called through the C ABI, against the FP64
CPU oracle on the same seeded inputs.

Bars (written here, per element):
  FP32:                     max |C - C_ref| <= 1e-5 * K * max|a| * max|b|
  BF16 output:              |C - C_ref| <= 2^-8 |C_ref| + 1e-3 sqrt(K)
  FP32 output, bf16 inputs: the FP32 bar with max|a|, max|b| of that entry's
                            bf16 inputs
C_ref is the oracle's unrounded double result.
"""
import math
import os

import numpy as np
import pytest
import torch

import gemm_inputs as gi
from _gpu_helpers import (ws, amax_bf16, check_bf16, check_f32, dev_bf16, dev_f32, host_bits,
                                host_values)

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import dense_gemm_05_amd as g5


def _say(msg):
    print(f"[parity] {msg}", flush=True)


@pytest.fixture(autouse=True)
def _no_forced_config(monkeypatch):
    monkeypatch.delenv("GEMM_FORCE_CONFIG", raising=False)


# ---------------------------------------------------------------- FP32

def test_sgemm_256_cube(oracle_mod):
    _say("sgemm 256^3")
    A, B = gi.sgemm_inputs(256)
    C = g5.gemm_sgemm(dev_f32(A), dev_f32(B))
    torch.cuda.synchronize()
    ref = oracle_mod.gemm_f32(A, B)
    check_f32(host_values(C), ref, 256, np.abs(A).max(), np.abs(B).max(), "sgemm 256^3")


SHAPES = [(1, 1, 1), (7, 9, 5), (16, 16, 16), (17, 33, 65), (64, 64, 64), (65, 127, 129),
          (127, 65, 33), (129, 257, 255), (255, 129, 31), (300, 200, 100), (3, 500, 1000)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_sgemm_ragged(oracle_mod, M, N, K):
    _say(f"sgemm {M}x{N}x{K}")
    A, B = gi.small_case("f32", M, N, K)
    C = g5.gemm_sgemm(dev_f32(A), dev_f32(B))
    ref = oracle_mod.gemm_f32(A, B)
    check_f32(host_values(C), ref, K, np.abs(A).max(), np.abs(B).max(), f"sgemm {M}x{N}x{K}")


def test_sgemm_padded_strides(oracle_mod):
    """lda > K, ldb > N, ldc > N (views into wider buffers)."""
    M, N, K = 70, 90, 110
    g = np.random.default_rng(31)
    Aw = gi.uniform_pm1(g, (M, K + 10))
    Bw = gi.uniform_pm1(g, (K, N + 7))
    dA, dB = dev_f32(Aw), dev_f32(Bw)
    Cfull = torch.full((M, N + 13), float("nan"), device="cuda")
    g5.gemm_sgemm(dA[:, :K], dB[:, :N], Cfull[:, :N])
    ref = oracle_mod.gemm_f32(Aw[:, :K], Bw[:, :N])
    host = host_values(Cfull)
    check_f32(host[:, :N], ref, K, np.abs(Aw[:, :K]).max(), np.abs(Bw[:, :N]).max(), "sgemm padded")
    assert np.all(np.isnan(host[:, N:])), "ldc padding was written"


def test_sgemm_4096_full(oracle_mod):
    """The 4096^3 workload at full size, in the launch configuration the
    benchmark times; every element against the oracle."""
    _say("sgemm 4096^3 (every element)")
    A, B = gi.sgemm_inputs(4096, workload=gi.W_SGEMM_LARGE)
    C = g5.gemm_sgemm(dev_f32(A), dev_f32(B))
    ref = oracle_mod.gemm_f32(A, B)
    check_f32(host_values(C), ref, 4096, np.abs(A).max(), np.abs(B).max(), "sgemm 4096")


# ---------------------------------------------------------------- BF16

BF16_SHAPES = [(17, 33, 65), (20, 8, 3), (33, 190, 7), (64, 64, 64), (129, 257, 255), (256, 192, 64),
               (257, 193, 130), (300, 385, 129), (512, 384, 128), (100, 1000, 77), (1, 300, 100),
               (5, 77, 1000), (16, 129, 64), (16, 64, 4100)]


@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("M,N,K", BF16_SHAPES)
def test_bf16_ragged(oracle_mod, M, N, K, out):
    _say(f"bf16 {M}x{N}x{K} -> {out}")
    A, B = gi.small_case("bf16", M, N, K, seed=1, scale_b=0.125)
    od = torch.bfloat16 if out == "bf16" else torch.float32
    C = g5.gemm_bf16(dev_bf16(A), dev_bf16(B), out_dtype=od, workspace=ws())
    ref = oracle_mod.gemm_bf16(A, B)
    if out == "bf16":
        check_bf16(host_values(C), ref, K, f"bf16 {M}x{N}x{K}")
    else:
        check_f32(host_values(C), ref, K, amax_bf16(A), amax_bf16(B), f"bf16->f32 {M}x{N}x{K}")


@pytest.mark.parametrize("cfg", ["bf16_256x192", "bf16_128x128", "bf16_256x128", "bf16_256x256", "generic",
                                 "decode_64"])
def test_bf16_every_config(oracle_mod, monkeypatch, cfg):
    """Each compiled configuration, forced, on a ragged problem with padded
    strides and odd K (misaligned rows)."""
    M = 16 if cfg == "decode_64" else 300
    N, K = 390, 261
    _say(f"bf16 forced {cfg} {M}x{N}x{K}")
    A, B = gi.small_case("bf16", M, N + 5, K + 3, seed=6, scale_b=0.125)
    dA, dB = dev_bf16(A), dev_bf16(B)
    monkeypatch.setenv("GEMM_FORCE_CONFIG", cfg)
    for od in (torch.bfloat16, torch.float32):
        Cfull = torch.full((M, N + 7), float("nan"), device="cuda", dtype=od)
        g5.gemm_bf16(dA[:, :K], dB[:K, :N], Cfull[:, :N], workspace=ws())
        ref = oracle_mod.gemm_bf16(np.ascontiguousarray(A[:, :K]), np.ascontiguousarray(B[:K, :N]))
        host = host_values(Cfull)
        if od == torch.bfloat16:
            check_bf16(host[:, :N], ref, K, f"{cfg} bf16")
        else:
            check_f32(host[:, :N], ref, K, amax_bf16(A[:, :K]), amax_bf16(B[:K, :N]), f"{cfg} f32")
        assert np.all(np.isnan(host[:, N:])), f"{cfg}: ldc padding was written"


@pytest.mark.parametrize("cfg", ["f32_128x128", "f32_64x64", "generic"])
def test_sgemm_every_config(oracle_mod, monkeypatch, cfg):
    M, N, K = 150, 170, 190
    A, B = gi.small_case("f32", M, N, K, seed=8)
    monkeypatch.setenv("GEMM_FORCE_CONFIG", cfg)
    C = g5.gemm_sgemm(dev_f32(A), dev_f32(B))
    ref = oracle_mod.gemm_f32(A, B)
    check_f32(host_values(C), ref, K, np.abs(A).max(), np.abs(B).max(), cfg)


@pytest.mark.parametrize("M,N,K,pad", [(256, 256, 256, 0), (64, 96, 32, 0), (96, 32, 224, 4), (320, 128, 160, 8)])
def test_sgemm_whole_k(oracle_mod, M, N, K, pad):
    """The whole-K FP32 kernel (all slabs staged before the first MFMA) on
    1 to 8 slabs; padded rows of A, B and C hold NaN, so a read past K or N
    or a write past N shows."""
    _say(f"sgemm whole-K {M}x{N}x{K} pad {pad}")
    A, B = gi.small_case("f32", M, N, K, seed=K + pad)
    Aw = np.full((M, K + pad), np.nan, np.float32)
    Bw = np.full((K, N + pad), np.nan, np.float32)
    Aw[:, :K], Bw[:, :N] = A, B
    dA, dB = dev_f32(Aw), dev_f32(Bw)
    Cfull = torch.full((M, N + pad), float("nan"), device="cuda", dtype=torch.float32)
    st, plan = g5.plan_query(g5.GEMM_OP_SGEMM, M, N, K, lda=K + pad, ldb=N + pad, ldc=N + pad,
                             a_addr=dA.data_ptr(), b_addr=dB.data_ptr(), c_addr=Cfull.data_ptr())
    assert st == 0 and plan.name == b"f32_32x32_wholek", plan.name
    g5.gemm_sgemm(dA[:, :K], dB[:, :N], Cfull[:, :N])
    host = host_values(Cfull)
    check_f32(host[:, :N], oracle_mod.gemm_f32(A, B), K, np.abs(A).max(), np.abs(B).max(), "sgemm whole-K")
    if pad:
        assert np.all(np.isnan(host[:, N:])), "ldc padding was written"


@pytest.mark.parametrize("with_ws", [True, False])
def test_ffn_projection_full_size(oracle_mod, with_ws):
    """X[1024,4096] . W[4096,12288] -> bf16, the benchmarked launch (through
    gemm_run with a workspace) and the named call without one; every element
    against the oracle."""
    _say(f"FFN 1024x12288x4096 workspace={with_ws}")
    X, W = gi.ffn_inputs()
    C = g5.gemm_bf16(dev_bf16(X), dev_bf16(W), workspace=ws() if with_ws else None)
    ref = oracle_mod.gemm_bf16(X, W)
    check_bf16(host_values(C), ref, 4096, "FFN")


@pytest.mark.parametrize("M,N,K,cfg", [(4096, 4096, 4096, b"bf16_256x256"), (2048, 2048, 8192, b"bf16_128x128")])
def test_large_bf16_products(oracle_mod, M, N, K, cfg):
    """Large bf16 products on the tile shapes the selector gives them
    (256x256 tiles for a 4096^3 product, 128x128 tiles for an output too
    small to fill the CUs with large tiles); every element."""
    _say(f"bf16 {M}x{N}x{K} ({cfg.decode()})")
    st, plan = g5.plan_query(g5.GEMM_OP_BF16, M, N, K)
    assert st == 0 and plan.name == cfg, plan.name
    g = np.random.default_rng(M + N + K)
    A = gi.to_bf16_bits(gi.normal(g, (M, K)))
    B = gi.to_bf16_bits(gi.normal(g, (K, N), 0.125))
    C = g5.gemm_bf16(dev_bf16(A), dev_bf16(B), workspace=ws())
    ref = oracle_mod.gemm_bf16(A, B)
    check_bf16(host_values(C), ref, K, f"bf16 {M}x{N}x{K}")


@pytest.mark.parametrize("with_ws", [True, False])
@pytest.mark.parametrize("M", [1, 4, 16])
def test_decode_full_size(oracle_mod, M, with_ws):
    """Decode shapes at full size, with a workspace (the split small-M path)
    and without (whole K per workgroup): every element."""
    _say(f"decode M={M} workspace={with_ws}")
    X, W = gi.decode_inputs(M)
    C = g5.gemm_bf16(dev_bf16(X), dev_bf16(W), workspace=ws() if with_ws else None)
    ref = oracle_mod.gemm_bf16(X, W)
    check_bf16(host_values(C), ref, 4096, f"decode M={M}")


@pytest.mark.parametrize("with_ws", [True, False])
@pytest.mark.parametrize("M", [1, 16])
def test_decode_one_slice_direct(oracle_mod, M, with_ws):
    """Decode rows against a weight with 192 strips of 128 columns (the
    merged gate|up weight [4096, 24576]): one workgroup per strip over all
    of K, stored directly with or without a workspace; every element."""
    N, K = 24576, 4096
    st, plan = g5.plan_query(g5.GEMM_OP_BF16, M, N, K, with_workspace=with_ws)
    assert st == 0 and plan.name == b"decode_splitk" and plan.grid == 192 and plan.workspace_bytes == 0
    _say(f"decode one slice M={M} N={N} workspace={with_ws}")
    X, Wgu = gi.swiglu_inputs(16, K, N // 2)
    X = np.ascontiguousarray(X[:M])
    C = g5.gemm_bf16(dev_bf16(X), dev_bf16(Wgu), workspace=ws() if with_ws else None)
    ref = oracle_mod.gemm_bf16(X, Wgu)
    check_bf16(host_values(C), ref, K, f"decode one slice M={M}")


@pytest.mark.parametrize("cfg", ["decode_64"])
@pytest.mark.parametrize("M,N,K,batch", [(7, 1000, 1000, 1), (1, 512, 4096, 1), (16, 1536, 520, 1),
                                         (4, 1000, 264, 3), (3, 2048, 24, 1), (5, 130, 31, 2)])
def test_decode_paths_ragged(oracle_mod, monkeypatch, cfg, M, N, K, batch):
    """The small-M kernel on N that is not a whole number of column chunks,
    K with a remainder (and K < 32), odd strides, and a batch."""
    _say(f"{cfg} batch={batch} {M}x{N}x{K}")
    g = np.random.default_rng([M, N, K, batch])
    A = gi.to_bf16_bits(gi.normal(g, (batch, M, K)))
    B = gi.to_bf16_bits(gi.normal(g, (batch, K, N), 0.125))
    monkeypatch.setenv("GEMM_FORCE_CONFIG", cfg)
    st, plan = g5.plan_query(g5.GEMM_OP_BF16, M, N, K, batch=batch)
    assert st == 0 and plan.name.decode() == cfg
    for od in (torch.bfloat16, torch.float32):
        C = g5.gemm_bf16_batched(dev_bf16(A), dev_bf16(B), out_dtype=od, workspace=ws())
        host = host_values(C)
        for b in range(batch):
            ref = oracle_mod.gemm_bf16(A[b], B[b])
            if od == torch.bfloat16:
                check_bf16(host[b], ref, K, f"{cfg} bf16 batch {b}")
            else:
                check_f32(host[b], ref, K, amax_bf16(A[b]), amax_bf16(B[b]), f"{cfg} f32 batch {b}")


@pytest.mark.parametrize("M,N,K,batch", [(1, 512, 4096, 1), (7, 1280, 1024, 1), (16, 384, 96, 3),
                                         (4, 256, 8192, 1), (3, 12288, 4096, 1), (5, 1664, 4160, 1),
                                         (9, 1024, 1024, 5)])
def test_decode_split_k(oracle_mod, monkeypatch, M, N, K, batch):
    """The split small-M path: 1, 2 and 8 K slices per strip, slices of
    unequal length, batches; two calls in a row, so the second runs on the
    counters the first left."""
    _say(f"decode_splitk {M}x{N}x{K} batch {batch}")
    monkeypatch.setenv("GEMM_FORCE_CONFIG", "decode_splitk")
    g = np.random.default_rng([M, N, K, batch, 5])
    X = gi.to_bf16_bits(gi.normal(g, (batch, M, K)))
    W = gi.to_bf16_bits(gi.normal(g, (batch, K, N), 0.125))
    dX, dW = dev_bf16(X), dev_bf16(W)
    for rep in range(2):
        C = g5.gemm_bf16_batched(dX, dW, out_dtype=torch.float32 if rep else torch.bfloat16, workspace=ws())
        host = host_values(C)
        for b in range(batch):
            ref = oracle_mod.gemm_bf16(X[b], W[b])
            if rep:
                check_f32(host[b], ref, K, amax_bf16(X[b]), amax_bf16(W[b]), f"splitk f32 b{b}")
            else:
                check_bf16(host[b], ref, K, f"splitk bf16 b{b}")


def test_decode_split_k_back_to_back(oracle_mod):
    """Twenty consecutive calls of the split path with fresh inputs each time,
    queued without synchronisation: every result must come from its own
    call's partial sums (a stale partial would show as a mismatch)."""
    _say("decode_splitk x20 back to back")
    M, N, K = 2, 2048, 2048
    g = np.random.default_rng(77)
    Xs = [gi.to_bf16_bits(gi.normal(g, (M, K))) for _ in range(20)]
    W = gi.to_bf16_bits(gi.normal(g, (K, N), 0.125))
    dW = dev_bf16(W)
    st, plan = g5.plan_query(g5.GEMM_OP_BF16, M, N, K)
    assert plan.name == b"decode_splitk" and plan.grid == 16 * 4
    outs = [g5.gemm_bf16(dev_bf16(X), dW, out_dtype=torch.float32, workspace=ws()) for X in Xs]
    for i, (X, C) in enumerate(zip(Xs, outs)):
        ref = oracle_mod.gemm_bf16(X, W)
        check_f32(host_values(C), ref, K, amax_bf16(X), amax_bf16(W), f"call {i}")


def test_decode_batch_invariance():
    """Rows of the M=1 and M=4 results equal the matching rows of M=16 bit for
    bit: the K split does not depend on M ("Operator & Runtime" §5.2.4)."""
    X16, W = gi.decode_inputs(16)
    dW = dev_bf16(W)
    C16 = host_bits(g5.gemm_bf16(dev_bf16(X16), dW, workspace=ws()))
    for M in (1, 4, 9):
        CM = host_bits(g5.gemm_bf16(dev_bf16(np.ascontiguousarray(X16[:M])), dW, workspace=ws()))
        assert np.array_equal(CM, C16[:M]), f"M={M} rows differ from M=16"


def test_decode_exchange_slots_reset(oracle_mod):
    """M = 1 with a workspace pairs the two K slices through exchange slots in
    the counter region: back-to-back calls with different rows on one
    workspace each match the oracle (a slot left set would mix two calls),
    the region is all zero afterwards, and a repeat gives the same bits."""
    N, K = 12288, 4096
    st, plan = g5.plan_query(g5.GEMM_OP_BF16, 1, N, K)
    assert st == 0 and plan.name == b"decode_splitk" and plan.workspace_bytes == g5.GEMM_WORKSPACE_COUNTER_BYTES
    w = g5.Workspace()
    _, W = gi.decode_inputs(1)
    dW = dev_bf16(W)
    g = np.random.default_rng(gi.SEED_BASE + 9100)
    outs = []
    for i in range(3):
        X = gi.to_bf16_bits(gi.normal(g, (1, K)) * np.float32(2.0 ** (i - 1)))
        C = g5.gemm_bf16(dev_bf16(X), dW, workspace=w)
        check_bf16(host_values(C), oracle_mod.gemm_bf16(X, W), K, f"exchange call {i}")
        outs.append((X, host_bits(C)))
    torch.cuda.synchronize()
    assert int(w.buf[:g5.GEMM_WORKSPACE_COUNTER_BYTES].count_nonzero()) == 0, "exchange slots left set"
    X, bits = outs[0]
    assert np.array_equal(host_bits(g5.gemm_bf16(dev_bf16(X), dW, workspace=w)), bits)


@pytest.mark.parametrize("with_ws", [True, False])
def test_batched_attention_scores(oracle_mod, with_ws):
    """32 x Q[1024,128] . K^T[128,1024] -> f32: every element of every entry."""
    _say(f"batched 32x1024x1024x128 workspace={with_ws}")
    Q, KT = gi.batched_inputs()
    C = g5.gemm_bf16_batched(dev_bf16(Q), dev_bf16(KT), out_dtype=torch.float32,
                             workspace=ws() if with_ws else None)
    host = host_values(C)
    ref = oracle_mod.gemm_bf16_batched(Q, KT)
    for b in range(32):
        check_f32(host[b], ref[b], 128, amax_bf16(Q[b]), amax_bf16(KT[b]), f"batch entry {b}")


@pytest.mark.parametrize("M,N,K,pa,batch", [(520, 1024, 2050, 1, 1), (520, 1024, 2050, 2, 1),
                                            (300, 1024, 2052, 2, 3), (512, 1024, 2048, 2, 1)])
def test_bf16_realigned_rows(oracle_mod, M, N, K, pa, batch):
    """Large products whose A rows are 2-, 4- or 8-byte aligned multiply
    from a copy of A with 16-byte aligned rows (asserted through the plan).
    A's padding holds NaN: a copy that read past K would poison C."""
    _say(f"realigned A {batch}x{M}x{N}x{K} pad {pa}")
    g = np.random.default_rng([M, N, K, pa, batch, 3])
    A = gi.to_bf16_bits(gi.normal(g, (batch, M, K + pa)))
    B = gi.to_bf16_bits(gi.normal(g, (batch, K, N), 0.125))
    A[:, :, K:] = 0x7FC0
    dA, dB = dev_bf16(A), dev_bf16(B)
    C = torch.empty((batch, M, N), device="cuda", dtype=torch.float32)
    st, plan = g5.plan_query(g5.GEMM_OP_BF16, M, N, K, batch=batch, lda=K + pa, a_addr=dA.data_ptr(),
                             b_addr=dB.data_ptr(), c_addr=C.data_ptr(), sA=M * (K + pa), sB=K * N, sC=M * N,
                             c_type=1)
    assert st == 0 and plan.family == 2 and plan.vec_a == 16 and plan.variant in (1, 2), (plan.name, plan.variant)
    split = 0
    if plan.ksplit > 1:       # few tiles: K also split over workgroups (partial tiles)
        tiles = batch * -(-M // plan.tile_m) * -(-N // plan.tile_n)
        split = tiles * plan.ksplit * plan.tile_m * plan.tile_n * 4
    r = lambda b: (b + 255) // 256 * 256
    assert plan.workspace_bytes == g5.GEMM_WORKSPACE_COUNTER_BYTES + r(split) + r(batch * M * ((K + 7) // 8 * 8) * 2)
    g5.gemm_bf16_batched(dA[:, :, :K], dB, C, workspace=ws())
    host = host_values(C)
    for b in range(batch):
        rows = np.arange(0, M, 7)
        ref = oracle_mod.gemm_bf16(np.ascontiguousarray(A[b][rows, :K]), B[b])
        check_f32(host[b][rows], ref, K, amax_bf16(A[b][:, :K]), amax_bf16(B[b]), f"realigned batch {b}")


@pytest.mark.parametrize("with_ws", [True, False])
def test_ragged_single_gemm(oracle_mod, with_ws):
    """M=1000, N=12280, K=4100 bf16 -> f32 (edge tiles in M and N, a K tail
    of 4, 8-byte aligned rows of A, realigned first with a workspace and
    copied 4 bytes per lane without); also with bf16 output.  Every element."""
    _say(f"ragged 1000x12280x4100 workspace={with_ws}")
    A, B = gi.ragged_inputs()
    dA, dB = dev_bf16(A), dev_bf16(B)
    w = ws() if with_ws else None
    st, plan = g5.plan_query(g5.GEMM_OP_BF16, 1000, 12280, 4100, c_type=1, with_workspace=with_ws)
    assert st == 0 and plan.variant == (2 if with_ws else 3)
    ref = oracle_mod.gemm_bf16(A, B)
    C = g5.gemm_bf16(dA, dB, out_dtype=torch.float32, workspace=w)
    check_f32(host_values(C), ref, 4100, amax_bf16(A), amax_bf16(B), "ragged f32")
    Cb = g5.gemm_bf16(dA, dB, out_dtype=torch.bfloat16, workspace=w)
    check_bf16(host_values(Cb), ref, 4100, "ragged bf16")


def test_batched_strides_broadcast_and_single(oracle_mod):
    g = np.random.default_rng(21)
    A = gi.to_bf16_bits(gi.normal(g, (3, 40, 50)))
    B = gi.to_bf16_bits(gi.normal(g, (1, 50, 70), 0.125))
    dA, dB = dev_bf16(A), dev_bf16(B)
    C = g5.gemm_bf16_batched(dA, dB.expand(3, 50, 70), out_dtype=torch.float32, workspace=ws())  # strideB = 0
    host = host_values(C)
    for b in range(3):
        check_f32(host[b], oracle_mod.gemm_bf16(A[b], B[0]), 50, amax_bf16(A[b]), amax_bf16(B), f"bcast {b}")
    # batch of one equals the single GEMM bit for bit
    C1 = g5.gemm_bf16_batched(dA[:1], dB, out_dtype=torch.float32, workspace=ws())
    Cs = g5.gemm_bf16(dA[0], dB[0], out_dtype=torch.float32, workspace=ws())
    assert torch.equal(C1[0], Cs)


# ---------------------------------------------------------- edge semantics

def test_k_zero_writes_zeros():
    A = torch.empty((5, 0), dtype=torch.bfloat16, device="cuda")
    B = torch.empty((0, 7), dtype=torch.bfloat16, device="cuda")
    C = torch.full((5, 7), 3.0, dtype=torch.bfloat16, device="cuda")
    g5.gemm_bf16(A, B, C, workspace=ws())
    assert torch.count_nonzero(C).item() == 0
    Cf = torch.full((5, 7), 3.0, device="cuda")
    g5.gemm_sgemm(A.float(), B.float(), Cf)
    assert torch.count_nonzero(Cf).item() == 0


@pytest.mark.parametrize("M,N,pad,batch,od", [(64, 1000, 8, 1, torch.float32), (64, 1000, 8, 1, torch.bfloat16),
                                              (33, 37, 3, 2, torch.float32), (17, 129, 7, 3, torch.bfloat16),
                                              (1024, 1024, 0, 4, torch.float32)])
def test_k_zero_fill_shapes(M, N, pad, batch, od):
    """K = 0 over aligned rows (16-byte chunks plus a column tail) and
    unaligned rows (element stores): C[:, :N] becomes 0, the ldc padding
    keeps its NaN."""
    A = torch.empty((batch, M, 0), dtype=torch.bfloat16, device="cuda")
    B = torch.empty((batch, 0, N), dtype=torch.bfloat16, device="cuda")
    Cfull = torch.full((batch, M, N + pad), float("nan"), dtype=od, device="cuda")
    g5.gemm_bf16_batched(A, B, Cfull[:, :, :N], workspace=ws())
    host = Cfull.float().cpu().numpy()
    assert np.all(host[:, :, :N] == 0)
    assert np.all(np.isnan(host[:, :, N:]))


def test_empty_m_leaves_c_untouched():
    A = torch.empty((0, 9), dtype=torch.bfloat16, device="cuda")
    B = torch.ones((9, 4), dtype=torch.bfloat16, device="cuda")
    C = torch.empty((0, 4), dtype=torch.bfloat16, device="cuda")
    assert g5.gemm_bf16(A, B, C, workspace=ws()).shape == (0, 4)


@pytest.mark.parametrize("M", [1, 40])   # decode path and tiled path
def test_bf16_round_to_nearest_even_ties(M):
    """K=2: 1*1 + 1*2^-8 = 1 + 2^-8 exactly in FP32 -> tie -> 1.0;
    (1+2^-7) + 2^-8 = 1 + 3*2^-8 -> tie -> 1 + 2^-6."""
    a = np.ones((M, 2), np.float32)
    b = np.array([[1.0, 1.0 + 2 ** -7], [2 ** -8, 2 ** -8]], np.float32)
    C = g5.gemm_bf16(dev_bf16(gi.to_bf16_bits(a)), dev_bf16(gi.to_bf16_bits(b)), workspace=ws())
    bits = host_bits(C)
    assert np.all(bits[:, 0] == 0x3F80) and np.all(bits[:, 1] == 0x3F82), bits[:2]


@pytest.mark.parametrize("M,N,K", [(64, 64, 64), (16, 100, 300), (1024, 1152, 4100), (300, 300, 300)])
def test_identity_and_all_ones(M, N, K):
    """All-ones: every entry is exactly K (bf16 output: RNE(K)); identity
    A = I gives C = B exactly."""
    ones_a = torch.ones((M, K), dtype=torch.bfloat16, device="cuda")
    ones_b = torch.ones((K, N), dtype=torch.bfloat16, device="cuda")
    Cf = g5.gemm_bf16(ones_a, ones_b, out_dtype=torch.float32, workspace=ws())
    assert torch.all(Cf == K)
    Cb = g5.gemm_bf16(ones_a, ones_b, workspace=ws())
    want = gi.bf16_bits_to_f32(gi.to_bf16_bits(np.array([K], np.float32)))[0]
    assert torch.all(Cb.float() == float(want))
    Cs = g5.gemm_sgemm(ones_a.float(), ones_b.float())
    assert torch.all(Cs == K)
    if M == K:
        eye = torch.eye(K, dtype=torch.bfloat16, device="cuda")
        B = torch.randn((K, N), device="cuda").to(torch.bfloat16)
        assert torch.equal(g5.gemm_bf16(eye, B, workspace=ws()), B)
        assert torch.equal(g5.gemm_sgemm(eye.float(), B.float()), B.float())


def test_deterministic_bitwise():
    X, W = gi.ffn_inputs(M=512, K=1024, N=3072)
    dX, dW = dev_bf16(X), dev_bf16(W)
    c1 = host_bits(g5.gemm_bf16(dX, dW, workspace=ws()))
    c2 = host_bits(g5.gemm_bf16(dX, dW, workspace=ws()))
    assert np.array_equal(c1, c2)
    A, B = gi.small_case("f32", 300, 300, 300)
    s1 = g5.gemm_sgemm(dev_f32(A), dev_f32(B))
    s2 = g5.gemm_sgemm(dev_f32(A), dev_f32(B))
    assert torch.equal(s1, s2)


def test_nan_sentinel_every_element_written_once():
    """C pre-filled with NaN inside a guard band: afterwards every logical
    element is finite and the padding columns and the rows after the last are
    still NaN."""
    for (M, N, K) in [(257, 193, 70), (1000, 1000, 64), (5, 300, 40)]:
        A, B = gi.small_case("bf16", M, N, K, seed=3)
        buf = torch.full((M + 3, N + 9), float("nan"), device="cuda")
        g5.gemm_bf16(dev_bf16(A), dev_bf16(B), buf[:M, :N], workspace=ws())
        h = buf.cpu().numpy()
        assert np.all(np.isfinite(h[:M, :N]))
        assert np.all(np.isnan(h[:M, N:])) and np.all(np.isnan(h[M:, :]))


# Each tiled-kernel variant on a shape chosen to select it (asserted through
# the host plan).  Padding columns of A and B and the ldc padding of C hold
# NaN: a kernel that read A beyond K, or let columns of B beyond N reach a
# stored output, or wrote outside the logical C, fails.
VARIANT_CASES = [
    # M, N, K, A row pad, B row pad, forced config (None: selector), expected variant
    (512, 384, 128, 0, 0, None, 1),              # aligned ring kernel
    (512, 384, 128, 0, 0, "bf16_256x192", 1),    # the same with 192-column tiles
    (300, 392, 264, 0, 0, None, 2),              # masked ring kernel, K tail of 8
    (300, 392, 264, 0, 0, "bf16_256x192", 2),
    (300, 392, 262, 0, 0, None, 3),              # 4-byte A copies (rows 4-byte aligned)
    (300, 392, 20, 4, 0, None, 2),               # K < 32: only the element-loaded tail stage
    (257, 200, 96, 8, 8, None, 2),               # edge tiles in M and N, padded rows
    (300, 392, 48, 0, 0, "bf16_128x128", 2),     # one whole and one partial slab
    (70, 392, 1000, 2, 0, None, 3),              # long K with a tail, few rows
]


@pytest.mark.parametrize("M,N,K,pa,pb,cfg,variant", VARIANT_CASES)
def test_bf16_kernel_variants(oracle_mod, monkeypatch, M, N, K, pa, pb, cfg, variant):
    _say(f"variant {variant} {M}x{N}x{K} pads ({pa},{pb}) config {cfg}")
    if cfg:
        monkeypatch.setenv("GEMM_FORCE_CONFIG", cfg)
    g = np.random.default_rng([M, N, K, pa, pb])
    A = gi.to_bf16_bits(gi.normal(g, (M, K + pa)))
    B = gi.to_bf16_bits(gi.normal(g, (K, N + pb), 0.125))
    A[:, K:] = 0x7FC0    # NaN in the padding
    B[:, N:] = 0x7FC0
    dA, dB = dev_bf16(A), dev_bf16(B)
    for od, ct in ((torch.bfloat16, 0), (torch.float32, 1)):
        Cfull = torch.full((M, N + 8), float("nan"), device="cuda", dtype=od)
        st, plan = g5.plan_query(g5.GEMM_OP_BF16, M, N, K, lda=K + pa, ldb=N + pb, ldc=N + 8,
                                 a_addr=dA.data_ptr(), b_addr=dB.data_ptr(), c_addr=Cfull.data_ptr(), c_type=ct)
        assert st == 0 and plan.family == 2 and plan.variant == variant, (plan.name, plan.variant)
        g5.gemm_bf16(dA[:, :K], dB[:, :N], Cfull[:, :N], workspace=ws())
        ref = oracle_mod.gemm_bf16(np.ascontiguousarray(A[:, :K]), np.ascontiguousarray(B[:, :N]))
        host = host_values(Cfull)
        if od == torch.bfloat16:
            check_bf16(host[:, :N], ref, K, f"variant {variant} bf16")
        else:
            check_f32(host[:, :N], ref, K, amax_bf16(A[:, :K]), amax_bf16(B[:, :N]), f"variant {variant} f32")
        assert np.all(np.isnan(host[:, N:])), "ldc padding was written"


@pytest.mark.parametrize("M,N,K,S,lda_pad,batch", [
    (300, 392, 262, 2, 0, 1),      # 4-byte A copies, K tail of 6
    (512, 512, 4096, 5, 0, 1),     # aligned whole tiles, uneven slices (25, 25, 25, 25, 28 stages)
    (257, 200, 1000, 7, 0, 1),     # ragged edges, K tail of 8 in the last slice
    (129, 136, 640, 4, 8, 3),      # batched, padded A rows
    (64, 128, 256, 2, 0, 2),       # one tile per batch entry
])
def test_bf16_ksplit(oracle_mod, monkeypatch, M, N, K, S, lda_pad, batch):
    """K split over S workgroups per tile (forced), every ring variant the
    shape selects, FP32 and bf16 output; NaN in the ldc padding shows any
    stray write; a second call gives the same bits (the per-tile counters
    are back at zero and the slice order is fixed)."""
    _say(f"bf16 ksplit {S} batch {batch} {M}x{N}x{K} lda pad {lda_pad}")
    g = np.random.default_rng([gi.SEED_BASE + 5000, M, N, K, S])
    A = gi.to_bf16_bits(gi.normal(g, (batch, M, K + lda_pad)))
    B = gi.to_bf16_bits(gi.normal(g, (batch, K, N), 0.125))
    dA, dB = dev_bf16(A), dev_bf16(B)
    monkeypatch.setenv("GEMM_FORCE_CONFIG", "bf16_128x128")
    monkeypatch.setenv("GEMM_FORCE_KSPLIT", str(S))
    for od in (torch.float32, torch.bfloat16):
        Cfull = torch.full((batch, M, N + 8), float("nan"), device="cuda", dtype=od)
        outs = []
        for _ in range(2):
            if batch == 1:
                g5.gemm_bf16(dA[0, :, :K], dB[0], Cfull[0, :, :N], workspace=ws())
            else:
                g5.gemm_bf16_batched(dA[:, :, :K], dB, Cfull[:, :, :N], workspace=ws())
            outs.append(Cfull.clone())
        assert torch.equal(outs[0].view(torch.int16 if od == torch.bfloat16 else torch.int32),
                           outs[1].view(torch.int16 if od == torch.bfloat16 else torch.int32)), "not deterministic"
        host = host_values(Cfull)
        for b in range(batch):
            Ab = np.ascontiguousarray(A[b, :, :K])
            ref = oracle_mod.gemm_bf16(Ab, B[b])
            if od == torch.bfloat16:
                check_bf16(host[b, :, :N], ref, K, f"ksplit {S} bf16 entry {b}")
            else:
                check_f32(host[b, :, :N], ref, K, amax_bf16(Ab), amax_bf16(B[b]), f"ksplit {S} f32 entry {b}")
        assert np.all(np.isnan(host[:, :, N:])), "ldc padding was written"


def test_ksplit_back_to_back_changing_split(oracle_mod, monkeypatch):
    """Calls with different splits and shapes on one stream, without
    synchronising in between: each sees zeroed counters."""
    monkeypatch.setenv("GEMM_FORCE_CONFIG", "bf16_128x128")
    cases = [(256, 384, 1024, 4), (256, 384, 1024, 2), (384, 256, 768, 6), (256, 384, 1024, 8)]
    res = []
    for M, N, K, S in cases:
        A, B = gi.small_case("bf16", M, N, K, seed=S, scale_b=0.125)
        monkeypatch.setenv("GEMM_FORCE_KSPLIT", str(S))
        res.append((A, B, g5.gemm_bf16(dev_bf16(A), dev_bf16(B), out_dtype=torch.float32, workspace=ws())))
    for (A, B, C), (M, N, K, S) in zip(res, cases):
        check_f32(host_values(C), oracle_mod.gemm_bf16(A, B), K, amax_bf16(A), amax_bf16(B), f"split {S}")


def test_ksplit_shard_full_size(oracle_mod):
    """The 1024x1536x4096 shard of an 8-way column split of the FFN
    projection: 96 tiles of 128x128, K split in 2 by the selector."""
    _say("bf16 1024x1536x4096 split")
    X, W = gi.ffn_inputs()
    W = np.ascontiguousarray(W[:, :1536])
    st, plan = g5.plan_query(g5.GEMM_OP_BF16, 1024, 1536, 4096)
    assert st == 0 and plan.ksplit == 2
    C = g5.gemm_bf16(dev_bf16(X), dev_bf16(W), workspace=ws())
    ref = oracle_mod.gemm_bf16(X, W)
    check_bf16(host_values(C), ref, 4096, "shard")


def test_concurrent_calls_from_two_threads():
    """Two host threads enqueue K-split calls on one stream at once, each with
    its own workspace (the library keeps no state between calls), one of them
    through sizes that keep growing its workspace: every result equals the
    same call made alone, bit for bit."""
    import threading
    shapes_a = [(256, 256, 4096)] * 12
    shapes_b = [(128 * i, 256, 2048) for i in (1, 2, 3, 4, 2, 5, 6, 3, 7, 8, 4, 8)]
    cases = {}
    for (M, N, K) in set(shapes_a + shapes_b):
        A, B = gi.small_case("bf16", M, N, K, seed=90, scale_b=0.125)
        dA, dB = dev_bf16(A), dev_bf16(B)
        cases[(M, N, K)] = (dA, dB, g5.gemm_bf16(dA, dB, out_dtype=torch.float32, workspace=ws()))
    torch.cuda.synchronize()
    for key in cases:
        st, plan = g5.plan_query(g5.GEMM_OP_BF16, *key, c_type=1)
        assert st == 0 and plan.ksplit > 1, key
    outs = {0: [], 1: []}
    errors = []
    shared = torch.cuda.Stream()
    shared.wait_stream(torch.cuda.current_stream())

    def worker(idx, shapes):
        try:
            with torch.cuda.stream(shared):
                w = g5.Workspace()
                for key in shapes:
                    dA, dB, _ = cases[key]
                    outs[idx].append((key, g5.gemm_bf16(dA, dB, out_dtype=torch.float32, workspace=w)))
        except Exception as e:          # reported below
            errors.append(e)

    ts = [threading.Thread(target=worker, args=(0, shapes_a)), threading.Thread(target=worker, args=(1, shapes_b))]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    shared.synchronize()
    torch.cuda.synchronize()
    assert not errors, errors
    for idx in (0, 1):
        for key, C in outs[idx]:
            assert torch.equal(C.view(torch.int32), cases[key][2].view(torch.int32)), (idx, key)


def test_calls_allocate_nothing_on_a_fresh_stream(oracle_mod):
    """The C entry points allocate, free and synchronise nothing: device
    memory in use is the same before and after a split small-M call through
    gemm_run (with a caller workspace) and a named call (without), both on a
    stream that has never run a GEMM; and the results equal the oracle's."""
    import ctypes
    X, W = gi.small_case("bf16", 1, 12288, 4096, seed=95, scale_b=0.125)
    dX, dW = dev_bf16(X), dev_bf16(W)
    C1 = torch.empty((1, 12288), dtype=torch.bfloat16, device="cuda")
    C2 = torch.empty_like(C1)
    st, plan = g5.plan_query(g5.GEMM_OP_BF16, 1, 12288, 4096)
    assert st == 0 and plan.name == b"decode_splitk"
    wsbuf = torch.zeros(plan.workspace_bytes, dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    L = g5.lib()
    st1 = L.gemm_run(g5.GEMM_OP_BF16, 1, 1, 12288, 4096, dX.data_ptr(), 4096, 0, dW.data_ptr(), 12288, 0,
                     C1.data_ptr(), 12288, 0, 0, 1.0, None, 0.0, None, None, wsbuf.data_ptr(), wsbuf.numel(),
                     ctypes.c_void_p(s.cuda_stream))
    st2 = L.gemm_bf16(1, 12288, 4096, dX.data_ptr(), 4096, dW.data_ptr(), 12288, C2.data_ptr(), 12288, 0,
                      ctypes.c_void_p(s.cuda_stream))
    s.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert st1 == 0 and st2 == 0
    assert free1 == free0, f"device free memory changed by {free0 - free1} bytes"
    assert int(wsbuf[:g5.GEMM_WORKSPACE_COUNTER_BYTES].count_nonzero()) == 0, "arrival counters not left at zero"
    ref = oracle_mod.gemm_bf16(X, W)
    check_bf16(host_values(C1), ref, 4096, "split small-M with workspace")
    check_bf16(host_values(C2), ref, 4096, "whole-K small-M without workspace")


@pytest.mark.parametrize("order", ["rowmajor", "bands"])
def test_tile_orders_give_identical_results(monkeypatch, order):
    """The tile orders the XCD-aware map is measured against (environment
    GEMM_TILE_ORDER) only move tiles between workgroups: every tile is
    computed the same way, so C is bitwise the default order's."""
    M, N, K = 1024, 3072, 1024
    _say(f"tile order {order} {M}x{N}x{K}")
    A, B = gi.small_case("bf16", M, N, K, seed=41, scale_b=0.125)
    dA, dB = dev_bf16(A), dev_bf16(B)
    ref = host_bits(g5.gemm_bf16(dA, dB, workspace=ws()))
    monkeypatch.setenv("GEMM_TILE_ORDER", order)
    got = host_bits(g5.gemm_bf16(dA, dB, workspace=ws()))
    assert np.array_equal(got, ref)
