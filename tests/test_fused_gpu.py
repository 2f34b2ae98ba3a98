"""GPU parity of the fused epilogues (gemm_bf16_silu, gemm_bf16_swiglu)
against the oracle, through the C ABI.

Page "Operator & Runtime" fuses SiLU into the output tile (§5.4.2) and the
SwiGLU product into the two projections sharing X (§5.3.1), keeping the
unfused program's bf16 roundings (§5.4.3).  The oracle computes both in
double from the exact products; the tolerances are derived in
_gpu_helpers.py from the bf16 GEMM bar.
"""
import numpy as np
import pytest
import torch

import gemm_inputs as gi
from _gpu_helpers import check_silu, check_swiglu, dev_bf16, host_bits, host_values, ws

import dense_gemm_05_amd as g5

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[fused] {msg}", flush=True)


@pytest.fixture(autouse=True)
def _no_forced_config(monkeypatch):
    monkeypatch.delenv("GEMM_FORCE_CONFIG", raising=False)


def _swiglu_case(M, N, K, seed):
    g = np.random.default_rng([gi.SEED_BASE + 3000 + seed, M, N, K])
    X = gi.to_bf16_bits(gi.normal(g, (M, K)))
    Wgu = gi.to_bf16_bits(gi.normal(g, (K, 2 * N), 0.125))
    return X, Wgu


def _swiglu_ref(oracle_mod, X, Wgu):
    N = Wgu.shape[1] // 2
    G = oracle_mod.gemm_bf16(X, np.ascontiguousarray(Wgu[:, :N]))
    U = oracle_mod.gemm_bf16(X, np.ascontiguousarray(Wgu[:, N:]))
    Z, g, u, t = oracle_mod.swiglu_bf16(X, Wgu)
    return Z, G, U, t, u


SHAPES = [(300, 392, 262), (256, 192, 256), (512, 576, 96), (17, 200, 64), (1, 128, 4100), (257, 96, 33)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_silu_ragged(oracle_mod, M, N, K):
    _say(f"silu {M}x{N}x{K}")
    A, B = gi.small_case("bf16", M, N, K, seed=21, scale_b=0.125)
    Y = g5.gemm_bf16_silu(dev_bf16(A), dev_bf16(B), workspace=ws())
    G = oracle_mod.gemm_bf16(A, B)
    check_silu(host_values(Y), G, oracle_mod.gemm_bf16_silu(A, B), K, f"silu {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_swiglu_ragged(oracle_mod, M, N, K):
    _say(f"swiglu {M}x{N}x{K}")
    X, Wgu = _swiglu_case(M, N, K, 1)
    Z = g5.gemm_bf16_swiglu(dev_bf16(X), dev_bf16(Wgu), workspace=ws())
    Zr, G, U, t, u = _swiglu_ref(oracle_mod, X, Wgu)
    check_swiglu(host_values(Z), G, U, t, u, Zr, K, f"swiglu {M}x{N}x{K}")


@pytest.mark.parametrize("cfg", ["bf16_256x192", "bf16_256x256", "bf16_128x128"])
@pytest.mark.parametrize("op", ["silu", "swiglu"])
def test_fused_every_config(oracle_mod, monkeypatch, cfg, op):
    """Each configuration compiled with the epilogues, forced, on a ragged
    problem with padded row strides: A rows of 266 elements (4-byte aligned:
    4-byte A copies) with K = 261 (a K tail), then 16-byte rows with
    K = 264; B and C rows padded by 8 elements.  NaN in the padding of the
    output shows any write past N."""
    M, N = 300, 392
    nb = N if op == "silu" else 2 * N
    for K, pa in ((261, 5), (264, 8)):
        _say(f"{op} forced {cfg} {M}x{N}x{K} A pad {pa}")
        g = np.random.default_rng([gi.SEED_BASE + 4000, K, pa, nb])
        A = gi.to_bf16_bits(gi.normal(g, (M, K + pa)))
        B = gi.to_bf16_bits(gi.normal(g, (K, nb + 8), 0.125))
        dA, dB = dev_bf16(A), dev_bf16(B)
        monkeypatch.setenv("GEMM_FORCE_CONFIG", cfg)
        Cfull = torch.full((M, N + 8), float("nan"), device="cuda", dtype=torch.bfloat16)
        fn = g5.gemm_bf16_silu if op == "silu" else g5.gemm_bf16_swiglu
        fn(dA[:, :K], dB[:, :nb], Cfull[:, :N])
        monkeypatch.delenv("GEMM_FORCE_CONFIG")
        host = host_values(Cfull)
        Av = np.ascontiguousarray(A[:, :K])
        Bv = np.ascontiguousarray(B[:, :nb])
        if op == "silu":
            check_silu(host[:, :N], oracle_mod.gemm_bf16(Av, Bv), oracle_mod.gemm_bf16_silu(Av, Bv), K, cfg)
        else:
            Zr, G, U, t, u = _swiglu_ref(oracle_mod, Av, Bv)
            check_swiglu(host[:, :N], G, U, t, u, Zr, K, cfg)
        assert np.all(np.isnan(host[:, N:])), f"{cfg} {op}: output padding was written"


def test_swiglu_ffn_full_size(oracle_mod):
    """The FFN's gate and up projections of X[1024,4096] with one merged
    weight [4096, 2 x 12288] -> Z [1024, 12288]: the benchmarked launch;
    every element."""
    _say("swiglu 1024x12288x4096 (every element)")
    X, Wgu = gi.swiglu_inputs()
    st, plan = g5.plan_query(g5.GEMM_OP_BF16_SWIGLU, 1024, 12288, 4096)
    assert st == 0 and plan.name == b"bf16_256x192" and plan.grid == 512 and plan.variant == 1
    Z = g5.gemm_bf16_swiglu(dev_bf16(X), dev_bf16(Wgu), workspace=ws())
    Zr, G, U, t, u = _swiglu_ref(oracle_mod, X, Wgu)
    check_swiglu(host_values(Z), G, U, t, u, Zr, 4096, "swiglu FFN")


def test_silu_ffn_full_size(oracle_mod):
    _say("silu 1024x12288x4096")
    X, W = gi.ffn_inputs()
    Y = g5.gemm_bf16_silu(dev_bf16(X), dev_bf16(W), workspace=ws())
    rows = np.array([0, 255, 256, 700, 1023])
    Xs = np.ascontiguousarray(X[rows])
    check_silu(host_values(Y)[rows], oracle_mod.gemm_bf16(Xs, W), oracle_mod.gemm_bf16_silu(Xs, W), 4096,
               "silu FFN rows")


def test_fused_deterministic_and_k_zero():
    X, Wgu = _swiglu_case(300, 200, 520, 3)
    dX, dW = dev_bf16(X), dev_bf16(Wgu)
    z1 = g5.gemm_bf16_swiglu(dX, dW, workspace=ws())
    z2 = g5.gemm_bf16_swiglu(dX, dW, workspace=ws())
    assert torch.equal(z1.view(torch.int16), z2.view(torch.int16))
    # K = 0: g = u = 0, SiLU(0) = 0, Z = 0; Y = SiLU(0) = 0
    Z = torch.full((300, 200), float("nan"), device="cuda", dtype=torch.bfloat16)
    g5.gemm_bf16_swiglu(dX[:, :0], dW[:0, :], Z, workspace=ws())
    assert torch.all(Z == 0)
    Y = torch.full((300, 200), float("nan"), device="cuda", dtype=torch.bfloat16)
    g5.gemm_bf16_silu(dX[:, :0], dW[:0, :200], Y, workspace=ws())
    assert torch.all(Y == 0)


def test_swiglu_matches_separate_products(monkeypatch):
    """Z from the fused call equals bf16(bf16(SiLU(g)) * u) computed from the
    library's own bf16 gate and up products, bit for bit: both take the same
    FP32 sums (same kernel, same summation order; the plain products are
    kept from splitting K, which the fused call never does) and round them
    once."""
    X, Wgu = _swiglu_case(512, 384, 640, 4)
    dX, dW = dev_bf16(X), dev_bf16(Wgu)
    Z = g5.gemm_bf16_swiglu(dX, dW, workspace=ws())
    monkeypatch.setenv("GEMM_FORCE_KSPLIT", "1")
    g = g5.gemm_bf16(dX, dW[:, :384], workspace=ws())
    u = g5.gemm_bf16(dX, dW[:, 384:], workspace=ws())
    # the elementwise step on the host in float32, from the GPU's bf16 g and u
    gf = host_values(g).astype(np.float32)
    sig = (gf / (np.float32(1) + np.exp(-gf, dtype=np.float32))).astype(np.float32)
    t = gi.bf16_bits_to_f32(gi.to_bf16_bits(sig))
    zf = gi.bf16_bits_to_f32(gi.to_bf16_bits(t * host_values(u).astype(np.float32)))
    got = host_values(Z).astype(np.float32)
    # t may differ by one bf16 step (at most 2^-7 of t) where SiLU lands
    # within float32 error of a bf16 rounding boundary (GPU exp and
    # reciprocal vs host exp and division); z = bf16(t u) then differs by at
    # most 2^-7 + 2 x 2^-9 of z.  Everything else is identical.
    same = got == zf
    assert same.mean() > 0.999, f"only {same.mean():.5f} identical"
    assert np.all(np.abs(got - zf) <= 2.0 ** -6 * np.abs(zf) + 1e-30)


@pytest.mark.parametrize("broadcast_x", [False, True])
def test_swiglu_batched_experts(oracle_mod, broadcast_x):
    """Batched SwiGLU: each entry (an expert of a mixture-of-experts FFN) has
    its own merged weight, and its own tokens or (stride 0) the same tokens;
    ragged tiles in M and N, a K tail."""
    batch, M, N, K = 4, 150, 200, 264
    _say(f"swiglu batched {batch}x{M}x{N}x{K} broadcast_x={broadcast_x}")
    g = np.random.default_rng([gi.SEED_BASE + 4100, int(broadcast_x)])
    X = gi.to_bf16_bits(gi.normal(g, (1 if broadcast_x else batch, M, K)))
    Wgu = gi.to_bf16_bits(gi.normal(g, (batch, K, 2 * N), 0.125))
    dX = dev_bf16(X)
    if broadcast_x:
        dX = dX.expand(batch, -1, -1)
    Z = g5.gemm_bf16_swiglu_batched(dX, dev_bf16(Wgu), workspace=ws())
    got = host_values(Z)
    for b in range(batch):
        Xb = X[0 if broadcast_x else b]
        Zr, G, U, t, u = _swiglu_ref(oracle_mod, Xb, Wgu[b])
        check_swiglu(got[b], G, U, t, u, Zr, K, f"swiglu expert {b}")


def test_silu_batched(oracle_mod, monkeypatch):
    """Batched SiLU on every fused config, each entry checked, NaN padding
    between entries untouched."""
    batch, M, N, K = 3, 130, 136, 200
    g = np.random.default_rng([gi.SEED_BASE + 4200])
    A = gi.to_bf16_bits(gi.normal(g, (batch, M, K)))
    B = gi.to_bf16_bits(gi.normal(g, (batch, K, N), 0.125))
    for cfg in ("bf16_256x192", "bf16_256x256", "bf16_128x128"):
        _say(f"silu batched forced {cfg}")
        monkeypatch.setenv("GEMM_FORCE_CONFIG", cfg)
        Cfull = torch.full((batch, M + 2, N), float("nan"), device="cuda", dtype=torch.bfloat16)
        g5.gemm_bf16_silu_batched(dev_bf16(A), dev_bf16(B), Cfull[:, :M], workspace=ws())
        host = host_values(Cfull)
        for b in range(batch):
            check_silu(host[b, :M], oracle_mod.gemm_bf16(A[b], B[b]), oracle_mod.gemm_bf16_silu(A[b], B[b]), K,
                       f"silu {cfg} entry {b}")
        assert np.all(np.isnan(host[:, M:])), "rows between entries were written"


# ----------------------------------------------------------------- small M
# M <= 16 runs on the small-M kernels, which apply SiLU and SwiGLU as they
# store: with a workspace the K-split path (for SwiGLU the gate and up
# columns of a strip are read by separate workgroups and combined by the
# last to finish), without one the whole-K 64-column kernel (both halves in
# one workgroup).  K % 32 != 0 and N % 64 != 0 take the whole-K kernel's
# general variant.
SMALL_M = [(1, 12288, 4096), (4, 384, 640), (16, 640, 1024), (3, 200, 100), (2, 256, 4128)]


def _small_m_plan(op, M, N, K, with_ws):
    st, plan = g5.plan_query(op, M, N, K, with_workspace=with_ws)
    assert st == 0 and plan.name.decode().startswith("decode"), (st, plan.name)
    return plan.name.decode()


@pytest.mark.parametrize("with_ws", [True, False])
@pytest.mark.parametrize("M,N,K", SMALL_M)
def test_silu_small_m(oracle_mod, M, N, K, with_ws):
    cfg = _small_m_plan(g5.GEMM_OP_BF16_SILU, M, N, K, with_ws)
    _say(f"silu small M {M}x{N}x{K} ws={with_ws} -> {cfg}")
    A, B = gi.small_case("bf16", M, N, K, seed=23, scale_b=0.125)
    Y = g5.gemm_bf16_silu(dev_bf16(A), dev_bf16(B), workspace=ws() if with_ws else None)
    torch.cuda.synchronize()
    G = oracle_mod.gemm_bf16(A, B)
    check_silu(host_values(Y), G, oracle_mod.gemm_bf16_silu(A, B), K, f"silu {M}x{N}x{K} {cfg}")


@pytest.mark.parametrize("with_ws", [True, False])
@pytest.mark.parametrize("M,N,K", SMALL_M)
def test_swiglu_small_m(oracle_mod, M, N, K, with_ws):
    cfg = _small_m_plan(g5.GEMM_OP_BF16_SWIGLU, M, N, K, with_ws)
    _say(f"swiglu small M {M}x{N}x{K} ws={with_ws} -> {cfg}")
    X, Wgu = _swiglu_case(M, N, K, 7)
    Z = g5.gemm_bf16_swiglu(dev_bf16(X), dev_bf16(Wgu), workspace=ws() if with_ws else None)
    torch.cuda.synchronize()
    Zr, G, U, t, u = _swiglu_ref(oracle_mod, X, Wgu)
    check_swiglu(host_values(Z), G, U, t, u, Zr, K, f"swiglu {M}x{N}x{K} {cfg}")


@pytest.mark.parametrize("with_ws", [True, False])
def test_small_m_fused_rows_independent_of_m(with_ws):
    """The small-M kernels split K the same way for every row count, so a
    row's SiLU or SwiGLU output does not depend on how many rows the call
    has: the first 3 rows of a 16-row call equal a 3-row call, bit for bit."""
    M, N, K = 16, 1024, 2048
    X, Wgu = _swiglu_case(M, N, K, 8)
    dX, dW = dev_bf16(X), dev_bf16(Wgu)
    w = ws() if with_ws else None
    z16 = host_bits(g5.gemm_bf16_swiglu(dX, dW, workspace=w))
    z3 = host_bits(g5.gemm_bf16_swiglu(dX[:3].contiguous(), dW, workspace=w))
    y16 = host_bits(g5.gemm_bf16_silu(dX, dW[:, :N].contiguous(), workspace=w))
    y3 = host_bits(g5.gemm_bf16_silu(dX[:3].contiguous(), dW[:, :N].contiguous(), workspace=w))
    assert np.array_equal(z16[:3], z3)
    assert np.array_equal(y16[:3], y3)


@pytest.mark.parametrize("broadcast_x", [False, True])
@pytest.mark.parametrize("with_ws", [True, False])
def test_swiglu_batched_small_m(oracle_mod, broadcast_x, with_ws):
    """Batched SwiGLU with a few tokens per expert (the small-M kernels take
    the batch as their second grid dimension)."""
    batch, M, N, K = 4, 5, 384, 512
    st, plan = g5.plan_query(g5.GEMM_OP_BF16_SWIGLU, M, N, K, batch=batch, with_workspace=with_ws)
    assert st == 0 and plan.name.decode().startswith("decode"), (st, plan.name)
    g = np.random.default_rng([gi.SEED_BASE + 4200, int(broadcast_x)])
    X = gi.to_bf16_bits(gi.normal(g, (1 if broadcast_x else batch, M, K)))
    Wgu = gi.to_bf16_bits(gi.normal(g, (batch, K, 2 * N), 0.125))
    dX = dev_bf16(X)
    if broadcast_x:
        dX = dX.expand(batch, -1, -1)
    Z = g5.gemm_bf16_swiglu_batched(dX, dev_bf16(Wgu), workspace=ws() if with_ws else None)
    got = host_values(Z)
    for b in range(batch):
        Zr, G, U, t, u = _swiglu_ref(oracle_mod, X[0 if broadcast_x else b], Wgu[b])
        check_swiglu(got[b], G, U, t, u, Zr, K, f"swiglu small-M expert {b}")



@pytest.mark.parametrize("M", [1, 16])
def test_small_m_exchange_equals_counter_combine(monkeypatch, M):
    """The small-M path's two workgroups per strip (two K slices of the
    plain product or SiLU; SwiGLU's gate and up) meet in exchange slots by
    default; GEMM_DECODE_PAIR=0 sends them through counters and partial sums
    instead.  Both give the same bits, for the product, SiLU and SwiGLU."""
    N, K = 12288, 4096
    _say(f"exchange against counter combine, M={M}")
    g = np.random.default_rng([gi.SEED_BASE + 9200, M])
    dX = dev_bf16(gi.to_bf16_bits(gi.normal(g, (M, K))))
    _, W = gi.decode_inputs(1)
    _, Wgu = gi.swiglu_inputs(1, K, N)
    dW, dWgu = dev_bf16(W), dev_bf16(Wgu)
    w = ws()
    calls = {"product": lambda: g5.gemm_bf16(dX, dW, workspace=w),
             "silu": lambda: g5.gemm_bf16_silu(dX, dW, workspace=w),
             "swiglu": lambda: g5.gemm_bf16_swiglu(dX, dWgu, workspace=w)}
    for name, op in (("product", g5.GEMM_OP_BF16), ("swiglu", g5.GEMM_OP_BF16_SWIGLU)):
        st, plan = g5.plan_query(op, M, N, K)
        assert st == 0 and plan.name == b"decode_splitk" and plan.workspace_bytes == g5.GEMM_WORKSPACE_COUNTER_BYTES, name
    paired = {k: host_bits(f()) for k, f in calls.items()}
    monkeypatch.setenv("GEMM_DECODE_PAIR", "0")
    st, plan = g5.plan_query(g5.GEMM_OP_BF16, M, N, K)
    assert st == 0 and plan.workspace_bytes > g5.GEMM_WORKSPACE_COUNTER_BYTES      # partial sums
    for k, f in calls.items():
        assert np.array_equal(host_bits(f()), paired[k]), k
