"""GPU parity of the affine epilogue C := alpha * (A.B) + bias + beta * C
(gemm_bf16_affine, and gemm_bf16_nt_affine with B given transposed) against
the oracle, through the C ABI.

The epilogue is applied to the finished output tile like the activations of
page "Operator & Runtime" §5.4.2, with §5.4.3's rounding rule: the product
is accumulated in FP32 and the result rounded once.  The oracle evaluates
alpha * P + bias + beta * C_old in double from the exact product P; the
tolerance is derived in _gpu_helpers.py from the bf16 and FP32 GEMM bars.
"""
import numpy as np
import pytest
import torch

import gemm_inputs as gi
from _gpu_helpers import amax_bf16, check_affine, dev_bf16, dev_f32, host_values, ws

import dense_gemm_05_amd as g5

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[affine] {msg}", flush=True)


@pytest.fixture(autouse=True)
def _no_forced_config(monkeypatch):
    monkeypatch.delenv("GEMM_FORCE_CONFIG", raising=False)
    monkeypatch.delenv("GEMM_FORCE_KSPLIT", raising=False)


def _case(M, N, K, seed, batch=1):
    """bf16 A ~ N(0,1), B ~ N(0,1/64), bias ~ N(0,1); old C ~ N(0,1) in float32
    and as bf16 bit patterns."""
    g = np.random.default_rng([gi.SEED_BASE + 5000 + seed, batch, M, N, K])
    A = gi.to_bf16_bits(gi.normal(g, (batch, M, K)))
    B = gi.to_bf16_bits(gi.normal(g, (batch, K, N), 0.125))
    bias = gi.to_bf16_bits(gi.normal(g, (N,)))
    old32 = gi.normal(g, (batch, M, N))
    return A, B, bias, old32, gi.to_bf16_bits(old32)


def _run_and_check(oracle_mod, A, B, bias, old32, old16, alpha, beta, out_f32, what, use_bias=True):
    batch, M, K = A.shape
    N = B.shape[2]
    dA, dB = dev_bf16(A), dev_bf16(B)
    dbias = dev_bf16(bias) if use_bias else None
    C = dev_f32(old32) if out_f32 else dev_bf16(old16)
    g5.gemm_bf16_affine(dA if batch > 1 else dA[0], dB if batch > 1 else dB[0], C if batch > 1 else C[0],
                        alpha=alpha, bias=dbias, beta=beta, workspace=ws())
    got = host_values(C)
    bias_vals = gi.bf16_bits_to_f32(bias).astype(np.float64) if use_bias else np.zeros(N)
    worst = 0.0
    for b in range(batch):
        old = old32[b] if out_f32 else old16[b]
        ref = oracle_mod.gemm_bf16_affine(A[b], B[b], alpha, bias if use_bias else None, beta, old)
        P = oracle_mod.gemm_bf16(A[b], B[b])
        old_vals = old.astype(np.float64) if out_f32 else gi.bf16_bits_to_f32(old).astype(np.float64)
        worst = max(worst, check_affine(got[b], ref, P, K, alpha, bias_vals, beta, old_vals, out_f32,
                                        amax_bf16(A[b]), amax_bf16(B[b]), f"{what} entry {b}"))
    return worst


SHAPES = [(300, 392, 264), (256, 192, 256), (17, 200, 64), (1, 128, 4100), (257, 96, 33), (512, 512, 4096)]


@pytest.mark.parametrize("out_f32", [False, True])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_affine_ragged(oracle_mod, M, N, K, out_f32):
    """Bias and beta*C together on ragged shapes (K tails, partial tiles,
    one row, the K-split plan of 512x512x4096), both output types."""
    _say(f"{M}x{N}x{K} out_f32={out_f32}")
    A, B, bias, old32, old16 = _case(M, N, K, 1)
    _run_and_check(oracle_mod, A, B, bias, old32, old16, -0.75, 0.5, out_f32, f"{M}x{N}x{K}")


@pytest.mark.parametrize("alpha,beta,use_bias", [(1.0, 0.0, True), (1.0, 1.0, False), (2.0, -1.0, True),
                                                 (0.5, 0.0, False)])
def test_affine_coefficients(oracle_mod, alpha, beta, use_bias):
    """The common cases: bias only, a residual add (beta = 1), scaling."""
    _say(f"alpha={alpha} beta={beta} bias={use_bias}")
    A, B, bias, old32, old16 = _case(300, 392, 520, 2)
    _run_and_check(oracle_mod, A, B, bias, old32, old16, alpha, beta, False, "coefficients", use_bias)


@pytest.mark.parametrize("cfg", ["bf16_256x192", "bf16_256x256", "bf16_128x128"])
def test_affine_every_config(oracle_mod, monkeypatch, cfg):
    """Each configuration compiled with the epilogue, forced, with padded row
    strides: A rows of 266 elements (4-byte copies) with K = 261, then
    16-byte rows with K = 264.  The padding of C holds NaN, which must stay
    (no write past N) and must not leak in (beta reads only C's columns)."""
    M, N = 300, 392
    for K, pa in ((261, 5), (264, 8)):
        _say(f"forced {cfg} {M}x{N}x{K} A pad {pa}")
        g = np.random.default_rng([gi.SEED_BASE + 5100, K, pa])
        A = gi.to_bf16_bits(gi.normal(g, (M, K + pa)))
        B = gi.to_bf16_bits(gi.normal(g, (K, N + 8), 0.125))
        bias = gi.to_bf16_bits(gi.normal(g, (N,)))
        old = gi.to_bf16_bits(gi.normal(g, (M, N)))
        Cfull = torch.full((M, N + 8), float("nan"), device="cuda", dtype=torch.bfloat16)
        Cfull[:, :N] = dev_bf16(old)
        monkeypatch.setenv("GEMM_FORCE_CONFIG", cfg)
        g5.gemm_bf16_affine(dev_bf16(A)[:, :K], dev_bf16(B)[:, :N], Cfull[:, :N], alpha=1.5, bias=dev_bf16(bias),
                            beta=-0.5, workspace=ws())
        monkeypatch.delenv("GEMM_FORCE_CONFIG")
        host = host_values(Cfull)
        Av, Bv = np.ascontiguousarray(A[:, :K]), np.ascontiguousarray(B[:, :N])
        ref = oracle_mod.gemm_bf16_affine(Av, Bv, 1.5, bias, -0.5, old)
        P = oracle_mod.gemm_bf16(Av, Bv)
        check_affine(host[:, :N], ref, P, K, 1.5, gi.bf16_bits_to_f32(bias).astype(np.float64), -0.5,
                     gi.bf16_bits_to_f32(old).astype(np.float64), False, what=cfg)
        assert np.all(np.isnan(host[:, N:])), f"{cfg}: output padding was written"


@pytest.mark.parametrize("S", [2, 3, 5])
def test_affine_ksplit(oracle_mod, monkeypatch, S):
    """K split over S workgroups per tile: the last to arrive applies the
    epilogue once (beta * C read once: a second application would show as
    an error of beta^2 C)."""
    _say(f"ksplit {S}")
    A, B, bias, old32, old16 = _case(200, 264, 1024, 3)
    monkeypatch.setenv("GEMM_FORCE_CONFIG", "bf16_128x128")
    monkeypatch.setenv("GEMM_FORCE_KSPLIT", str(S))
    st, plan = g5.plan_query(g5.GEMM_OP_BF16_AFFINE, 200, 264, 1024, c_type=1)
    assert st == 0 and plan.ksplit == S
    _run_and_check(oracle_mod, A, B, bias, old32, old16, 1.0, 2.0, True, f"ksplit {S}")


def test_affine_batched_broadcast(oracle_mod):
    """Batched entries with their own A and C and one shared B (batch stride
    0) and bias."""
    _say("batched")
    A, B, bias, old32, old16 = _case(130, 136, 200, 4, batch=3)
    B = np.broadcast_to(B[:1], B.shape).copy()
    dA, dB1 = dev_bf16(A), dev_bf16(B[0])
    C = dev_bf16(old16)
    g5.gemm_bf16_affine(dA, dB1.unsqueeze(0).expand(3, -1, -1), C, alpha=1.0, bias=dev_bf16(bias), beta=1.0, workspace=ws())
    got = host_values(C)
    for b in range(3):
        ref = oracle_mod.gemm_bf16_affine(A[b], B[b], 1.0, bias, 1.0, old16[b])
        check_affine(got[b], ref, oracle_mod.gemm_bf16(A[b], B[b]), 200, 1.0,
                     gi.bf16_bits_to_f32(bias).astype(np.float64), 1.0,
                     gi.bf16_bits_to_f32(old16[b]).astype(np.float64), False, what=f"batched {b}")


def test_affine_without_product():
    """alpha = 0 reads neither A nor B (NaN there does not propagate) and K = 0
    forms no product: C := bias + beta * C, each rounded once; beta = 0 does
    not read C (NaN there does not propagate)."""
    M, N, K = 70, 136, 64
    g = np.random.default_rng([gi.SEED_BASE + 5200])
    bias = gi.to_bf16_bits(gi.normal(g, (N,)))
    old = gi.normal(g, (M, N))
    bv = gi.bf16_bits_to_f32(bias)
    want = (bv[None, :].astype(np.float64) - 2.0 * old).astype(np.float32)   # exact in double, one rounding
    nanA = torch.full((M, K), float("nan"), device="cuda", dtype=torch.bfloat16)
    nanB = torch.full((K, N), float("nan"), device="cuda", dtype=torch.bfloat16)
    C = dev_f32(old)
    g5.gemm_bf16_affine(nanA, nanB, C, alpha=0.0, bias=dev_bf16(bias), beta=-2.0, workspace=ws())
    assert np.array_equal(host_values(C).astype(np.float32), want)
    C = dev_f32(old)
    g5.gemm_bf16_affine(nanA[:, :0], nanB[:0], C, alpha=3.0, bias=dev_bf16(bias), beta=-2.0, workspace=ws())
    assert np.array_equal(host_values(C).astype(np.float32), want)
    Cb = torch.full((M, N), float("nan"), device="cuda", dtype=torch.bfloat16)
    g5.gemm_bf16_affine(nanA[:, :0], nanB[:0], Cb, alpha=1.0, bias=dev_bf16(bias), beta=0.0, workspace=ws())
    assert np.array_equal(host_values(Cb), np.broadcast_to(bv, (M, N)).astype(np.float64))
    A, B, _, _, _ = _case(M, N, K, 5)
    Cn = torch.full((M, N), float("nan"), device="cuda", dtype=torch.float32)
    g5.gemm_bf16_affine(dev_bf16(A[0]), dev_bf16(B[0]), Cn, alpha=1.0, bias=None, beta=0.0, workspace=ws())
    assert torch.isfinite(Cn).all()


@pytest.mark.parametrize("S", [1, 3])
def test_affine_identity_matches_plain_product(monkeypatch, S):
    """alpha = 1, no bias, beta = 0 gives gemm_bf16's values exactly on the
    same tile configuration and K split: the same FP32 sums, and
    fma(1, s, 0) = s (up to the sign of zero)."""
    A, B, _, _, _ = _case(300, 392, 640, 6)
    dA, dB = dev_bf16(A[0]), dev_bf16(B[0])
    monkeypatch.setenv("GEMM_FORCE_CONFIG", "bf16_128x128")
    monkeypatch.setenv("GEMM_FORCE_KSPLIT", str(S))
    for out in (torch.bfloat16, torch.float32):
        plain = g5.gemm_bf16(dA, dB, out_dtype=out, workspace=ws())
        C = torch.empty_like(plain)
        g5.gemm_bf16_affine(dA, dB, C, workspace=ws())
        assert torch.equal(C.float(), plain.float()), out


@pytest.mark.parametrize("M,N,K,batch", [(1, 12288, 4096, 1), (4, 12288, 4096, 1), (16, 12288, 4096, 1),
                                         (5, 200, 64, 2), (3, 1024, 1000, 1), (16, 384, 1024, 3)])
def test_affine_small_m(oracle_mod, M, N, K, batch):
    """M <= 16 on the small-M kernels (the K-split one for N % 128 == 0 and
    K % 32 == 0, else the whole-K one), bias and beta * C in both output
    types; the decode shape of the FFN at full size."""
    for out_f32 in (False, True):
        _say(f"small M {batch}x{M}x{N}x{K} out_f32={out_f32}")
        A, B, bias, old32, old16 = _case(M, N, K, 7, batch=batch)
        _run_and_check(oracle_mod, A, B, bias, old32, old16, 1.25, -1.0, out_f32, f"small M {M}x{N}x{K}")


def test_affine_small_m_rows_do_not_depend_on_m():
    """The small-M K partition does not depend on M: row 0 of an M = 1 call
    equals row 0 of an M = 16 call bit for bit, epilogue included."""
    A, B, bias, _, old16 = _case(16, 12288, 4096, 8)
    dA, dB, db = dev_bf16(A[0]), dev_bf16(B[0]), dev_bf16(bias)
    C16 = dev_bf16(old16[0])
    C1 = dev_bf16(old16[0][:1])
    g5.gemm_bf16_affine(dA, dB, C16, alpha=0.5, bias=db, beta=1.0, workspace=ws())
    g5.gemm_bf16_affine(dA[:1], dB, C1, alpha=0.5, bias=db, beta=1.0, workspace=ws())
    assert torch.equal(C1.view(torch.int16), C16[:1].view(torch.int16))


def test_affine_ffn_full_size(oracle_mod):
    """The FFN projection X[1024,4096] . W[4096,12288] with a bias and a
    residual add (beta = 1) into a bf16 C: rows from every row tile, all
    columns."""
    _say("ffn 1024x12288x4096 bias + residual")
    X, W = gi.ffn_inputs()
    g = np.random.default_rng([gi.SEED_BASE + 5300])
    bias = gi.to_bf16_bits(gi.normal(g, (12288,)))
    res = gi.to_bf16_bits(gi.normal(g, (1024, 12288)))
    C = dev_bf16(res)
    g5.gemm_bf16_affine(dev_bf16(X), dev_bf16(W), C, alpha=1.0, bias=dev_bf16(bias), beta=1.0, workspace=ws())
    rows = np.array([0, 255, 256, 700, 1023])
    Xs = np.ascontiguousarray(X[rows])
    ref = oracle_mod.gemm_bf16_affine(Xs, W, 1.0, bias, 1.0, np.ascontiguousarray(res[rows]))
    check_affine(host_values(C)[rows], ref, oracle_mod.gemm_bf16(Xs, W), 4096, 1.0,
                 gi.bf16_bits_to_f32(bias).astype(np.float64), 1.0,
                 gi.bf16_bits_to_f32(res[rows]).astype(np.float64), False, what="ffn rows")


# ------------------------------------------------------------ B given transposed

def _nt_check(oracle_mod, A, Bt, bias, old, alpha, beta, got, out_f32, what):
    B = np.ascontiguousarray(Bt.T)
    ref = oracle_mod.gemm_bf16_affine(A, B, alpha, bias, beta, old)
    old_vals = old.astype(np.float64) if out_f32 else gi.bf16_bits_to_f32(old).astype(np.float64)
    check_affine(got, ref, oracle_mod.gemm_bf16(A, B), A.shape[1], alpha,
                 gi.bf16_bits_to_f32(bias).astype(np.float64), beta, old_vals, out_f32,
                 amax_bf16(A), amax_bf16(Bt), what)


@pytest.mark.parametrize("cfg", [None, "bf16_256x192", "bf16_256x256", "bf16_128x128"])
@pytest.mark.parametrize("M,N,K,pb", [(300, 392, 264, 8), (257, 200, 1000, 0), (300, 392, 262, 0)])
def test_nt_affine_ragged(oracle_mod, monkeypatch, cfg, M, N, K, pb):
    """A linear layer's output with its bias and a residual (Bt [N, K]): every
    ring config with the transposed B and the epilogue, both output types;
    K = 262 gives 4-byte aligned Bt rows (realigned first)."""
    g = np.random.default_rng([gi.SEED_BASE + 5400, M, N, K, pb])
    A = gi.to_bf16_bits(gi.normal(g, (M, K)))
    Bt = gi.to_bf16_bits(gi.normal(g, (N, K + pb), 0.125))
    bias = gi.to_bf16_bits(gi.normal(g, (N,)))
    old32 = gi.normal(g, (M, N))
    old16 = gi.to_bf16_bits(old32)
    if cfg:
        monkeypatch.setenv("GEMM_FORCE_CONFIG", cfg)
    for out_f32 in (False, True):
        _say(f"nt affine {cfg} {M}x{N}x{K} out_f32={out_f32}")
        C = dev_f32(old32) if out_f32 else dev_bf16(old16)
        g5.gemm_bf16_nt_affine(dev_bf16(A), dev_bf16(Bt)[:, :K], C, alpha=0.75, bias=dev_bf16(bias), beta=1.0, workspace=ws())
        _nt_check(oracle_mod, A, np.ascontiguousarray(Bt[:, :K]), bias, old32 if out_f32 else old16, 0.75, 1.0,
                  host_values(C), out_f32, f"nt affine {cfg}")


@pytest.mark.parametrize("S", [2, 4])
def test_nt_affine_ksplit(oracle_mod, monkeypatch, S):
    _say(f"nt affine ksplit {S}")
    g = np.random.default_rng([gi.SEED_BASE + 5500, S])
    A = gi.to_bf16_bits(gi.normal(g, (200, 1024)))
    Bt = gi.to_bf16_bits(gi.normal(g, (264, 1024), 0.125))
    bias = gi.to_bf16_bits(gi.normal(g, (264,)))
    old = gi.normal(g, (200, 264))
    monkeypatch.setenv("GEMM_FORCE_CONFIG", "bf16_128x128")
    monkeypatch.setenv("GEMM_FORCE_KSPLIT", str(S))
    C = dev_f32(old)
    g5.gemm_bf16_nt_affine(dev_bf16(A), dev_bf16(Bt), C, alpha=1.0, bias=dev_bf16(bias), beta=-0.5, workspace=ws())
    _nt_check(oracle_mod, A, Bt, bias, old, 1.0, -0.5, host_values(C), True, f"nt affine split {S}")


@pytest.mark.parametrize("M,N,K,batch", [(1, 12288, 4096, 1), (16, 12288, 4096, 1), (5, 200, 72, 2), (3, 1000, 4104, 1)])
def test_nt_affine_small_m(oracle_mod, M, N, K, batch):
    """M <= 16 on the small-M transposed-B kernel with the epilogue (K tails,
    batched, both outputs): a decode step of a linear layer with bias and
    residual."""
    g = np.random.default_rng([gi.SEED_BASE + 5600, M, N, K, batch])
    A = gi.to_bf16_bits(gi.normal(g, (batch, M, K)))
    Bt = gi.to_bf16_bits(gi.normal(g, (batch, N, K), 0.125))
    bias = gi.to_bf16_bits(gi.normal(g, (N,)))
    old32 = gi.normal(g, (batch, M, N))
    old16 = gi.to_bf16_bits(old32)
    st, plan = g5.plan_query(g5.GEMM_OP_BF16_NT_AFFINE, M, N, K, batch=batch)
    assert st == 0 and plan.name == b"decode_nt"
    for out_f32 in (False, True):
        _say(f"nt affine small M {batch}x{M}x{N}x{K} out_f32={out_f32}")
        C = dev_f32(old32) if out_f32 else dev_bf16(old16)
        dA, dB = dev_bf16(A), dev_bf16(Bt)
        if batch == 1:
            g5.gemm_bf16_nt_affine(dA[0], dB[0], C[0], alpha=1.0, bias=dev_bf16(bias), beta=1.0, workspace=ws())
        else:
            g5.gemm_bf16_nt_affine(dA, dB, C, alpha=1.0, bias=dev_bf16(bias), beta=1.0, workspace=ws())
        got = host_values(C)
        for b in range(batch):
            _nt_check(oracle_mod, A[b], Bt[b], bias, (old32 if out_f32 else old16)[b], 1.0, 1.0, got[b], out_f32,
                      f"nt affine small M entry {b}")


def test_nt_affine_linear_layer_full_size(oracle_mod):
    """The FFN projection as a linear layer (weight [12288, 4096]) with bias
    and residual, bf16: sampled rows, all columns."""
    _say("nt affine 1024x12288x4096")
    X, W = gi.ffn_inputs()
    Wt = np.ascontiguousarray(W.T)
    g = np.random.default_rng([gi.SEED_BASE + 5700])
    bias = gi.to_bf16_bits(gi.normal(g, (12288,)))
    res = gi.to_bf16_bits(gi.normal(g, (1024, 12288)))
    C = dev_bf16(res)
    g5.gemm_bf16_nt_affine(dev_bf16(X), dev_bf16(Wt), C, alpha=1.0, bias=dev_bf16(bias), beta=1.0, workspace=ws())
    rows = np.array([0, 255, 256, 700, 1023])
    _nt_check(oracle_mod, np.ascontiguousarray(X[rows]), Wt, bias, np.ascontiguousarray(res[rows]), 1.0, 1.0,
              host_values(C)[rows], False, "nt affine FFN rows")


# ------------------------------------------------------------ A given transposed

@pytest.mark.parametrize("cfg", [None, "bf16_256x192", "bf16_256x256", "bf16_128x128"])
@pytest.mark.parametrize("M,N,K,pa", [(304, 392, 264, 8), (300, 200, 1000, 0)])
def test_tn_affine_ragged(oracle_mod, monkeypatch, cfg, M, N, K, pa):
    """At [K, M] with the affine epilogue on every transposed-A config; M = 300
    (not a multiple of 8) goes through the padded copy of At."""
    g = np.random.default_rng([gi.SEED_BASE + 5800, M, N, K, pa])
    At = gi.to_bf16_bits(gi.normal(g, (K, M + pa)))
    B = gi.to_bf16_bits(gi.normal(g, (K, N), 0.125))
    bias = gi.to_bf16_bits(gi.normal(g, (N,)))
    old32 = gi.normal(g, (M, N))
    old16 = gi.to_bf16_bits(old32)
    A = np.ascontiguousarray(At[:, :M].T)
    if cfg:
        monkeypatch.setenv("GEMM_FORCE_CONFIG", cfg)
    for out_f32 in (False, True):
        _say(f"tn affine {cfg} {M}x{N}x{K} out_f32={out_f32}")
        C = dev_f32(old32) if out_f32 else dev_bf16(old16)
        g5.gemm_bf16_tn_affine(dev_bf16(At)[:, :M], dev_bf16(B), C, alpha=-1.5, bias=dev_bf16(bias), beta=0.5, workspace=ws())
        old = old32 if out_f32 else old16
        ref = oracle_mod.gemm_bf16_affine(A, B, -1.5, bias, 0.5, old)
        old_vals = old.astype(np.float64) if out_f32 else gi.bf16_bits_to_f32(old).astype(np.float64)
        check_affine(host_values(C), ref, oracle_mod.gemm_bf16(A, B), K, -1.5,
                     gi.bf16_bits_to_f32(bias).astype(np.float64), 0.5, old_vals, out_f32, amax_bf16(A),
                     amax_bf16(B), f"tn affine {cfg}")


@pytest.mark.parametrize("S", [2, 3])
def test_tn_affine_ksplit(oracle_mod, monkeypatch, S):
    g = np.random.default_rng([gi.SEED_BASE + 5900, S])
    At = gi.to_bf16_bits(gi.normal(g, (1024, 200)))
    B = gi.to_bf16_bits(gi.normal(g, (1024, 264), 0.125))
    old = gi.normal(g, (200, 264))
    A = np.ascontiguousarray(At.T)
    monkeypatch.setenv("GEMM_FORCE_CONFIG", "bf16_128x128")
    monkeypatch.setenv("GEMM_FORCE_KSPLIT", str(S))
    C = dev_f32(old)
    g5.gemm_bf16_tn_affine(dev_bf16(At), dev_bf16(B), C, alpha=1.0, bias=None, beta=1.0, workspace=ws())
    ref = oracle_mod.gemm_bf16_affine(A, B, 1.0, None, 1.0, old)
    check_affine(host_values(C), ref, oracle_mod.gemm_bf16(A, B), 1024, 1.0, np.zeros(264), 1.0,
                 old.astype(np.float64), True, amax_bf16(A), amax_bf16(B), f"tn affine split {S}")


def test_tn_affine_gradient_accumulation_full_size(oracle_mod):
    """dW [4096, 12288] (float) += X^T . dY with X [1024, 4096], dY [1024, 12288]:
    two accumulation steps from a seeded dW, rows from every row tile."""
    _say("tn affine wgrad accumulation 4096x12288x1024")
    X, dY = gi.wgrad_inputs()
    g = np.random.default_rng([gi.SEED_BASE + 6000])
    dW0 = gi.normal(g, (4096, 12288))
    dX, dD = dev_bf16(X), dev_bf16(dY)
    C = dev_f32(dW0)
    g5.gemm_bf16_tn_affine(dX, dD, C, alpha=1.0, bias=None, beta=1.0, workspace=ws())
    g5.gemm_bf16_tn_affine(dX, dD, C, alpha=1.0, bias=None, beta=1.0, workspace=ws())
    rows = np.array([0, 255, 256, 2047, 4095])
    Xs = np.ascontiguousarray(X[:, rows].T)
    P = oracle_mod.gemm_bf16(Xs, dY)
    ref = dW0[rows].astype(np.float64) + 2.0 * P
    # two FP32 accumulations: each adds the FP32 bar of one product and
    # 2^-20 of the magnitudes combined
    bound = 2 * (1e-5 * 1024 * amax_bf16(X) * amax_bf16(dY)) + 2.0 ** -19 * (np.abs(ref) + 2 * np.abs(P))
    got = host_values(C[torch.from_numpy(rows).cuda()])
    err = np.abs(got - ref)
    assert np.all(err <= bound), f"max err {err.max()} (bound {bound.min()}..{bound.max()})"
