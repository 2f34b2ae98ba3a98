"""GPU parity of the FP8 (E4M3FN) path against the oracle, through the C ABI:
per-row quantization (gemm_fp8_quantize_rows, codes and factors bit for
bit) and the scaled FP8 product (gemm_fp8_nt).

Page "Operator & Runtime" (section 5.4.3, Examples 5-7 and 5-8): the whole
row's maximum sets the factor, the input is quantized once before the GEMM,
and the FP32 sums are dequantized by the row and column factors.
"""
import numpy as np
import pytest
import torch

import gemm_inputs as gi
from _gpu_helpers import check_bf16, dev_bf16, host_values, ws

import dense_gemm_05_amd as g5

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[fp8] {msg}", flush=True)


@pytest.fixture(autouse=True)
def _no_forced_config(monkeypatch):
    monkeypatch.delenv("GEMM_FORCE_CONFIG", raising=False)
    monkeypatch.delenv("GEMM_FORCE_KSPLIT", raising=False)
    monkeypatch.delenv("GEMM_QA_TILE_N", raising=False)


def dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def check_fp8(C, ref, K, amax_a, amax_b, out, what):
    """FP32 accumulation of exact products: the FP32 bar over the
    dequantized operands; a bf16 output adds one rounding (2^-8 |C_ref|)."""
    bound = 1e-5 * max(K, 1) * amax_a * amax_b + (2.0 ** -8 * np.abs(ref) if out == "bf16" else 0.0)
    err = np.abs(C - ref)
    assert np.all(np.isfinite(C)), f"{what}: non-finite output"
    bad = err > bound
    if np.any(bad):
        idx = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} out of bound, first at {idx}: got {C[idx]!r} want {ref[idx]!r}")


@pytest.mark.parametrize("rows,cols,ldx_pad,ldq_pad", [
    (7, 300, 0, 0), (64, 4096, 0, 0), (33, 1000, 5, 3), (5, 8, 0, 1), (3, 13, 2, 0), (300, 264, 8, 8),
    (4, 8192, 0, 0), (3, 9000, 4, 2),         # rows held in registers up to 4096; longer rows are read twice
    (2050, 1000, 3, 5), (4099, 4096, 0, 0),   # thousands of rows, ragged last workgroup
    (2049, 4100, 2, 0),
    (1024, 4096, 0, 0), (1025, 1000, 0, 0),   # the last size with four waves per row, the first with one
])
def test_quantize_rows_bit_exact(oracle_mod, rows, cols, ldx_pad, ldq_pad):
    """Codes and factors equal the oracle's bit for bit: normal rows of
    several magnitudes, a zero row, a row whose maximum is negative, a row
    with one nonzero, padded and odd row strides."""
    _say(f"quantize {rows}x{cols} pads {ldx_pad},{ldq_pad}")
    g = np.random.default_rng([gi.SEED_BASE + 7000, rows, cols])
    x = gi.normal(g, (rows, cols + ldx_pad))
    x *= np.float32(2.0) ** g.integers(-12, 12, (rows, 1)).astype(np.float32)
    x[0] = 0
    if rows > 1:
        x[1, :] = np.abs(x[1, :]) * 0.5
        x[1, cols // 2] = -np.float32(3.0)
    if rows > 2:
        x[2, :] = 0
        x[2, cols - 1] = np.float32(10.0)
    X = gi.to_bf16_bits(x)
    Qref, sref = oracle_mod.quantize_rows_e4m3(np.ascontiguousarray(X[:, :cols]))
    dX = dev_bf16(X)
    Qfull = torch.full((rows, cols + ldq_pad), 0xAB, dtype=torch.uint8, device="cuda")
    scale = torch.full((rows,), float("nan"), dtype=torch.float32, device="cuda")
    g5.gemm_fp8_quantize_rows(dX[:, :cols], Qfull[:, :cols], scale)
    Q = Qfull.cpu().numpy()
    assert np.array_equal(Q[:, :cols], Qref), f"{int((Q[:, :cols] != Qref).sum())} codes differ"
    assert np.array_equal(scale.cpu().numpy().view(np.uint32), sref.view(np.uint32)), "factors differ"
    assert np.all(Q[:, cols:] == 0xAB), "row padding of Q was written"


# (x, amax) pairs of bf16 values whose exact quotient x * 448 / amax lies on
# the midpoint of two E4M3FN neighbours (200, 84, 336, 1.5625, 0.65625, 184):
# the exact rule of Example 5-7 takes the even code.
_TIES = [(0.00133514404296875, 0.00299072265625), (0.001190185546875, 0.00634765625),
         (0.0047607421875, 0.00634765625), (0.00133514404296875, 0.3828125),
         (0.001190185546875, 0.8125), (0.00122833251953125, 0.00299072265625)]


def test_quantize_rows_exact_ties(oracle_mod):
    """Quotients exactly on a midpoint, both signs, amax given by a negative
    element, and a wide row of random multiples of the tie numerators: the
    kernel's codes equal the oracle's exact ones bit for bit."""
    _say("quantize exact ties")
    g = np.random.default_rng([gi.SEED_BASE + 7050])
    rows = []
    for x, amax in _TIES:
        r = np.zeros(64, np.float32)
        r[0], r[1], r[2] = x, -amax, -x
        # more exact ties of the same row: x * 2^j stays a bf16 value below amax
        for j, e in enumerate(range(-6, 0)):
            r[3 + j] = np.float32(x) * np.float32(2.0 ** e)
        r[10:] = (g.random(54).astype(np.float32) * 2 - 1) * np.float32(amax)
        rows.append(r)
    X = gi.to_bf16_bits(np.stack(rows))
    Qref, sref = oracle_mod.quantize_rows_e4m3(X)
    Q, scale = g5.gemm_fp8_quantize_rows(dev_bf16(X))
    assert np.array_equal(Q.cpu().numpy(), Qref), f"{int((Q.cpu().numpy() != Qref).sum())} codes differ"
    assert np.array_equal(scale.cpu().numpy().view(np.uint32), sref.view(np.uint32)), "factors differ"


def _fp8_case(M, N, K, seed, pa=0, pb=0, scales=True):
    g = np.random.default_rng([gi.SEED_BASE + 7100 + seed, M, N, K, pa, pb])
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    # codes spread over the whole range, weighted to moderate magnitudes
    A = g.choice(finite, (M, K + pa))
    Bt = g.choice(finite, (N, K + pb))
    sa = (2.0 ** g.uniform(-8, -4, M)).astype(np.float32) if scales else None
    sb = (2.0 ** g.uniform(-8, -4, N)).astype(np.float32) if scales else None
    return A, Bt, sa, sb


def _amax(oracle_mod, codes, s):
    d = np.abs(oracle_mod.e4m3_decode(np.unique(codes)))
    return float(d.max()) * (float(np.abs(s).max()) if s is not None else 1.0)


@pytest.mark.parametrize("cfg", [None, "bf16_256x192", "bf16_256x256", "bf16_128x128"])
@pytest.mark.parametrize("M,N,K,pa,pb,scales", [
    (300, 392, 256, 0, 0, True),     # 16-byte rows, ragged M and N
    (300, 392, 260, 0, 12, True),    # A rows 4-byte aligned (4-byte copies), K tail of 4
    (257, 190, 1000, 8, 8, False),   # no factors, K tail of 40
    (512, 384, 128, 0, 0, True),     # whole tiles for 128x128
])
def test_fp8_nt_parity(oracle_mod, monkeypatch, cfg, M, N, K, pa, pb, scales):
    _say(f"fp8 {cfg} {M}x{N}x{K} pads {pa},{pb} scales {scales}")
    A, Bt, sa, sb = _fp8_case(M, N, K, 1, pa, pb, scales)
    ref = oracle_mod.gemm_fp8_nt(np.ascontiguousarray(A[:, :K]), sa, np.ascontiguousarray(Bt[:, :K]), sb)
    dA, dB = dev_u8(A), dev_u8(Bt)
    dsa = None if sa is None else torch.from_numpy(sa).cuda()
    dsb = None if sb is None else torch.from_numpy(sb).cuda()
    if cfg:
        monkeypatch.setenv("GEMM_FORCE_CONFIG", cfg)
    am, bm = _amax(oracle_mod, A[:, :K], sa), _amax(oracle_mod, Bt[:, :K], sb)
    for out, od in (("f32", torch.float32), ("bf16", torch.bfloat16)):
        Cfull = torch.full((M, N + 4), float("nan"), device="cuda", dtype=od)
        g5.gemm_fp8_nt(dA[:, :K], dsa, dB[:, :K], dsb, Cfull[:, :N], workspace=ws())
        host = host_values(Cfull)
        check_fp8(host[:, :N], ref, K, am, bm, out, f"fp8 {cfg} {out}")
        assert np.all(np.isnan(host[:, N:])), "ldc padding was written"


@pytest.mark.parametrize("S", [2, 3])
def test_fp8_nt_ksplit(oracle_mod, monkeypatch, S):
    M, N, K = 200, 264, 1024
    A, Bt, sa, sb = _fp8_case(M, N, K, 2)
    monkeypatch.setenv("GEMM_FORCE_CONFIG", "bf16_128x128")
    monkeypatch.setenv("GEMM_FORCE_KSPLIT", str(S))
    C = g5.gemm_fp8_nt(dev_u8(A), torch.from_numpy(sa).cuda(), dev_u8(Bt), torch.from_numpy(sb).cuda(),
                       out_dtype=torch.float32, workspace=ws())
    ref = oracle_mod.gemm_fp8_nt(A, sa, Bt, sb)
    check_fp8(host_values(C), ref, K, _amax(oracle_mod, A, sa), _amax(oracle_mod, Bt, sb), "f32", f"fp8 split {S}")


def test_fp8_small_integers_exact(oracle_mod):
    """Codes of small integers and power-of-two factors: every partial sum is
    an integer below 2^24, so the FP32 result is exact, bit for bit."""
    g = np.random.default_rng(5)
    M, N, K = 260, 200, 512
    vals = np.arange(-6, 7, dtype=np.float64)
    A = oracle_mod.e4m3_encode(g.choice(vals, (M, K)))
    Bt = oracle_mod.e4m3_encode(g.choice(vals, (N, K)))
    sa = (2.0 ** g.integers(-3, 3, M)).astype(np.float32)
    sb = (2.0 ** g.integers(-3, 3, N)).astype(np.float32)
    C = g5.gemm_fp8_nt(dev_u8(A), torch.from_numpy(sa).cuda(), dev_u8(Bt), torch.from_numpy(sb).cuda(),
                       out_dtype=torch.float32, workspace=ws())
    assert np.array_equal(host_values(C), oracle_mod.gemm_fp8_nt(A, sa, Bt, sb))


def test_fp8_ffn_end_to_end(oracle_mod):
    """The FFN projection in FP8: X [1024,4096] quantized per row (tokens),
    W^T [12288,4096] quantized per row (output channels), both on the GPU
    (codes bit-exact with the oracle's), then the scaled product against
    the oracle on sampled rows."""
    _say("fp8 FFN 1024x12288x4096")
    X, W = gi.ffn_inputs()
    Wt = np.ascontiguousarray(W.T)
    qX, sX = g5.gemm_fp8_quantize_rows(dev_bf16(X))
    qW, sW = g5.gemm_fp8_quantize_rows(dev_bf16(Wt))
    rX, rsX = oracle_mod.quantize_rows_e4m3(X)
    rows = np.array([0, 1, 255, 256, 511, 777, 1023])
    assert np.array_equal(qX.cpu().numpy(), rX) and np.array_equal(sX.cpu().numpy(), rsX)
    rW, rsW = oracle_mod.quantize_rows_e4m3(Wt)
    assert np.array_equal(qW.cpu().numpy(), rW) and np.array_equal(sW.cpu().numpy(), rsW)
    st, plan = g5.plan_query(g5.GEMM_OP_FP8_NT, 1024, 12288, 4096)
    assert st == 0 and plan.name == b"bf16_256x192" and plan.variant == 1
    C = g5.gemm_fp8_nt(qX, sX, qW, sW, workspace=ws())
    ref = oracle_mod.gemm_fp8_nt(np.ascontiguousarray(rX[rows]), rsX[rows], rW, rsW)
    check_fp8(host_values(C)[rows], ref, 4096, _amax(oracle_mod, rX, rsX), _amax(oracle_mod, rW, rsW), "bf16",
              "fp8 FFN rows")


@pytest.mark.parametrize("M,N,K,pb,scales", [(1, 12288, 4096, 0, True), (4, 1000, 4100, 12, True),
                                             (16, 392, 256, 0, False), (7, 200, 72, 8, True), (3, 40, 8, 8, True)])
def test_fp8_nt_small_m(oracle_mod, M, N, K, pb, scales):
    """M <= 16 with 16-byte aligned Bt rows: the FP8 GEMV over the rows of Bt
    (decode_nt); ragged N, K tails (K % 64 != 0), with and without factors,
    both outputs, NaN padding of C untouched."""
    _say(f"fp8 small M {M}x{N}x{K} pb {pb} scales {scales}")
    A, Bt, sa, sb = _fp8_case(M, N, K, 3, 0, pb, scales)
    st, plan = g5.plan_query(g5.GEMM_OP_FP8_NT, M, N, K, ldb=K + pb)
    assert st == 0 and plan.name == b"decode_nt"
    ref = oracle_mod.gemm_fp8_nt(A, sa, np.ascontiguousarray(Bt[:, :K]), sb)
    dA, dB = dev_u8(A), dev_u8(Bt)
    dsa = None if sa is None else torch.from_numpy(sa).cuda()
    dsb = None if sb is None else torch.from_numpy(sb).cuda()
    am, bm = _amax(oracle_mod, A, sa), _amax(oracle_mod, Bt[:, :K], sb)
    for out, od in (("f32", torch.float32), ("bf16", torch.bfloat16)):
        Cfull = torch.full((M, N + 4), float("nan"), device="cuda", dtype=od)
        g5.gemm_fp8_nt(dA, dsa, dB[:, :K], dsb, Cfull[:, :N], workspace=ws())
        host = host_values(Cfull)
        check_fp8(host[:, :N], ref, K, am, bm, out, f"fp8 small M {out}")
        assert np.all(np.isnan(host[:, N:])), "ldc padding was written"


def test_fp8_small_m_exact_and_row_invariant(oracle_mod):
    """Small-integer codes with power-of-two factors through the small-M path
    give the oracle's bits; the rows of an M = 1 and an M = 5 call equal the
    same rows of an M = 16 call (the K partition does not depend on M)."""
    g = np.random.default_rng(6)
    N, K = 392, 1000
    vals = np.arange(-6, 7, dtype=np.float64)
    A = oracle_mod.e4m3_encode(g.choice(vals, (16, K)))
    Bt = oracle_mod.e4m3_encode(g.choice(vals, (N, K + 8)))
    sa = (2.0 ** g.integers(-3, 3, 16)).astype(np.float32)
    sb = (2.0 ** g.integers(-3, 3, N)).astype(np.float32)
    dA, dB = dev_u8(A), dev_u8(Bt)[:, :K]
    dsa, dsb = torch.from_numpy(sa).cuda(), torch.from_numpy(sb).cuda()
    c16 = g5.gemm_fp8_nt(dA, dsa, dB, dsb, out_dtype=torch.float32, workspace=ws())
    assert np.array_equal(host_values(c16), oracle_mod.gemm_fp8_nt(A, sa, np.ascontiguousarray(Bt[:, :K]), sb))
    for M in (1, 5):
        cm = g5.gemm_fp8_nt(dA[:M], dsa[:M], dB, dsb, out_dtype=torch.float32, workspace=ws())
        assert torch.equal(cm.view(torch.int32), c16[:M].view(torch.int32)), f"M={M}"


# ------------------------------------------------ weights stored [K, N]
@pytest.mark.parametrize("K,N,ldw_pad,ldq_pad", [(64, 64, 0, 0), (300, 130, 6, 3), (4096, 200, 0, 0),
                                                 (1000, 77, 1, 16), (5, 9, 0, 0)])
def test_quantize_cols_bit_exact(oracle_mod, K, N, ldw_pad, ldq_pad):
    """Per-column quantization of a weight stored [K, N] into the rows of
    Qt [N, K]: codes and factors equal the oracle's bit for bit; columns of
    several magnitudes, a zero column, a column whose maximum is negative;
    padded and odd strides, row padding of Qt untouched."""
    _say(f"quantize cols {K}x{N} pads {ldw_pad},{ldq_pad}")
    g = np.random.default_rng([gi.SEED_BASE + 7300, K, N])
    w = gi.normal(g, (K, N + ldw_pad)) * np.float32(2.0) ** g.integers(-10, 10, (1, N + ldw_pad)).astype(np.float32)
    w[:, 0] = 0
    if N > 1:
        w[K // 2, 1] = -np.float32(1e3)
    W = gi.to_bf16_bits(w)
    Qref, sref = oracle_mod.quantize_cols_e4m3(np.ascontiguousarray(W[:, :N]))
    Qfull = torch.full((N, K + ldq_pad), 0xAB, dtype=torch.uint8, device="cuda")
    scale = torch.full((N,), float("nan"), dtype=torch.float32, device="cuda")
    g5.gemm_fp8_quantize_cols(dev_bf16(W)[:, :N], Qfull[:, :K], scale)
    Q = Qfull.cpu().numpy()
    assert np.array_equal(Q[:, :K], Qref), f"{int((Q[:, :K] != Qref).sum())} codes differ"
    assert np.array_equal(scale.cpu().numpy().view(np.uint32), sref.view(np.uint32)), "factors differ"
    assert np.all(Q[:, K:] == 0xAB), "row padding of Qt was written"


def test_fp8_example_5_8_weight_k_by_n(oracle_mod):
    """Operator & Runtime §5.4.3, Example 5-8: a [4096, 4096] input quantized
    per row, an FP8 weight [4096, 1536] stored [K, N] (quantized per output
    column into Bt), 16-bit output; sampled rows of every column against
    the oracle, the codes of both operands bit-exact."""
    _say("fp8 Example 5-8 shape 4096x1536x4096")
    g = np.random.default_rng([gi.SEED_BASE + 7400])
    X = gi.to_bf16_bits(gi.normal(g, (4096, 4096)))
    W = gi.to_bf16_bits(gi.normal(g, (4096, 1536), 0.125))
    qX, sX = g5.gemm_fp8_quantize_rows(dev_bf16(X))
    qW, sW = g5.gemm_fp8_quantize_cols(dev_bf16(W))
    rX, rsX = oracle_mod.quantize_rows_e4m3(X)
    rW, rsW = oracle_mod.quantize_cols_e4m3(W)
    assert np.array_equal(qX.cpu().numpy(), rX) and np.array_equal(sX.cpu().numpy(), rsX)
    assert np.array_equal(qW.cpu().numpy(), rW) and np.array_equal(sW.cpu().numpy(), rsW)
    C = g5.gemm_fp8_nt(qX, sX, qW, sW, workspace=ws())
    rows = np.array([0, 1, 127, 128, 2047, 3000, 4095])
    ref = oracle_mod.gemm_fp8_nt(np.ascontiguousarray(rX[rows]), rsX[rows], rW, rsW)
    check_fp8(host_values(C)[rows], ref, 4096, _amax(oracle_mod, rX, rsX), _amax(oracle_mod, rW, rsW), "bf16",
              "Example 5-8 rows")


# ------------------------------------------------ batched FP8 products
@pytest.mark.parametrize("with_ws", [True, False])
@pytest.mark.parametrize("M,N,K", [(300, 392, 256), (5, 392, 320)])
@pytest.mark.parametrize("bcast", ["none", "a", "b"])
def test_fp8_nt_batched(oracle_mod, M, N, K, bcast, with_ws):
    """A batch of scaled FP8 products (the experts of an MoE layer): each
    entry its own codes and factors, or one operand (and its factors)
    broadcast along the batch; tiled (M = 300) and small-M (M = 5) paths."""
    batch = 3
    _say(f"fp8 batched {batch}x{M}x{N}x{K} broadcast {bcast} ws={with_ws}")
    cases = [_fp8_case(M, N, K, 10 + b) for b in range(batch)]
    A = np.stack([c[0] for c in cases])
    Bt = np.stack([c[1] for c in cases])
    sa = np.stack([c[2] for c in cases])
    sb = np.stack([c[3] for c in cases])
    dA, dB = dev_u8(A), dev_u8(Bt)
    dsa, dsb = torch.from_numpy(sa).cuda(), torch.from_numpy(sb).cuda()
    if bcast == "a":
        dA, dsa = dA[:1].expand(batch, -1, -1), dsa[0]
    if bcast == "b":
        dB, dsb = dB[:1].expand(batch, -1, -1), dsb[0]
    C = g5.gemm_fp8_nt(dA, dsa, dB, dsb, out_dtype=torch.float32, workspace=ws() if with_ws else None)
    got = host_values(C)
    for b in range(batch):
        ia = 0 if bcast == "a" else b
        ib = 0 if bcast == "b" else b
        ref = oracle_mod.gemm_fp8_nt(A[ia], sa[ia], Bt[ib], sb[ib])
        check_fp8(got[b], ref, K, _amax(oracle_mod, A[ia], sa[ia]), _amax(oracle_mod, Bt[ib], sb[ib]), "f32",
                  f"fp8 batched entry {b}")


# ------------------------------------------------ FP8 with the affine epilogue
def _check_fp8_affine(C, ref, D, K, am, bm, alpha, bias_vals, beta, old_vals, out, what):
    """The FP32 accumulation bar on D scaled by |alpha|, the FP32 epilogue's
    fused multiply-adds (2^-20 of the magnitudes), and a bf16 output's
    rounding (2^-8 |C_ref|)."""
    mags = np.abs(alpha * D) + np.abs(bias_vals)[None, :] + np.abs(beta * old_vals)
    bound = abs(alpha) * 1e-5 * max(K, 1) * am * bm + 2.0 ** -20 * mags
    if out == "bf16":
        bound = bound + 2.0 ** -8 * np.abs(ref)
    err = np.abs(C - ref)
    assert np.all(np.isfinite(C)), f"{what}: non-finite output"
    bad = err > bound
    if np.any(bad):
        idx = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} out of bound, first at {idx}: got {C[idx]!r} want {ref[idx]!r}")


@pytest.mark.parametrize("cfg", [None, "bf16_256x256", "bf16_128x128"])
@pytest.mark.parametrize("M,N,K", [(300, 392, 256), (7, 200, 144), (512, 384, 1024)])
def test_fp8_nt_affine(oracle_mod, monkeypatch, cfg, M, N, K):
    """C := alpha * (scaled FP8 product) + bias + beta * C, both outputs,
    tiled and small-M paths (a forced config applies to M > 16 only)."""
    if cfg and M <= 16:
        pytest.skip("small M runs on the GEMV kernel")
    _say(f"fp8 affine {cfg} {M}x{N}x{K}")
    A, Bt, sa, sb = _fp8_case(M, N, K, 20)
    g = np.random.default_rng([gi.SEED_BASE + 7500, M])
    bias = gi.to_bf16_bits(gi.normal(g, (N,)))
    bv = gi.bf16_bits_to_f32(bias).astype(np.float64)
    if cfg:
        monkeypatch.setenv("GEMM_FORCE_CONFIG", cfg)
    am, bm = _amax(oracle_mod, A, sa), _amax(oracle_mod, Bt, sb)
    D = oracle_mod.gemm_fp8_nt(A, sa, Bt, sb)
    dA, dB = dev_u8(A), dev_u8(Bt)
    dsa, dsb, db = torch.from_numpy(sa).cuda(), torch.from_numpy(sb).cuda(), dev_bf16(bias)
    for out, od in (("f32", torch.float32), ("bf16", torch.bfloat16)):
        old = gi.normal(g, (M, N)).astype(np.float32)
        if od == torch.bfloat16:
            old_bits = gi.to_bf16_bits(old)
            C = dev_bf16(old_bits)
            ov = gi.bf16_bits_to_f32(old_bits).astype(np.float64)
            C_old = old_bits
        else:
            C = torch.from_numpy(old).cuda()
            ov = old.astype(np.float64)
            C_old = old
        alpha, beta = 0.5, -1.25
        g5.gemm_fp8_nt_affine(dA, dsa, dB, dsb, C, alpha=alpha, bias=db, beta=beta, workspace=ws())
        ref = oracle_mod.gemm_fp8_nt_affine(A, sa, Bt, sb, alpha=alpha, bias=bias, beta=beta, C_old=C_old)
        _check_fp8_affine(host_values(C), ref, D, K, am, bm, alpha, bv, beta, ov, out, f"fp8 affine {cfg} {out}")


# ------------------------------------------------ quantization inside the GEMM
@pytest.mark.parametrize("tile_n", ["auto", "128", "256"])
@pytest.mark.parametrize("M,N,K", [(300, 392, 256), (257, 200, 320), (4096, 1536, 1024), (1, 128, 64),
                                   (130, 1000, 4096)])
def test_fp8_quant_a_equals_separate(oracle_mod, monkeypatch, M, N, K, tile_n):
    """Example 5-8's fused alternative: X quantized inside the GEMM gives the
    factors of gemm_fp8_quantize_rows bit for bit and the C of the separate
    path on 128x128 tiles bit for bit, with 128- or 256-column tiles (each
    output's sum is the same sequence of MFMAs: whole stage pairs, K % 128
    == 0, or an odd stage count); ragged M and N; also within the FP8 bar
    of the oracle."""
    _say(f"fp8 quant-A {M}x{N}x{K} tile_n {tile_n}")
    if tile_n != "auto":
        monkeypatch.setenv("GEMM_QA_TILE_N", tile_n)
    g = np.random.default_rng([gi.SEED_BASE + 7600, M, N, K])
    X = gi.to_bf16_bits(gi.normal(g, (M, K)) * np.float32(2.0) ** g.integers(-6, 6, (M, 1)).astype(np.float32))
    Wt = gi.to_bf16_bits(gi.normal(g, (N, K), 0.125))
    dX = dev_bf16(X)
    qW, sW = g5.gemm_fp8_quantize_rows(dev_bf16(Wt))
    qX, sX = g5.gemm_fp8_quantize_rows(dX)
    monkeypatch.setenv("GEMM_FORCE_CONFIG", "bf16_128x128")
    monkeypatch.setenv("GEMM_FORCE_KSPLIT", "1")
    C_sep = g5.gemm_fp8_nt(qX, sX, qW, sW, out_dtype=torch.float32, workspace=ws())
    C_f, sX_f = g5.gemm_fp8_nt_quant_a(dX, qW, sW, out_dtype=torch.float32, workspace=ws())
    assert torch.equal(sX_f.view(torch.int32), sX.view(torch.int32)), "row factors differ"
    assert torch.equal(C_f.view(torch.int32), C_sep.view(torch.int32)), \
        f"{int((C_f != C_sep).sum())} of {M * N} outputs differ from the separate path"
    rX, rsX = oracle_mod.quantize_rows_e4m3(X)
    rW, rsW = oracle_mod.quantize_rows_e4m3(Wt)
    rows = np.unique(np.linspace(0, M - 1, min(M, 9)).astype(int))
    ref = oracle_mod.gemm_fp8_nt(np.ascontiguousarray(rX[rows]), rsX[rows], rW, rsW)
    check_fp8(host_values(C_f)[rows], ref, K, _amax(oracle_mod, rX, rsX), _amax(oracle_mod, rW, rsW), "f32",
              "fp8 quant-A rows")


def test_fp8_quant_a_bf16_out_and_repeat():
    """bf16 output, the same bits on a second call with a caller tensor as
    workspace, and the nearest-code rule at exact ties inside the GEMM."""
    M, N, K = 64, 256, 128
    g = np.random.default_rng([gi.SEED_BASE + 7650])
    x = gi.normal(g, (M, K))
    for i, (t, amax) in enumerate(_TIES):                   # quotients exactly on midpoints
        x[i, 0], x[i, 1] = t, -amax
    X = gi.to_bf16_bits(x)
    dX = dev_bf16(X)
    qW, sW = g5.gemm_fp8_quantize_rows(dev_bf16(gi.to_bf16_bits(gi.normal(g, (N, K), 0.125))))
    wsb = torch.zeros(g5.GEMM_WORKSPACE_COUNTER_BYTES + 4096, dtype=torch.uint8, device="cuda")
    C1, s1 = g5.gemm_fp8_nt_quant_a(dX, qW, sW, workspace=wsb)
    C2, s2 = g5.gemm_fp8_nt_quant_a(dX, qW, sW, workspace=wsb)
    assert torch.equal(C1.view(torch.int16), C2.view(torch.int16)) and torch.equal(s1, s2)
    qX, sX = g5.gemm_fp8_quantize_rows(dX)
    C_sep = g5.gemm_fp8_nt(qX, sX, qW, sW)
    # (the separate product may take other tiles: compare within the bar)
    assert torch.equal(s1.view(torch.int32), sX.view(torch.int32))
    got, ref = host_values(C1), host_values(C_sep)
    assert np.all(np.abs(got - ref) <= 2.0 ** -7 * np.abs(ref) + 1e-6)


def _fp8_midpoints():
    """Every positive rounding midpoint of E4M3FN below 448: (2f+1)·2^-10
    between subnormals, T·2^(E-4) (T odd, 17..31) between normals."""
    mids = [(2 * f + 1) * 2.0 ** -10 for f in range(8)]
    mids += [T * 2.0 ** (E - 4) for E in range(-6, 9) for T in range(17, 32, 2) if T * 2.0 ** (E - 4) < 448]
    return np.array(mids, np.float64)


@pytest.mark.parametrize("tile_n", ["128", "256"])
def test_fp8_quant_a_codes_exact(oracle_mod, monkeypatch, tile_n):
    """The codes made inside the GEMM equal the oracle's exact ones bit for
    bit, including rows whose quotients sit exactly on rounding midpoints
    (amax = 7·2^k or 448), next to them (amax = 1, 3), bf16 subnormals, -0,
    and row maxima at and beyond both ends of the range where the kernel
    uses the reciprocal-and-residual quotient (2^-126 and 2^118) as well as
    outside it (2^-127, 2^-130, 2^119, just above 2^118).  Bt is the
    identity in codes (1.0 = 0x38) with factors 1, so C[m, n] is the code of
    X[m, n] times the row factor, one rounding, which separates every code
    (but not the two zeros)."""
    K = N = 256
    amaxes = [1.0, 3.0, 7.0, 448.0, 7 * 2.0 ** -40, 7 * 2.0 ** 60, 2.0 ** -126, 1.5 * 2.0 ** -126,
              2.0 ** -127, 2.0 ** -130, 2.0 ** 118, 1.0078125 * 2.0 ** 118, 2.0 ** 119, 0.3828125]
    g = np.random.default_rng([gi.SEED_BASE + 7700])
    mids = _fp8_midpoints()
    rows = []
    for amax in amaxes:
        for variant in range(3):
            x = np.zeros(K, np.float64)
            x[0] = amax if variant != 1 else -amax
            t = mids * amax / 448.0
            x[1:1 + len(t)] = t * np.where(g.random(len(t)) < 0.5, -1.0, 1.0)
            rest = 1 + len(t)
            if variant == 2:                                   # neighbours of the midpoints
                near = np.resize(x[1:rest], K - rest)             # the midpoint quotients, cycled
                x[rest:] = np.nextafter(near.astype(np.float32), np.float32(np.inf)).astype(np.float64) * 1.003
            else:
                x[rest:] = g.uniform(-amax, amax, K - rest)
            x[rest] = -0.0
            x[rest + 1] = 2.0 ** -133                          # bf16 subnormals
            x[rest + 2] = -3 * 2.0 ** -131
            rows.append(np.clip(x, -amax, amax))
    M = len(rows)
    X = gi.to_bf16_bits(np.array(rows, np.float32))
    assert np.all(np.isfinite(gi.bf16_bits_to_f32(X)))
    _say(f"fp8 quant-A codes {M}x{N}x{K} tile_n {tile_n}")
    monkeypatch.setenv("GEMM_QA_TILE_N", tile_n)
    ident = np.zeros((N, K), np.uint8)
    ident[np.arange(N), np.arange(K)] = 0x38
    qI = dev_u8(ident)
    ones = torch.ones(N, dtype=torch.float32, device="cuda")
    C, sX = g5.gemm_fp8_nt_quant_a(dev_bf16(X), qI, ones, out_dtype=torch.float32, workspace=ws())
    codes, scales = oracle_mod.quantize_rows_e4m3(X)
    assert np.array_equal(sX.cpu().numpy().view(np.int32), scales.astype(np.float32).view(np.int32))
    expect = (oracle_mod.e4m3_decode(codes).astype(np.float32) * scales.astype(np.float32)[:, None]).astype(np.float32)
    got = C.cpu().numpy()
    bad = np.argwhere(got.view(np.int32) != expect.view(np.int32))
    bad = [tuple(b) for b in bad if not (got[tuple(b)] == 0 and expect[tuple(b)] == 0)]
    assert not bad, f"{len(bad)} codes differ, first at {bad[:4]} (row amax {[amaxes[b[0] // 3] for b in bad[:4]]})"


def test_fp8_quant_a_leaves_workspace_counters_zero(oracle_mod):
    """The row maxima go past the workspace's counter region, so a Workspace
    shared with gemm_run calls keeps its arrival counters at zero: a K-split
    small-M product right after a quantized-inside call on the same
    workspace is still correct."""
    w = g5.Workspace()
    X = torch.randn(300, 256, device="cuda").to(torch.bfloat16)
    qW, sW = g5.gemm_fp8_quantize_rows((torch.randn(512, 256, device="cuda") * 0.125).to(torch.bfloat16))
    g5.gemm_fp8_nt_quant_a(X, qW, sW, workspace=w)
    torch.cuda.synchronize()
    assert int(w.buf[:g5.GEMM_WORKSPACE_COUNTER_BYTES].count_nonzero()) == 0, "counters written"
    M, N, K = 1, 12288, 4096
    A, B = gi.small_case("bf16", M, N, K, seed=31, scale_b=0.125)
    st, plan = g5.plan_query(g5.GEMM_OP_BF16, M, N, K)
    assert st == 0 and plan.name == b"decode_splitk", plan.name
    C = g5.gemm_bf16(dev_bf16(A), dev_bf16(B), workspace=w)
    check_bf16(host_values(C), oracle_mod.gemm_bf16(A, B), K, "split small-M after quant-A")
