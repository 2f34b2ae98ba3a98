"""GPU parity of the SwiGLU output stored as E4M3FN codes
(gemm_bf16_swiglu_e4m3 and its batched form) against the oracle, through the
C ABI.

Page "Operator & Runtime" §5.3.1 carries Example 5-4 on by quantizing
Z = SiLU(G) (.) U with one fixed scale factor, so that the fused program
reads the operands and writes one byte per output.  The oracle
(quantize_fixed_e4m3) maps the range amax to 448 and takes the nearest
E4M3FN value of the binary32 quotient.

Two kinds of check:
  * exact: X rows that pick single rows of the weight make every sum exact,
    and gates of at least 17 make SiLU(g) round to g, so each code is fixed
    by the arithmetic alone and must equal the oracle's bit for bit --
    codes on E4M3FN values and on midpoints (ties to even), saturation,
    signed zero, several ranges, on the ring kernel, the split small-M path
    and the whole-K small-M kernel;
  * random operands: every code lies in the range the kernel's FP32 sums
    allow (_gpu_helpers.swiglu_code_range) and equals the oracle's where
    that range holds one code.
"""
import numpy as np
import pytest
import torch

import gemm_inputs as gi
from _gpu_helpers import check_swiglu_codes, dev_bf16, swiglu_code_range, swiglu_sums, ws

import dense_gemm_05_amd as g5

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[swiglu-e4m3] {msg}", flush=True)


@pytest.fixture(autouse=True)
def _no_overrides(monkeypatch):
    for v in ("GEMM_FORCE_CONFIG", "GEMM_DECODE_PAIR", "GEMM_FORCE_KSPLIT"):
        monkeypatch.delenv(v, raising=False)


def _host_u8(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _plan_name(M, N, K, with_ws, ldc=None):
    st, p = g5.plan_query(g5.GEMM_OP_BF16_SWIGLU, M, N, K, ldc=ldc, c_type=g5.GEMM_OUT_E4M3,
                          with_workspace=with_ws)
    assert st == 0
    return p.name.decode()


def _exact_case(oracle_mod, M, K, N, seed):
    """X [M, K] with X[i, i % K] = 1 (one weight row per output row); the
    first 128 output columns have gate 32 (one 0) and up values v / 32 for v on every
    E4M3FN value and midpoint, both signs, past 448 and zero (so z = v); the
    rest random gates in [17, 2048) and up values of random sign in
    [2^-14, 4)."""
    g = np.random.default_rng([gi.SEED_BASE + 3100 + seed, M, N, K])
    X = np.zeros((M, K), np.float32)
    X[np.arange(M), np.arange(M) % K] = 1.0
    vals = oracle_mod.e4m3_decode(np.arange(127, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2
    v = np.concatenate([vals, mids, [500.0, 1000.0, 32768.0, 0.0]])
    v = np.concatenate([v, -v])
    crafted = g.permutation(np.resize(v, K * 128)).reshape(K, 128) / 32.0
    # row 0 (read by every call) starts with the special cases: saturation
    # on both signs, +0, -0 (a zero gate, SiLU(0) = 0 on both sides, times
    # a negative up value: a sum over K itself gives +0, never -0), and two
    # ties (1.0625 -> 1, 1.1875 -> 1.25)
    crafted[0, :6] = np.array([500.0, -1000.0, 0.0, -5.0, 1.0625, 1.1875]) / 32.0
    Wg = np.empty((K, N), np.float32)
    Wu = np.empty((K, N), np.float32)
    Wg[:, :128] = 32.0
    Wg[0, 3] = 0.0
    Wu[:, :128] = crafted
    Wg[:, 128:] = 2.0 ** g.uniform(np.log2(17.0), 11.0, (K, N - 128))
    Wu[:, 128:] = np.where(g.random((K, N - 128)) < 0.5, -1.0, 1.0) * 2.0 ** g.uniform(-14.0, 2.0, (K, N - 128))
    Wgu = gi.to_bf16_bits(np.concatenate([Wg, Wu], axis=1))
    Xb = gi.to_bf16_bits(X)
    # the bf16 weights are the values used: gates stay >= 17 (but the zero
    # one), crafted ups exact
    wv = gi.bf16_bits_to_f32(Wgu)
    gates = wv[:, :N].copy()
    gates[0, 3] = 17.0
    assert gates.min() >= 17.0 and np.array_equal(wv[:, N:N + 128], crafted.astype(np.float32))
    return Xb, np.ascontiguousarray(Wgu)


PATHS = [("ring", 300, True), ("split", 1, True), ("split16", 16, True), ("whole_k", 16, False)]
RANGES = [448.0, 3.0, 1000.3, 0.0123]


@pytest.mark.parametrize("amax", RANGES)
@pytest.mark.parametrize("path,M,with_ws", PATHS)
def test_swiglu_e4m3_codes_exact(oracle_mod, path, M, with_ws, amax):
    K, N = 64, 256
    name = _plan_name(M, N, K, with_ws)
    _say(f"exact {path} {M}x{N}x{K} amax={amax} -> {name}")
    want_family = {"ring": "bf16_", "split": "decode_splitk", "split16": "decode_splitk", "whole_k": "decode_64"}
    assert name.startswith(want_family[path]), name
    X, Wgu = _exact_case(oracle_mod, M, K, N, 1)
    Zq = torch.full((M, N), 0xAA, dtype=torch.uint8, device="cuda")
    g5.gemm_bf16_swiglu_e4m3(dev_bf16(X), dev_bf16(Wgu), amax, Zq, workspace=ws() if with_ws else None)
    got = _host_u8(Zq)
    want = oracle_mod.swiglu_e4m3(X, Wgu, np.float32(amax))
    diff = np.argwhere(got != want)
    assert diff.size == 0, (f"{path} amax={amax}: {len(diff)} codes differ, first at {tuple(diff[0])}: "
                            f"got {got[tuple(diff[0])]:#04x} want {want[tuple(diff[0])]:#04x}")
    if amax == 448.0:
        # z on the special cases of row 0 (output row 0 reads weight row 0)
        assert list(want[0, :6]) == [0x7e, 0xfe, 0x00, 0x80, 0x38, 0x3a]


SHAPES = [(300, 392, 262, True), (256, 192, 256, True), (17, 200, 64, True), (1, 128, 4100, True),
          (16, 1024, 2048, True), (16, 1024, 2048, False), (1, 12288, 4096, True)]


@pytest.mark.parametrize("M,N,K,with_ws", SHAPES)
def test_swiglu_e4m3_random(oracle_mod, M, N, K, with_ws):
    """Random operands of the bf16 SwiGLU tests, ragged tiles and K tails, a
    range that saturates the largest outputs; rows of N bytes padded to a
    multiple of 16 (ldz > N where N % 16 != 0), the padding untouched."""
    ldz = (N + 15) // 16 * 16
    name = _plan_name(M, N, K, with_ws, ldc=ldz + 16 if M > 1 else N)
    _say(f"random {M}x{N}x{K} ws={with_ws} -> {name}")
    g = np.random.default_rng([gi.SEED_BASE + 3200, M, N, K])
    X = gi.to_bf16_bits(gi.normal(g, (M, K)))
    Wgu = gi.to_bf16_bits(gi.normal(g, (K, 2 * N), 0.125))
    if M * N * K > 2 ** 27:                      # the oracle on sampled rows
        rows = np.unique(np.linspace(0, M - 1, 4).astype(int))
    else:
        rows = np.arange(M)
    Xs = np.ascontiguousarray(X[rows])
    Zr, *_ = oracle_mod.swiglu_bf16(Xs, Wgu)
    # a general binary32 range (the division) and a bf16 one (the fast quotient)
    a32 = np.float32(0.6 * np.abs(Zr).max())
    a16 = np.float32(oracle_mod.round_bf16_value([0.45 * float(a32)])[0])
    dX, dW = dev_bf16(X), dev_bf16(Wgu)
    for amax in (a32, a16):
        full = torch.full((M, ldz + 16), 0xAA, dtype=torch.uint8, device="cuda")
        Zq = full[:, :N]
        g5.gemm_bf16_swiglu_e4m3(dX, dW, float(amax), Zq, workspace=ws() if with_ws else None)
        host = _host_u8(full)
        assert np.all(host[:, N:] == 0xAA), "row padding was written"
        c_lo, c_hi = swiglu_code_range(oracle_mod, Xs, Wgu, amax)
        frac = check_swiglu_codes(oracle_mod, host[rows, :N], c_lo, c_hi, f"{M}x{N}x{K} {name} amax={amax}",
                                  min_unique=0.15)
        _say(f"  amax {amax}: decided {frac:.3f}")
        # the oracle itself lies in the range
        want = oracle_mod.swiglu_e4m3(Xs, Wgu, amax)
        d = oracle_mod.e4m3_decode
        assert np.all((d(c_lo) <= d(want)) & (d(want) <= d(c_hi)))


def test_swiglu_e4m3_ffn_full_size(oracle_mod):
    """The FFN's gate and up projections, X [1024, 4096] and the merged
    weight [4096, 2 x 12288], with the output stored as codes: the
    benchmarked launch; every element, for a general and a bf16 range."""
    _say("ffn 1024x12288x4096 (every element)")
    X, Wgu = gi.swiglu_inputs()
    assert _plan_name(1024, 12288, 4096, True) == "bf16_256x192"
    Zr, *_ = oracle_mod.swiglu_bf16(np.ascontiguousarray(X[:64]), Wgu)
    dX, dW = dev_bf16(X), dev_bf16(Wgu)
    a32 = np.float32(0.5 * np.abs(Zr).max())
    a16 = np.float32(oracle_mod.round_bf16_value([float(a32)])[0])
    got = {}
    for amax in (a32, a16):
        got[float(amax)] = _host_u8(g5.gemm_bf16_swiglu_e4m3(dX, dW, float(amax), workspace=ws()))
    sums = swiglu_sums(oracle_mod, X, Wgu)
    for amax in (a32, a16):
        c_lo, c_hi = swiglu_code_range(oracle_mod, X, Wgu, amax, sums)
        frac = check_swiglu_codes(oracle_mod, got[float(amax)], c_lo, c_hi, f"ffn amax={amax}", min_unique=0.15)
        _say(f"  amax {amax}: decided {frac:.3f}")


@pytest.mark.parametrize("broadcast_x", [False, True])
def test_swiglu_e4m3_batched(oracle_mod, broadcast_x):
    """Batched codes (experts, each with its own weight; tokens shared when
    X's batch stride is 0), one range for every entry; entry strides with a
    gap between entries, untouched."""
    batch, M, N, K = 3, 150, 208, 264
    _say(f"batched {batch}x{M}x{N}x{K} broadcast_x={broadcast_x}")
    g = np.random.default_rng([gi.SEED_BASE + 3300, int(broadcast_x)])
    X = gi.to_bf16_bits(gi.normal(g, (1 if broadcast_x else batch, M, K)))
    Wgu = gi.to_bf16_bits(gi.normal(g, (batch, K, 2 * N), 0.125))
    amax = np.float32(4.0)                        # (a bf16 value: the fast quotient)
    dX = dev_bf16(X)
    if broadcast_x:
        dX = dX.expand(batch, -1, -1)
    full = torch.full((batch, M + 1, N), 0xAA, dtype=torch.uint8, device="cuda")
    g5.gemm_bf16_swiglu_e4m3_batched(dX, dev_bf16(Wgu), float(amax), full[:, :M], workspace=ws())
    host = _host_u8(full)
    assert np.all(host[:, M] == 0xAA)
    for b in range(batch):
        Xb = np.ascontiguousarray(X[0 if broadcast_x else b])
        c_lo, c_hi = swiglu_code_range(oracle_mod, Xb, np.ascontiguousarray(Wgu[b]), amax)
        check_swiglu_codes(oracle_mod, host[b, :M], c_lo, c_hi, f"expert {b}", min_unique=0.5)


def test_swiglu_e4m3_k_zero_and_empty():
    """K = 0: every sum is 0, SiLU(0) * 0 = +0, code 0x00 everywhere; M = 0
    writes nothing."""
    X = torch.empty((40, 0), dtype=torch.bfloat16, device="cuda")
    W = torch.empty((0, 2 * 64), dtype=torch.bfloat16, device="cuda")
    Zq = torch.full((40, 64), 0xAA, dtype=torch.uint8, device="cuda")
    g5.gemm_bf16_swiglu_e4m3(X, W, 1.0, Zq, workspace=ws())
    assert np.all(_host_u8(Zq) == 0)
    Zq = torch.full((40, 64), 0xAA, dtype=torch.uint8, device="cuda")
    g5.gemm_bf16_swiglu_e4m3(X[:0], W, 1.0, Zq[:0])
    assert np.all(_host_u8(Zq) == 0xAA)


@pytest.mark.parametrize("M,with_ws", [(300, True), (1, True), (16, False)])
def test_swiglu_e4m3_is_the_quantized_bf16_output(M, with_ws):
    """Fusing the quantization keeps the unfused program's rounding: the
    codes equal, bit for bit, the separate quantization step
    (act_quantize_e4m3) applied to the bf16 SwiGLU output of the same call
    shape, on the ring kernel and the small-M paths, for a bf16 range (the
    fast quotient) and a general one (the division)."""
    N, K = 384, 640
    _say(f"fused vs separate quantization {M}x{N}x{K} ws={with_ws}")
    g = np.random.default_rng([gi.SEED_BASE + 3400, M])
    X = gi.to_bf16_bits(gi.normal(g, (M, K)))
    Wgu = gi.to_bf16_bits(gi.normal(g, (K, 2 * N), 0.125))
    dX, dW = dev_bf16(X), dev_bf16(Wgu)
    w = ws() if with_ws else None
    Zb = g5.gemm_bf16_swiglu(dX, dW, workspace=w)
    for amax in (3.0, 2.9):
        q_fused = _host_u8(g5.gemm_bf16_swiglu_e4m3(dX, dW, amax, workspace=w))
        q_sep = _host_u8(g5.act_quantize_e4m3(Zb, amax))
        assert np.array_equal(q_fused, q_sep), f"amax={amax}: {int((q_fused != q_sep).sum())} codes differ"
