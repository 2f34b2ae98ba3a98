"""Pins for the oracle's FP8 (E4M3FN) quantization and scaled product (no GPU).

Page "Operator & Runtime" (section 5.4.3) quantizes to E4M3FN -- one sign,
four exponent and three mantissa bits, largest finite value 448 -- with a
scale from the whole row's maximum (Example 5-7), and compares quantizing
before the GEMM with quantizing inside it (Example 5-8).  Each pin checks
the oracle against something other than its own code: the page's printed
values, the format's fixed points, exact small-integer products and
brute-force rational arithmetic.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import gemm_inputs as gi

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        return [l.split() for l in fh if l.strip() and not l.startswith("#")]


def test_page_example_row_scale(oracle_mod):
    """Example 5-7: whole-row max 10 turns the first element into code 44
    (dequantized 55/56); the first block alone (max 1) keeps it exact."""
    (n, blk, v1, v2, fmax), (scaled, rounded, num, den), (scaled1, deq1, dn, dd, pct) = _golden_rows(
        "op_runtime_5_4_3_e4m3_row_scale.txt")
    n, blk, v1, v2 = int(n), int(blk), float(v1), float(v2)
    x = np.zeros((1, n), np.float32)
    x[0, 0], x[0, blk] = v1, v2
    Q, s = oracle_mod.quantize_rows_e4m3(gi.to_bf16_bits(x))
    assert oracle_mod.e4m3_decode([Q[0, 0]])[0] == float(rounded)
    assert oracle_mod.e4m3_decode([Q[0, blk]])[0] == float(fmax)
    assert np.all(Q[0, 1:blk] == 0) and np.all(Q[0, blk + 1:] == 0)
    deq = float(oracle_mod.e4m3_decode([Q[0, 0]])[0]) * float(s[0])
    assert abs(deq - int(num) / int(den)) < 1e-6                  # 55/56, up to the binary32 factor
    assert abs(float(s[0]) - v2 / float(fmax)) <= 2.0 ** -24 * v2 / float(fmax)   # binary32 rounding
    # the first block alone: scaled value exactly 448, dequantized exactly 1
    Q1, s1 = oracle_mod.quantize_rows_e4m3(gi.to_bf16_bits(x[:, :blk]))
    assert oracle_mod.e4m3_decode([Q1[0, 0]])[0] == float(scaled1)
    # exact in rationals: 448 * (1 / 448); the stored factor is 1/448 in binary32
    assert abs(oracle_mod.e4m3_decode([Q1[0, 0]])[0] * float(s1[0]) - float(deq1)) <= 2.0 ** -24
    assert Fraction(int(oracle_mod.e4m3_decode([Q1[0, 0]])[0])) * Fraction(1, 448) == Fraction(deq1)
    diff = float(deq1) - int(num) / int(den)
    assert Fraction(diff).limit_denominator(1000) == Fraction(int(dn), int(dd))
    assert round(100 * diff, 1) == float(pct)
    assert abs(float(scaled) - v1 * float(fmax) / v2) < 1e-12


def test_e4m3fn_fixed_points(oracle_mod):
    """Values the format's definition fixes: 1 = 0 0111 000, the largest
    finite 448 = 1.75 * 2^8, NaN at exponent 15 mantissa 7, the smallest
    subnormal 2^-9 and normal 2^-6, the sign bit."""
    d = lambda c: float(oracle_mod.e4m3_decode([c])[0])
    assert d(0b0_0111_000) == 1.0
    assert d(0b0_1111_110) == 448.0 and d(0b1_1111_110) == -448.0
    assert math.isnan(d(0x7F)) and math.isnan(d(0xFF))
    assert d(0b0_1111_101) == 416.0                                # 1.625 * 256
    assert d(0x01) == 2.0 ** -9 and d(0x07) == 7 * 2.0 ** -9 and d(0x08) == 2.0 ** -6
    assert d(0x00) == 0.0 and d(0x80) == 0.0 and math.copysign(1, d(0x80)) < 0
    vals = oracle_mod.e4m3_decode(np.arange(256, dtype=np.uint8))
    fin = vals[np.isfinite(vals)]
    assert len(fin) == 254 and fin.max() == 448.0 and fin.min() == -448.0
    # 127 distinct non-negative values, strictly increasing with the code
    pos = vals[:0x7F]
    assert np.all(np.diff(pos) > 0)


def test_e4m3fn_encode_round_trip_and_ties(oracle_mod):
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = oracle_mod.e4m3_decode(codes)
    assert np.array_equal(oracle_mod.e4m3_encode(vals), codes)
    # midpoints between neighbours go to the neighbour with the even mantissa
    pos = oracle_mod.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2
    got = oracle_mod.e4m3_encode(mids)
    lo = np.arange(0x7E, dtype=np.uint8)
    want = np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint8)
    assert np.array_equal(got, want)
    # hand-picked: 44.8 -> 44, 46 (tie 44/48) -> 48, 2^-10 (tie 0 / 2^-9) -> 0,
    # 3 * 2^-10 (tie 2^-9 / 2^-8) -> 2^-8, above 448 saturates, NaN -> 0x7f
    enc = lambda x: int(oracle_mod.e4m3_encode([x])[0])
    assert oracle_mod.e4m3_decode([enc(44.8)])[0] == 44.0
    assert oracle_mod.e4m3_decode([enc(46.0)])[0] == 48.0
    assert enc(2.0 ** -10) == 0x00 and enc(3 * 2.0 ** -10) == 0x02
    assert enc(460.0) == 0x7E and enc(1e6) == 0x7E and enc(-1e6) == 0xFE
    assert enc(float("nan")) == 0x7F
    # nearest: on a fine grid, no finite code is closer than the chosen one
    xs = np.linspace(-450, 450, 20001)
    ch = oracle_mod.e4m3_decode(oracle_mod.e4m3_encode(xs))
    allv = np.sort(oracle_mod.e4m3_decode(np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)))
    best = np.min(np.abs(xs[:, None] - allv[None, :]), axis=1)
    inrange = np.abs(xs) <= 448
    assert np.all(np.abs(xs - ch)[inrange] <= best[inrange] + 1e-12)


def test_quantize_rows_properties(oracle_mod):
    g = np.random.default_rng(7)
    X = gi.to_bf16_bits(gi.normal(g, (6, 300)))
    X[3] = 0                                                       # a zero row
    Q, s = oracle_mod.quantize_rows_e4m3(X)
    xf = gi.bf16_bits_to_f32(X).astype(np.float64)
    for r in range(6):
        amax = np.abs(xf[r]).max()
        if amax == 0:
            assert np.all(Q[r] == 0) and s[r] == 0
            continue
        assert s[r] == np.float32(np.float32(amax) / np.float32(448))
        k = np.argmax(np.abs(xf[r]))
        assert oracle_mod.e4m3_decode([Q[r, k]])[0] == math.copysign(448.0, xf[r, k])
        # every dequantized value is within half a step of its exact value
        deq = oracle_mod.e4m3_decode(Q[r]) * float(s[r])
        rel = np.abs(deq - xf[r]) / np.maximum(np.abs(xf[r]), amax * 2.0 ** -6)
        assert rel.max() <= 2.0 ** -4 * 1.0001


def test_fp8_product_brute_force(oracle_mod):
    """Tiny scaled products against exact rational arithmetic; scales and
    codes arbitrary (finite), including subnormals and negative values."""
    g = np.random.default_rng(11)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    for M, N, K in [(1, 1, 1), (3, 4, 5), (5, 2, 7)]:
        A = g.choice(finite, (M, K))
        Bt = g.choice(finite, (N, K))
        sa = (g.random(M) * 4).astype(np.float32)
        sb = (g.random(N) * 4).astype(np.float32)
        C = oracle_mod.gemm_fp8_nt(A, sa, Bt, sb)
        dec = lambda c: Fraction(float(oracle_mod.e4m3_decode([c])[0]))
        for i in range(M):
            for j in range(N):
                exact = sum(dec(A[i, k]) * dec(Bt[j, k]) for k in range(K)) * Fraction(float(sa[i])) * Fraction(float(sb[j]))
                assert abs(Fraction(C[i, j]) - exact) <= abs(exact) * Fraction(1, 2 ** 52)
        C1 = oracle_mod.gemm_fp8_nt(A, None, Bt, None)              # no scales: factors of 1
        assert C1[0, 0] == float(sum(dec(A[0, k]) * dec(Bt[0, k]) for k in range(K)))


def test_fp8_product_small_integers(oracle_mod):
    """Codes of small integers (exact in E4M3FN) give integer products."""
    enc = lambda v: oracle_mod.e4m3_encode(np.asarray(v, np.float64))
    A = enc([[1, 2, -3], [4, 0, 5]])
    Bt = enc([[1, 1, 1], [2, -1, 0.5]])
    C = oracle_mod.gemm_fp8_nt(A, None, Bt, None)
    # [1, 2, -3].[2, -1, 0.5] = 2 - 2 - 1.5; [4, 0, 5].[2, -1, 0.5] = 8 + 2.5
    assert np.array_equal(C, np.array([[0.0, -1.5], [9.0, 10.5]]))
    C2 = oracle_mod.gemm_fp8_nt(A, np.array([2, 0.5], np.float32), Bt, np.array([1, 4], np.float32))
    assert np.array_equal(C2, np.array([[0.0, -12.0], [4.5, 21.0]]))


def _nearest_code_exact(x, amax, mags):
    """The E4M3FN code nearest to x * 448 / amax in rational arithmetic,
    ties to the even code, by brute force over the 127 magnitudes."""
    if amax == 0:
        return 0x80 if math.copysign(1.0, x) < 0 else 0x00
    q = abs(Fraction(x)) * 448 / Fraction(amax)
    best = min(range(len(mags)), key=lambda c: (abs(q - mags[c]), c % 2))
    return (0x80 if x < 0 or math.copysign(1.0, x) < 0 else 0x00) | best


# (x, amax) pairs, bf16 values, whose quotient x * 448 / amax is exactly the
# midpoint of two E4M3FN neighbours (200 = (192 + 208) / 2, 84 = (80 + 88) / 2,
# 336 = (320 + 352) / 2, 1.5625 = (1.5 + 1.625) / 2, 0.65625 = (0.625 + 0.6875) / 2).
_TIES = [(0.00133514404296875, 0.00299072265625), (0.001190185546875, 0.00634765625),
         (0.0047607421875, 0.00634765625), (0.00133514404296875, 0.3828125),
         (0.001190185546875, 0.8125), (0.00122833251953125, 0.00299072265625)]


def test_quantize_rows_exact_against_rationals(oracle_mod):
    """Operator & Runtime §5.4.3, Example 5-7: each code is the E4M3FN value
    nearest to the exact quotient x * 448 / amax.  Checked element by element
    against rational arithmetic and a brute-force nearest-value search, on
    rows of several magnitudes (codes across the subnormal range too) and on
    rows built so that quotients fall exactly on midpoints."""
    mags = [Fraction(float(v)) for v in oracle_mod.e4m3_decode(np.arange(127, dtype=np.uint8))]
    g = np.random.default_rng(5)
    rows = [gi.normal(g, (1, 160)) * s for s in (1.0, 1e-3, 300.0)]
    rows.append((g.random((1, 160)) * 2 - 1).astype(np.float32))
    X = gi.to_bf16_bits(np.concatenate(rows, 0))
    ties = np.zeros((len(_TIES), 3), np.float32)
    for i, (x, amax) in enumerate(_TIES):
        ties[i] = [x, -amax, -x]                    # amax as a negative entry, the tie on both signs
    Q, s = oracle_mod.quantize_rows_e4m3(X)
    xf = gi.bf16_bits_to_f32(X).astype(np.float64)
    for r in range(X.shape[0]):
        amax = float(np.abs(xf[r]).max())
        for k in range(X.shape[1]):
            assert int(Q[r, k]) == _nearest_code_exact(float(xf[r, k]), amax, mags), (r, k)
    Qt, st = oracle_mod.quantize_rows_e4m3(gi.to_bf16_bits(ties))
    tf = gi.bf16_bits_to_f32(gi.to_bf16_bits(ties)).astype(np.float64)
    assert np.array_equal(tf, ties.astype(np.float64))            # the inputs are bf16 values
    for r in range(len(_TIES)):
        for k in range(3):
            assert int(Qt[r, k]) == _nearest_code_exact(float(tf[r, k]), float(np.abs(tf[r]).max()), mags)


def test_quantize_rows_exact_ties(oracle_mod):
    """Quotients exactly on a midpoint go to the even code.  The two-rounding
    binary32 form fl(x * fl(448 / amax)) moves some of them off the midpoint
    and to the odd neighbour; the exact rule does not."""
    flips = 0
    for x, amax in _TIES:
        q = Fraction(x) * 448 / Fraction(amax)
        row = gi.to_bf16_bits(np.array([[x, amax]], np.float32))
        Q, s = oracle_mod.quantize_rows_e4m3(row)
        v = Fraction(float(oracle_mod.e4m3_decode([Q[0, 0]])[0]))
        lo = max(Fraction(float(d)) for d in oracle_mod.e4m3_decode(np.arange(127, dtype=np.uint8))
                 if Fraction(float(d)) <= q)
        hi = min(Fraction(float(d)) for d in oracle_mod.e4m3_decode(np.arange(127, dtype=np.uint8))
                 if Fraction(float(d)) >= q)
        assert (lo + hi) / 2 == q and lo != hi                  # an exact tie
        assert int(Q[0, 0]) % 2 == 0 and v in (lo, hi)          # the even neighbour
        # the binary32 two-rounding form, emulated
        y32 = float(np.float32(x) * (np.float32(448.0) / np.float32(amax)))
        alt = lo if abs(Fraction(y32) - lo) < abs(Fraction(y32) - hi) else hi
        flips += alt != v
    assert flips >= 1                                            # the pin separates the two rules


def test_quantize_cols_exact_against_rationals(oracle_mod):
    """Per-column quantization of a weight [K, N]: every code of column j is
    the E4M3FN value nearest to W[k][j] * 448 / amax_j (rational arithmetic,
    brute force), written at [j][k], with factor amax_j / 448; a zero
    column, a column whose maximum is negative, columns of very different
    magnitudes and an exact tie."""
    mags = [Fraction(float(v)) for v in oracle_mod.e4m3_decode(np.arange(127, dtype=np.uint8))]
    g = np.random.default_rng(6)
    K, N = 24, 7
    w = gi.normal(g, (K, N)) * np.float32(2.0) ** np.arange(-6, 8, 2, dtype=np.float32)[None, :]
    w[:, 0] = 0
    w[5, 1] = -np.float32(40.0)
    x, amax = _TIES[0]
    w[:, 2] = 0
    w[0, 2], w[1, 2], w[2, 2] = x, -amax, amax * 0.25
    W = gi.to_bf16_bits(w)
    Qt, s = oracle_mod.quantize_cols_e4m3(W)
    assert Qt.shape == (N, K) and s.shape == (N,)
    wf = gi.bf16_bits_to_f32(W).astype(np.float64)
    for j in range(N):
        am = float(np.abs(wf[:, j]).max())
        assert s[j] == np.float32(am / 448.0)
        for k in range(K):
            assert int(Qt[j, k]) == _nearest_code_exact(float(wf[k, j]), am, mags), (j, k)
    assert np.all(Qt[0] == 0) and s[0] == 0
    assert Qt[1, 5] == 0xFE                                     # -448: the column's maximum, negative
    assert Qt[2, 0] == oracle_mod.e4m3_encode(np.array([200.0]))[0] and Qt[2, 0] % 2 == 0   # the tie, even code


def test_fp8_affine_reductions(oracle_mod):
    """The FP8 affine oracle against its parts: alpha = 1, no bias, beta = 0
    is the scaled product; alpha = 0 is bias + beta * C_old alone; in
    general it is alpha * D + bias + beta * C_old with D in rationals on a
    tiny case (brute force over the decoded codes)."""
    g = np.random.default_rng(8)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    M, N, K = 3, 5, 7
    A, Bt = g.choice(finite, (M, K)), g.choice(finite, (N, K))
    sa = (2.0 ** g.integers(-4, 4, M)).astype(np.float32)
    sb = (2.0 ** g.integers(-4, 4, N)).astype(np.float32)
    bias = gi.to_bf16_bits(gi.normal(g, (N,)))
    old = gi.to_bf16_bits(gi.normal(g, (M, N)))
    D = oracle_mod.gemm_fp8_nt(A, sa, Bt, sb)
    assert np.array_equal(oracle_mod.gemm_fp8_nt_affine(A, sa, Bt, sb), D)
    bv = gi.bf16_bits_to_f32(bias).astype(np.float64)
    ov = gi.bf16_bits_to_f32(old).astype(np.float64)
    C0 = oracle_mod.gemm_fp8_nt_affine(A, sa, Bt, sb, alpha=0.0, bias=bias, beta=-2.0, C_old=old)
    assert np.array_equal(C0, bv[None, :] - 2.0 * ov)
    alpha, beta = 0.75, 0.5
    C = oracle_mod.gemm_fp8_nt_affine(A, sa, Bt, sb, alpha=alpha, bias=bias, beta=beta, C_old=old)
    da = [[Fraction(float(v)) for v in row] for row in oracle_mod.e4m3_decode(A)]
    db = [[Fraction(float(v)) for v in row] for row in oracle_mod.e4m3_decode(Bt)]
    for i in range(M):
        for j in range(N):
            d = sum(da[i][k] * db[j][k] for k in range(K)) * Fraction(float(sa[i])) * Fraction(float(sb[j]))
            exact = Fraction(alpha) * d + Fraction(float(bv[j])) + Fraction(beta) * Fraction(float(ov[i, j]))
            assert abs(Fraction(float(C[i, j])) - exact) <= abs(exact) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 60)
