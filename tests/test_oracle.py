"""Pins for the CPU oracle (no GPU).

The oracle is the plain definition C[i][j] = sum_k A[i][k] B[k][j] accumulated
in FP64.  Each pin below checks it against something other than itself: exact
closed forms (identity, all-ones, rank-1), exact rational arithmetic on tiny
inputs, the non-associativity example of page "Operator & Runtime" section
5.2.4, an independent library product, and the bit-level definition of
round-to-nearest-even bf16.  The mutant test at the end shows that plausible
mistakes (a dropped term, a transposed operand, swapped operands, a wrong sign)
each fail at least one pin.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import gemm_inputs as gi

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32(x):
    return np.asarray(x, np.float32)


def bits(x):
    return gi.to_bf16_bits(np.asarray(x, np.float32))


# ---------------------------------------------------------------- pin helpers
# Each takes a gemm(A, B) callable on float32 arrays and returns None on
# success or a string naming the failure.  The same helpers run against the
# real oracle and against planted mistakes.

def pin_identity(gemm):
    g = np.random.default_rng(1)
    B = f32(g.integers(-9, 10, (6, 5)))
    A = f32(g.integers(-9, 10, (4, 6)))
    if not np.array_equal(gemm(np.eye(6, dtype=np.float32), B), B.astype(np.float64)):
        return "I.B != B"
    if not np.array_equal(gemm(A, np.eye(6, dtype=np.float32)), A.astype(np.float64)):
        return "A.I != A"
    return None


def pin_all_ones(gemm):
    for (M, N, K) in [(3, 4, 5), (2, 7, 100), (1, 1, 4100)]:
        C = gemm(np.ones((M, K), np.float32), np.ones((K, N), np.float32))
        if not np.all(C == K):
            return f"all-ones {M}x{N}x{K} != K"
    return None


def pin_rank1(gemm):
    u = np.array([1, -2, 3, 0, 5], np.float32)
    v = np.array([2, -1, 4, 7], np.float32)
    for K in (1, 3, 8):
        A = np.repeat(u[:, None], K, axis=1)
        B = np.repeat(v[None, :], K, axis=0)
        want = K * np.outer(u.astype(np.float64), v.astype(np.float64))
        if not np.array_equal(gemm(A, B), want):
            return f"rank-1 K={K}"
    return None


def pin_bruteforce(gemm):
    g = np.random.default_rng(7)
    for (M, N, K) in [(3, 5, 7), (7, 2, 4), (1, 8, 3), (8, 1, 6), (5, 5, 5)]:
        A = f32(g.integers(-64, 65, (M, K)) / 16.0)
        B = f32(g.integers(-64, 65, (K, N)) / 8.0)
        C = gemm(A, B)
        for i in range(M):
            for j in range(N):
                want = sum((Fraction(float(A[i, k])) * Fraction(float(B[k, j])) for k in range(K)),
                           Fraction(0))
                if Fraction(float(C[i, j])) != want:
                    return f"brute force {M}x{N}x{K} at ({i},{j})"
    return None


def pin_fp64_accumulation(gemm):
    with open(os.path.join(GOLDEN, "op_runtime_5_2_4_fp_order.txt")) as fh:
        line = [l for l in fh if l.strip() and not l.startswith("#")][0]
    a_s, b_s, c_s = [p.split() for p in line.split(";")]
    a = f32([float.fromhex(x) if "0x" in x else float(x) for x in a_s])[None, :]
    b = f32([float.fromhex(x) if "0x" in x else float(x) for x in b_s])[:, None]
    want = float.fromhex(c_s[0])
    got = gemm(a, b)[0, 0]
    if got != want:
        return f"1+2^-24+2^-24 gave {got!r}"
    # the same sum in float32, left to right, loses both small terms
    s = np.float32(0)
    for x, y in zip(a[0], b[:, 0]):
        s = np.float32(s + x * y)
    if s != np.float32(1.0):
        return "float32 left-to-right reference is wrong"
    return None


def pin_library(gemm):
    g = np.random.default_rng(11)
    A = gi.uniform_pm1(g, (37, 53))
    B = gi.uniform_pm1(g, (53, 29))
    C = gemm(A, B)
    ref = A.astype(np.float64) @ B.astype(np.float64)
    if np.max(np.abs(C - ref)) > 1e-12:
        return "differs from numpy float64 matmul"
    return None


ALL_PINS = [pin_identity, pin_all_ones, pin_rank1, pin_bruteforce, pin_fp64_accumulation,
            pin_library]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_f32_pins(oracle_mod, pin):
    assert pin(oracle_mod.gemm_f32) is None


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_bf16_pins(oracle_mod, pin):
    # All pin inputs are exactly representable in bf16 except the library pin,
    # whose operands are rounded first; the bf16 oracle must then agree with
    # the float32 oracle run on the widened values.
    def gemm_via_bf16(A, B):
        Ab, Bb = bits(A), bits(B)
        if pin is not pin_library:
            assert np.array_equal(gi.bf16_bits_to_f32(Ab), A)
            assert np.array_equal(gi.bf16_bits_to_f32(Bb), B)
        return oracle_mod.gemm_bf16(Ab, Bb)
    if pin is pin_library:
        g = np.random.default_rng(11)
        A = gi.uniform_pm1(g, (37, 53))
        B = gi.uniform_pm1(g, (53, 29))
        Ab, Bb = bits(A), bits(B)
        ref = gi.bf16_bits_to_f32(Ab).astype(np.float64) @ gi.bf16_bits_to_f32(Bb).astype(np.float64)
        assert np.max(np.abs(oracle_mod.gemm_bf16(Ab, Bb) - ref)) <= 1e-12
    else:
        assert pin(gemm_via_bf16) is None


def test_oracle_mutants_fail_pins(oracle_mod):
    """Planted mistakes around the oracle each fail at least one pin."""
    g = oracle_mod.gemm_f32

    def drop_last_term(A, B):
        K = A.shape[1]
        if K == 1:
            return np.zeros((A.shape[0], B.shape[1]))
        return g(np.ascontiguousarray(A[:, :K - 1]), np.ascontiguousarray(B[:K - 1]))

    def transposed_b(A, B):
        # only square B admits this slip; the 5x5x5 brute-force case has one
        if B.shape[0] == B.shape[1]:
            return g(A, np.ascontiguousarray(B.T))
        return g(A, B)

    def swapped(A, B):
        if A.shape[0] == A.shape[1] == B.shape[0] == B.shape[1]:
            return g(B, A)
        return g(A, B)

    def negated_last_term(A, B):
        K = A.shape[1]
        C = g(A, B)
        return C - 2.0 * np.outer(A[:, K - 1].astype(np.float64), B[K - 1].astype(np.float64))

    def float32_accumulate(A, B):
        M, K = A.shape
        N = B.shape[1]
        C = np.zeros((M, N), np.float32)
        for k in range(K):
            C = (C + np.outer(A[:, k], B[k]).astype(np.float32)).astype(np.float32)
        return C.astype(np.float64)

    def row_offset(A, B):
        C = g(A, B)
        if C.shape[0] > 1:
            C = np.roll(C, 1, axis=0)
        return C

    for mutant in (drop_last_term, transposed_b, swapped, negated_last_term,
                   float32_accumulate, row_offset):
        fails = [p.__name__ for p in ALL_PINS if p(mutant) is not None]
        assert fails, f"planted mistake {mutant.__name__} passed every pin"


def test_oracle_strided_operands_ignore_padding(oracle_mod):
    g = np.random.default_rng(3)
    Afull = gi.uniform_pm1(g, (9, 20))
    Bfull = gi.uniform_pm1(g, (13, 17))
    Afull[:, 13:] = np.nan     # padding beyond K
    Bfull[:, 11:] = np.nan     # padding beyond N
    A = Afull[:, :13]
    B = Bfull[:, :11]
    C = oracle_mod.gemm_f32(A, B)
    assert np.all(np.isfinite(C))
    ref = oracle_mod.gemm_f32(np.ascontiguousarray(A), np.ascontiguousarray(B))
    assert np.array_equal(C, ref)
    Ab, Bb = bits(Afull), bits(Bfull)
    Cb = oracle_mod.gemm_bf16(Ab[:, :13], Bb[:, :11])
    assert np.all(np.isfinite(Cb))


def test_oracle_empty_and_k0(oracle_mod):
    assert oracle_mod.gemm_f32(np.zeros((0, 4), np.float32), np.zeros((4, 3), np.float32)).shape == (0, 3)
    C = oracle_mod.gemm_f32(np.zeros((3, 0), np.float32), np.zeros((0, 2), np.float32))
    assert C.shape == (3, 2) and np.all(C == 0.0)   # empty sum
    Cb = oracle_mod.gemm_bf16(np.zeros((2, 0), np.uint16), np.zeros((0, 5), np.uint16))
    assert np.all(Cb == 0.0)


def test_oracle_batched_matches_single(oracle_mod):
    g = np.random.default_rng(5)
    A = bits(gi.normal(g, (3, 6, 10)))
    B = bits(gi.normal(g, (3, 10, 4)))
    C = oracle_mod.gemm_bf16_batched(A, B)
    for b in range(3):
        assert np.array_equal(C[b], oracle_mod.gemm_bf16(A[b], B[b]))
    # entries are really independent: different entries give different results
    assert not np.array_equal(C[0], C[1])


def test_oracle_dot_matches_gemm(oracle_mod):
    g = np.random.default_rng(9)
    A = bits(gi.normal(g, (5, 33)))
    B = bits(gi.normal(g, (33, 7)))
    C = oracle_mod.gemm_bf16(A, B)
    for (i, j) in [(0, 0), (4, 6), (2, 3)]:
        assert oracle_mod.dot_bf16(A, B, i, j) == C[i, j]
    Af, Bf = gi.uniform_pm1(g, (4, 9)), gi.uniform_pm1(g, (9, 3))
    Cf = oracle_mod.gemm_f32(Af, Bf)
    assert oracle_mod.dot_f32(Af, Bf, 3, 2) == Cf[3, 2]


# ------------------------------------------------------------ bf16 rounding

def _f(u32):
    return np.array([u32], np.uint32).view(np.float32)[0]


ROUND_CASES = [
    # (float32 value, expected bf16 bits, why)
    (1.0 + 2.0 ** -8, 0x3F80, "tie, kept part even: stays 1.0"),
    (1.0 + 3 * 2.0 ** -8, 0x3F82, "tie, kept part odd: rounds up to 1+2^-6"),
    (-(1.0 + 2.0 ** -8), 0xBF80, "negative tie to even"),
    (1.0 + 2.0 ** -8 + 2.0 ** -20, 0x3F81, "just above half: up"),
    (1.0 + 2.0 ** -8 - 2.0 ** -20, 0x3F80, "just below half: down"),
    (4100.0, 0x4580, "all-ones K=4100 rounds to 4096"),
    (4096.0, 0x4580, "exact"),
    (1000.0, 0x447A, "exact"),
    (256.0, 0x4380, "exact"),
    (float(_f(0x7F7FFFFF)), 0x7F80, "largest float rounds to +inf"),
    (float(_f(0xFF7FFFFF)), 0xFF80, "most negative float rounds to -inf"),
    (float(_f(0x7F7F7FFF)), 0x7F7F, "below half: stays finite max bf16"),
    (float("inf"), 0x7F80, "+inf"),
    (float("-inf"), 0xFF80, "-inf"),
    (0.0, 0x0000, "+0"),
    (-0.0, 0x8000, "-0"),
    (float(_f(0x00008000)), 0x0000, "subnormal tie to even (0)"),
    (float(_f(0x00018000)), 0x0002, "subnormal tie to even (up)"),
]


@pytest.mark.parametrize("x,want,why", ROUND_CASES, ids=[c[2] for c in ROUND_CASES])
def test_oracle_round_bf16(oracle_mod, x, want, why):
    got = int(oracle_mod.round_bf16(np.array([x], np.float32))[0])
    assert got == want, f"{why}: got {got:#06x}"


def test_oracle_round_bf16_nan(oracle_mod):
    for pattern in (0x7FC00000, 0x7F800001, 0xFF800001, 0x7F810000):
        got = int(oracle_mod.round_bf16(np.array([pattern], np.uint32).view(np.float32))[0])
        assert (got & 0x7F80) == 0x7F80 and (got & 0x7F) != 0, hex(pattern)


def test_oracle_round_bf16_is_nearest(oracle_mod):
    """Exhaustive property over a grid of patterns: the result is one of the two
    neighbouring bf16 values and the nearer one (ties: even mantissa)."""
    g = np.random.default_rng(13)
    u = g.integers(0, 0x7F7F0000, 20000, dtype=np.uint32)
    u = np.concatenate([u, (u & 0xFFFF0000) | 0x8000])   # plus exact ties
    x = u.view(np.float32)
    r = oracle_mod.round_bf16(x).astype(np.uint32)
    lo = (u >> 16)
    hi = lo + 1
    flo = (lo << 16).view(np.float32).astype(np.float64)
    fhi = (hi << 16).view(np.float32).astype(np.float64)
    xd = x.astype(np.float64)
    dlo, dhi = xd - flo, fhi - xd
    expect = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    assert np.array_equal(r, expect)


def test_inputs_rounding_agrees_with_oracle_rounding(oracle_mod):
    """The input generator's float32->bf16 rounding (used to make operands) and
    the oracle's rounding are written independently; they must agree."""
    g = np.random.default_rng(17)
    x = np.concatenate([gi.normal(g, 100000), f32([c[0] for c in ROUND_CASES])])
    assert np.array_equal(gi.to_bf16_bits(x), oracle_mod.round_bf16(x))
