"""Pins for the oracle's fused-epilogue references (no GPU).

Page "Operator & Runtime" fuses an activation into the GEMM's output tile
(section 5.4.2, Y = SiLU(A.W)) and the SwiGLU product into the two
projections that share X (section 5.3.1, Z = SiLU(G) (.) U), and requires
the unfused program's rounding to survive: the FP32 product is rounded to
bf16 before the activation (section 5.4.3).  Each pin below checks the
oracle against something other than its own code: the value the page
prints, identities of SiLU, exact integer products, the bit-level bf16
rounding already pinned in test_oracle.py, and hand-worked bf16 values.
"""
import math
from fractions import Fraction
import os

import numpy as np
import pytest

import gemm_inputs as gi

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bits(x):
    return gi.to_bf16_bits(np.asarray(x, np.float32))


# ---------------------------------------------------------------- SiLU

def test_silu_page_example(oracle_mod):
    """The page's pair of partial sums 1 and -1 (section 5.4.3)."""
    with open(os.path.join(GOLDEN, "op_runtime_5_4_3_silu_partial_sums.txt")) as fh:
        rows = [l for l in fh if l.strip() and not l.startswith("#")]
    parts, full, page_value, decimals = [c.split() for c in rows[0].split(";")]
    parts = [float(x) for x in parts]
    assert oracle_mod.silu([sum(parts)])[0] == float(full[0])
    s = float(oracle_mod.silu(parts).sum())
    assert round(s, int(decimals[0])) == float(page_value[0])
    # closed form: SiLU(1) + SiLU(-1) = sigmoid(1) - sigmoid(-1) = tanh(1/2)
    assert abs(s - math.tanh(0.5)) < 1e-15


def test_silu_identities(oracle_mod):
    x = np.array([0.0, 0.25, 1.0, 3.5, 10.0, 37.0])
    s_pos, s_neg = oracle_mod.silu(x), oracle_mod.silu(-x)
    # SiLU(x) - SiLU(-x) = x sigmoid(x) + x sigmoid(-x) = x
    assert np.allclose(s_pos - s_neg, x, rtol=0, atol=1e-14)
    # SiLU(x) / x = sigmoid(x) = 1 / (1 + e^-x), which is 1/2 at 0 and tends to 1
    assert oracle_mod.silu([0.0])[0] == 0.0
    assert oracle_mod.silu([40.0])[0] == 40.0
    assert -1e-15 < oracle_mod.silu([-40.0])[0] < 0
    # the minimum of SiLU is about -0.2785 at x ~ -1.2785 (W(1/e) + 1)
    xs = np.linspace(-3, 0, 30001)
    m = oracle_mod.silu(xs)
    assert abs(m.min() + 0.27846454) < 1e-7 and abs(xs[m.argmin()] + 1.2784645) < 1e-3


# ---------------------------------------------------------------- bf16 of a double

ROUND_D_CASES = [
    (1 + 2 ** -8, 1.0, "tie rounds to the even neighbour (down)"),
    (1 + 3 * 2 ** -8, 1 + 2 ** -6, "tie rounds to the even neighbour (up)"),
    (1 + 2 ** -8 + 2 ** -40, 1 + 2 ** -7, "just above a tie rounds up (binary32 first would round twice)"),
    (257.0, 256.0, "257 is a tie between 256 and 258"),
    (-259.0, -260.0, "ties to even for negatives"),
    (1.5 * 2 ** -130, 1.5 * 2 ** -130, "subnormal, exact"),
    (2 ** -134, 0.0, "half the smallest subnormal rounds to zero (even)"),
    (3 * 2 ** -134, 2 ** -132, "tie between 2^-133 and 2^-132 rounds to the even one"),
    ((2 - 2 ** -8) * 2 ** 127, math.inf, "half an ulp above the largest finite value overflows"),
    ((2 - 2 ** -7) * 2 ** 127, (2 - 2 ** -7) * 2 ** 127, "largest finite value"),
]


@pytest.mark.parametrize("x,want,why", ROUND_D_CASES, ids=[c[2] for c in ROUND_D_CASES])
def test_round_bf16_value(oracle_mod, x, want, why):
    assert oracle_mod.round_bf16_value([x])[0] == want, why


def test_round_bf16_value_agrees_with_binary32_rounding(oracle_mod):
    """For values that are exact in binary32, rounding the double must give
    the bf16 that the (separately pinned) binary32 rounding gives."""
    g = np.random.default_rng(11)
    x = np.concatenate([g.standard_normal(20000) * 10.0 ** g.integers(-30, 30, 20000),
                        [0.0, -0.0, 1e-40, -3e38]]).astype(np.float32)
    want = (oracle_mod.round_bf16(x).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    got = oracle_mod.round_bf16_value(x.astype(np.float64))
    assert np.array_equal(got, want)


# ---------------------------------------------------------------- Y = SiLU(A.W)

def test_gemm_silu_exact_integers(oracle_mod):
    """Small-integer operands: A.W is an exact integer product (checked with
    numpy int64), bf16-representable here, so Y = SiLU(A.W) in double."""
    g = np.random.default_rng(5)
    A = g.integers(-3, 4, (7, 9)); W = g.integers(-3, 4, (9, 6))
    C = A @ W                                     # int64, |C| <= 81
    Y = oracle_mod.gemm_bf16_silu(bits(A), bits(W))
    Cf = C.astype(np.float64)
    assert np.allclose(Y, Cf / (1.0 + np.exp(-Cf)), rtol=1e-15, atol=0)


def test_gemm_silu_rounds_before_the_activation(oracle_mod):
    """A.W = 257 is not a bf16 value; the product is rounded (to 256) before
    SiLU, as section 5.4.3 requires, so Y = SiLU(256) = 256, not 257."""
    A = bits(np.ones((1, 257))); W = bits(np.ones((257, 1)))
    assert oracle_mod.gemm_bf16_silu(A, W)[0, 0] == 256.0


# ---------------------------------------------------------------- SwiGLU

def _merged(Wg, Wu):
    return np.ascontiguousarray(np.concatenate([Wg, Wu], axis=1))


def test_swiglu_gate_and_up_halves(oracle_mod):
    """X = [1, 1], gate column sums to 64 and up column to 2: SiLU(64) is 64
    in bf16, so Z = 128.  Swapping gate and up would give
    bf16(SiLU(2)) * 64 = 1.7578125 * 64 = 112.5."""
    X = bits([[1.0, 1.0]])
    Wg = bits([[32.0], [32.0]]); Wu = bits([[1.0], [1.0]])
    Z, g, u, t = oracle_mod.swiglu_bf16(X, _merged(Wg, Wu))
    assert (g[0, 0], u[0, 0], t[0, 0], Z[0, 0]) == (64.0, 2.0, 64.0, 128.0)
    Zs, *_ = oracle_mod.swiglu_bf16(X, _merged(Wu, Wg))
    assert Zs[0, 0] == 112.5


def test_swiglu_rounds_the_activation(oracle_mod):
    """g = 1, u = 3: SiLU(1) = 0.7310585... rounds to the bf16 value
    0.73046875 (187 * 2^-8) before the product, so Z = 2.19140625 exactly
    (without that rounding it would be 2.1931757...)."""
    X = bits([[1.0]])
    Z, g, u, t = oracle_mod.swiglu_bf16(X, _merged(bits([[1.0]]), bits([[3.0]])))
    assert t[0, 0] == 187 * 2.0 ** -8 and Z[0, 0] == 2.19140625


def test_swiglu_zero_gate_and_strided_weights(oracle_mod):
    """A zero gate gives Z = 0 whatever U is; a merged weight with padded
    rows (ldw > 2N) gives the same result as the unpadded one."""
    g = np.random.default_rng(9)
    X = bits(g.standard_normal((5, 16)))
    Wg = bits(np.zeros((16, 4))); Wu = bits(g.standard_normal((16, 4)))
    Z, *_ = oracle_mod.swiglu_bf16(X, _merged(Wg, Wu))
    assert np.all(Z == 0)
    Wg = bits(g.standard_normal((16, 4)))
    W = _merged(Wg, Wu)
    Wpad = np.zeros((16, 11), np.uint16); Wpad[:, :8] = W
    Z1, *_ = oracle_mod.swiglu_bf16(X, W)
    Z2, *_ = oracle_mod.swiglu_bf16(X, Wpad[:, :8])
    assert np.array_equal(Z1, Z2)


def test_swiglu_matches_its_parts(oracle_mod):
    """Z equals the plain products of the two halves, each rounded to bf16,
    through SiLU, rounded, and multiplied: assembled here from the separately
    pinned product and rounding functions."""
    g = np.random.default_rng(12)
    X = bits(g.standard_normal((6, 40)))
    Wg = bits(g.standard_normal((40, 5)) * 0.125); Wu = bits(g.standard_normal((40, 5)) * 0.125)
    Z, gg, uu, tt = oracle_mod.swiglu_bf16(X, _merged(Wg, Wu))
    G = oracle_mod.round_bf16_value(oracle_mod.gemm_bf16(X, Wg))
    U = oracle_mod.round_bf16_value(oracle_mod.gemm_bf16(X, Wu))
    T = oracle_mod.round_bf16_value(oracle_mod.silu(G))
    assert np.array_equal(gg, G) and np.array_equal(uu, U) and np.array_equal(tt, T)
    assert np.array_equal(Z, T * U)


def _e4m3_mags(oracle_mod):
    return [Fraction(float(v)) for v in oracle_mod.e4m3_decode(np.arange(127, dtype=np.uint8))]


def _nearest_code_of(y, mags):
    """Nearest E4M3FN code of the binary32 value y by brute force over the
    127 magnitudes in rational arithmetic, ties to the even code, beyond 448
    saturating."""
    q = min(abs(Fraction(float(y))), mags[-1])
    best = min(range(len(mags)), key=lambda c: (abs(q - mags[c]), c % 2))
    return (0x80 if math.copysign(1.0, float(y)) < 0 else 0x00) | best


def _fixed_quotient_f32(z, amax):
    """The binary32 steps of the fixed-range quantization, in numpy float32
    arithmetic (IEEE, correctly rounded): fl(fl(fl(z) * 448) / amax)."""
    with np.errstate(over="ignore"):
        return (np.float32(z) * np.float32(448.0)) / np.float32(amax)


def test_swiglu_e4m3_codes_brute_force(oracle_mod):
    """Section 5.3.1 quantizes Z = SiLU(G) (.) U with one fixed scale: each
    code is the E4M3FN value nearest to the binary32 quotient z * 448 / amax,
    z the bf16 value the unfused program stores (section 5.4.3 keeps that
    rounding under fusion).  Checked element by element against numpy's
    float32 arithmetic and a brute-force rational nearest-value search, for
    a range that saturates a fifth of the outputs and for one that saturates
    none (both a bf16 value and a general binary32 value)."""
    mags = _e4m3_mags(oracle_mod)
    g = np.random.default_rng(31)
    X = bits(g.standard_normal((7, 48)))
    W = _merged(bits(g.standard_normal((48, 9)) * 0.25), bits(g.standard_normal((48, 9)) * 0.25))
    Z, gg, uu, tt = oracle_mod.swiglu_bf16(X, W)
    top = float(np.abs(Z).max())
    for amax in (np.float32(np.quantile(np.abs(Z), 0.8)), np.float32(top * 1.0001), np.float32(0.75)):
        Q = oracle_mod.swiglu_e4m3(X, W, amax)
        for (i, j), z in np.ndenumerate(oracle_mod.round_bf16_value(tt * uu)):
            assert int(Q[i, j]) == _nearest_code_of(_fixed_quotient_f32(z, amax), mags), (amax, i, j)
    sat = oracle_mod.swiglu_e4m3(X, W, np.float32(np.quantile(np.abs(Z), 0.8)))
    assert 0.1 < np.mean((sat & 0x7f) == 0x7e) < 0.3


def test_swiglu_e4m3_closed_forms(oracle_mod):
    """With amax = 448 the quotient is z itself: z = t * u on an E4M3FN value
    keeps it exactly, z on a midpoint goes to the even neighbour, z beyond
    448 saturates, and a zero gate (SiLU(0) = 0) or -0 gives the signed zero
    code.  g >= 17 keeps t = g (SiLU(g) rounds to g in bf16)."""
    d = lambda c: float(oracle_mod.e4m3_decode([c])[0])
    # gate 32, up u: z = 32 u
    ups = [0.25, 1.5 / 32, -3.0 / 32, 1.0625 / 32, 1.1875 / 32, 500.0 / 32, -480.0 / 32, 0.0]
    X = bits([[1.0]])
    Wg = bits([[32.0] * len(ups)]); Wu = bits([ups])
    Q = oracle_mod.swiglu_e4m3(X, _merged(Wg, Wu), 448.0)[0]
    assert [d(c) for c in Q[:3]] == [8.0, 1.5, -3.0]           # exact E4M3FN values
    assert d(Q[3]) == 1.0 and d(Q[4]) == 1.25                  # ties: 1.0625 -> 1.0, 1.1875 -> 1.25 (even)
    assert Q[5] == 0x7e and Q[6] == 0xfe                       # +-448
    assert Q[7] == 0x00
    Qz = oracle_mod.swiglu_e4m3(bits([[1.0]]), _merged(bits([[0.0]]), bits([[-5.0]])), 1.0)
    assert Qz[0, 0] == 0x80                                    # 0 * -5 = -0
    # the range scales the quotient: amax = 4 * 448 divides z by 4
    Q4 = oracle_mod.swiglu_e4m3(X, _merged(Wg, Wu), 4 * 448.0)[0]
    assert [d(c) for c in Q4[:3]] == [2.0, 0.375, -0.75]


def test_swiglu_e4m3_decision_in_binary32(oracle_mod):
    """The page leaves the quotient's precision open; the oracle takes it in
    binary32.  For a range amax that is no bf16 value, the exact quotient can
    lie just above a midpoint while its binary32 rounding lands on it: the
    oracle then takes the even neighbour, as the binary32 quotient says, not
    the odd one the exact quotient is nearer to.  Such pairs are found by
    search and checked in rational arithmetic."""
    mags = _e4m3_mags(oracle_mod)
    found = 0
    X = bits([[1.0]])
    for mid_lo in range(40, 100):                              # midpoints between codes c and c + 1
        m = (mags[mid_lo] + mags[mid_lo + 1]) / 2
        z = 17.0 * float(np.float32(mags[mid_lo]))             # z = 17 v, exact in bf16 * bf16
        a0 = np.float32(float(Fraction(z) * 448 / m))
        for amax in (a0, np.nextafter(a0, np.float32(0)), np.nextafter(a0, np.float32(1e30))):
            exact = Fraction(z) * 448 / Fraction(float(amax))
            y = _fixed_quotient_f32(z, amax)
            if Fraction(float(y)) != m or exact == m:
                continue
            Q = oracle_mod.swiglu_e4m3(X, _merged(bits([[17.0]]), bits([[float(mags[mid_lo])]])), amax)
            even = mid_lo if mid_lo % 2 == 0 else mid_lo + 1
            nearer = mid_lo + 1 if exact > m else mid_lo
            assert int(Q[0, 0]) == even
            found += even != nearer
    assert found >= 1                                          # the pin separates the two readings


def test_silu_mul_chain_matches_swiglu(oracle_mod):
    """The activation chain on stored G and U (section 5.3.1, Example 5-4)
    is the element-wise part of the SwiGLU reference: fed the bf16 g and u
    that the pinned SwiGLU reference rounds its products to, it returns the
    same t and z."""
    g = np.random.default_rng(33)
    X = bits(g.standard_normal((5, 24)))
    W = _merged(bits(g.standard_normal((24, 7)) * 0.5), bits(g.standard_normal((24, 7)) * 0.5))
    Z, gg, uu, tt = oracle_mod.swiglu_bf16(X, W)
    t, z = oracle_mod.silu_mul_bf16(bits(gg), bits(uu))
    assert np.array_equal(t, tt) and np.array_equal(z, Z)


def test_silu_mul_chain_closed_forms(oracle_mod):
    """t = bf16(SiLU(g)): SiLU(1) = 0.7310585... rounds to 187 * 2^-8, so
    with u = 3, z = 2.19140625; SiLU(0) = 0; SiLU(g) rounds to g for g >= 17
    (e^-17 < 2^-24); SiLU(-90) ~ -7.4e-38 is a tiny negative bf16 value
    whose product with a positive u keeps the sign; SiLU(-100) ~ -3.7e-42
    lies below half the smallest bf16 subnormal (2^-134) and rounds to -0."""
    G = bits([1.0, 0.0, 17.0, 250.0, -90.0, -100.0])
    U = bits([3.0, -5.0, 0.5, -2.0, 1.0, 1.0])
    t, z = oracle_mod.silu_mul_bf16(G, U)
    assert t[0] == 187 * 2.0 ** -8 and z[0] == 2.19140625
    assert t[1] == 0.0 and z[1] == 0.0 and math.copysign(1.0, z[1]) < 0   # 0 * -5 = -0
    assert t[2] == 17.0 and z[2] == 8.5 and t[3] == 250.0 and z[3] == -500.0
    assert -1e-37 < t[4] < -1e-38 and z[4] == t[4]
    assert t[5] == 0.0 and math.copysign(1.0, t[5]) < 0


# ---------------------------------------------------------------- affine epilogue

def test_affine_reduces_to_product(oracle_mod):
    """alpha = 1, no bias, beta = 0 is the plain product; alpha scales it."""
    A, B = gi.small_case("bf16", 5, 6, 7, seed=3)
    P = oracle_mod.gemm_bf16(A, B)
    assert np.array_equal(oracle_mod.gemm_bf16_affine(A, B), P)
    assert np.array_equal(oracle_mod.gemm_bf16_affine(A, B, alpha=-2.5), -2.5 * P)


def test_affine_bias_and_old_c_closed_forms(oracle_mod):
    """With A = 0 the result is bias[j] + beta * C_old[i][j] exactly (both
    bf16 and float C_old); with identity A it is alpha * B + bias + beta * C_old."""
    M, N = 4, 6
    A0 = np.zeros((M, 3), np.uint16)
    B = bits(np.arange(3 * N, dtype=np.float32).reshape(3, N))
    bias = bits(np.array([1, -2, 0.5, 4, -0.25, 8], np.float32))
    old = np.arange(M * N, dtype=np.float32).reshape(M, N) - 7
    got = oracle_mod.gemm_bf16_affine(A0, B, alpha=3.0, bias=bias, beta=0.5, C_old=bits(old))
    want = gi.bf16_bits_to_f32(bias)[None, :].astype(np.float64) + 0.5 * gi.bf16_bits_to_f32(bits(old))
    assert np.array_equal(got, want)
    got32 = oracle_mod.gemm_bf16_affine(A0, B, alpha=3.0, bias=None, beta=-1.0, C_old=old)
    assert np.array_equal(got32, -old.astype(np.float64))
    I = bits(np.eye(3, dtype=np.float32))
    got_i = oracle_mod.gemm_bf16_affine(I, B, alpha=2.0, bias=bias, beta=1.0, C_old=old[:3])
    want_i = 2.0 * gi.bf16_bits_to_f32(B) + gi.bf16_bits_to_f32(bias)[None, :] + old[:3]
    assert np.array_equal(got_i, want_i.astype(np.float64))


def test_affine_ignores_old_c_when_beta_is_zero(oracle_mod):
    """beta = 0 never reads C_old (NaN there does not propagate)."""
    A, B = gi.small_case("bf16", 3, 4, 5, seed=4)
    old = np.full((3, 4), np.nan, np.float32)
    assert np.all(np.isfinite(oracle_mod.gemm_bf16_affine(A, B, beta=0.0, C_old=old)))
