"""GPU parity of the activation chain on stored operands (gemm_act_chain)
against the oracle, through the C ABI.

Page "Operator & Runtime" §5.3.1, Example 5-4: with G and U stored, the
chain computes T = SiLU(G), Z = T (.) U and the codes of Z with one fixed
scale, each step alone or fused.  The oracle (silu_mul_bf16,
quantize_fixed_e4m3) works in double from the same bf16 inputs:
  * the product and the quantization take no transcendental step and are
    compared bit for bit;
  * SiLU is evaluated in FP32 by the kernel (hardware exponential and
    reciprocal: a relative error below 2^-20 + |g| 2^-22), so t may round
    to the neighbouring bf16 value where SiLU(g) lies that close to a
    midpoint between two bf16 values; everything downstream is bracketed
    by the two candidates and must equal the oracle where they coincide.
Fused and separate steps are also compared with each other, bit for bit.
"""
import math

import numpy as np
import pytest
import torch

import gemm_inputs as gi
from _gpu_helpers import dev_bf16

import dense_gemm_05_amd as g5

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[act-chain] {msg}", flush=True)


def _host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _vals(bits):
    return gi.bf16_bits_to_f32(np.ascontiguousarray(bits)).astype(np.float64)


def _t_range(oracle_mod, G):
    """bf16 values bracketing the kernel's t = bf16(SiLU_fp32(g))."""
    g = _vals(G)
    s = oracle_mod.silu(g)
    rel = 2.0 ** -20 + np.abs(g) * 2.0 ** -22
    with np.errstate(invalid="ignore"):
        lo = oracle_mod.round_bf16_value(s - rel * np.abs(s))
        hi = oracle_mod.round_bf16_value(s + rel * np.abs(s))
    return lo, hi


def _z_range(oracle_mod, G, U):
    t_lo, t_hi = _t_range(oracle_mod, G)
    u = _vals(U)
    a, b = t_lo * u, t_hi * u
    rb = oracle_mod.round_bf16_value
    return rb(np.minimum(a, b)), rb(np.maximum(a, b))


def _check_bracket(got, lo, hi, want, what, min_unique=0.99):
    """got within [lo, hi] (values; NaN where the oracle is NaN), equal to
    want where lo == hi."""
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan), f"{what}: NaN positions differ"
    g, l, h, w = got[~nan], lo[~nan], hi[~nan], want[~nan]
    bad = (g < l) | (g > h)
    assert not bad.any(), f"{what}: {int(bad.sum())} values outside their bracket"
    uniq = l == h
    assert np.array_equal(g[uniq], w[uniq]), f"{what}: {int((g[uniq] != w[uniq]).sum())} decided values differ"
    frac = float(uniq.mean()) if uniq.size else 1.0
    assert frac >= min_unique, f"{what}: only {frac:.4f} decided"
    return frac


def _layout(M, N, kind, dtype=torch.bfloat16):
    """An output tensor [M, N]: 'contig' (ld = N), 'padded' (ld = N rounded
    up to 16 elements, plus 16) or 'odd' (ld = N + 3 and an odd element
    offset: rows neither 16- nor 8-byte aligned)."""
    if kind == "contig":
        return torch.empty((M, N), dtype=dtype, device="cuda")
    if kind == "padded":
        ld = (N + 15) // 16 * 16 + 16
        return torch.empty((M, ld), dtype=dtype, device="cuda")[:, :N]
    ld = N + 3
    return torch.empty((M * ld + 1,), dtype=dtype, device="cuda")[1:].view(M, ld)[:, :N]


def _dev_like(bits, kind):
    t = _layout(bits.shape[0], bits.shape[1], kind)
    t.copy_(dev_bf16(bits))
    return t


CASES = [(1024, 12288, "contig"), (300, 392, "padded"), (37, 1003, "contig"), (64, 264, "odd")]


@pytest.mark.parametrize("M,N,kind", CASES)
def test_act_chain_steps(oracle_mod, M, N, kind):
    """Each step and each fusion on the page's shape [1024, 12288] and on
    ragged, padded and misaligned layouts (the last two run element by
    element), against the oracle."""
    _say(f"steps {M}x{N} {kind}")
    if (M, N) == (1024, 12288):
        G, U = gi.act_chain_inputs()
    else:
        g = np.random.default_rng([gi.SEED_BASE + 3500, M, N])
        G = gi.to_bf16_bits(gi.normal(g, (M, N), 8.0))
        U = gi.to_bf16_bits(gi.normal(g, (M, N), 8.0))
    dG, dU = _dev_like(G, kind), _dev_like(U, kind)
    t_ref, z_ref = oracle_mod.silu_mul_bf16(G, U)
    rb = oracle_mod.round_bf16_value

    # SiLU
    T = g5.act_silu(dG, _layout(M, N, kind))
    t = _vals(_host(T.view(torch.int16)).view(np.uint16))
    t_lo, t_hi = _t_range(oracle_mod, G)
    frac = _check_bracket(t, t_lo, t_hi, t_ref, "silu")
    _say(f"  silu decided {frac:.5f}")

    # the product of the stored T (the oracle's own t, so its result is fixed) and U
    Tb = gi.to_bf16_bits(t_ref.astype(np.float32))
    Z = g5.act_mul(_dev_like(Tb, kind), dU, _layout(M, N, kind))
    z = _vals(_host(Z.view(torch.int16)).view(np.uint16))
    assert np.array_equal(z, rb(t_ref * _vals(U))), "product step"

    # SiLU and the product fused
    Zf = g5.act_swiglu(dG, dU, _layout(M, N, kind))
    zf = _vals(_host(Zf.view(torch.int16)).view(np.uint16))
    z_lo, z_hi = _z_range(oracle_mod, G, U)
    _check_bracket(zf, z_lo, z_hi, rb(z_ref), "silu*u")

    # quantization of a stored Z (the oracle's own bf16 Z), bf16 and general ranges
    Zb = gi.to_bf16_bits(rb(z_ref).astype(np.float32))
    dZ = _dev_like(Zb, kind)
    for amax in (64.0, 61.7):
        Q = g5.act_quantize_e4m3(dZ, amax, _layout(M, N, kind, torch.uint8))
        want = oracle_mod.quantize_fixed_e4m3(_vals(Zb), np.float32(amax))
        assert np.array_equal(_host(Q), want), f"quantization amax={amax}"

    # all three fused: the codes of the fused bf16 Z
    d = oracle_mod.e4m3_decode
    for amax in (64.0, 61.7):
        Qf = _host(g5.act_swiglu_e4m3(dG, dU, amax, _layout(M, N, kind, torch.uint8)))
        c_lo = oracle_mod.quantize_fixed_e4m3(z_lo, np.float32(amax))
        c_hi = oracle_mod.quantize_fixed_e4m3(z_hi, np.float32(amax))
        want = oracle_mod.quantize_fixed_e4m3(rb(z_ref), np.float32(amax))
        _check_bracket(d(Qf), d(c_lo), d(c_hi), d(want), f"fused codes amax={amax}")


@pytest.mark.parametrize("kind", ["contig", "padded", "odd"])
def test_act_chain_fused_equals_separate(kind):
    """A fused step gives the same bits as the separate steps in sequence:
    SwiGLU = product(SiLU(G), U); the fused codes = quantization(SwiGLU);
    on whole-chunk and element-by-element layouts alike."""
    M, N = 200, 1000 if kind != "contig" else 1024
    _say(f"fused vs separate {M}x{N} {kind}")
    g = np.random.default_rng([gi.SEED_BASE + 3600, M, N])
    G = gi.to_bf16_bits(gi.normal(g, (M, N), 8.0))
    U = gi.to_bf16_bits(gi.normal(g, (M, N), 8.0))
    dG, dU = _dev_like(G, kind), _dev_like(U, kind)
    Zs = g5.act_mul(g5.act_silu(dG, _layout(M, N, kind)), dU, _layout(M, N, kind))
    Zf = g5.act_swiglu(dG, dU, _layout(M, N, kind))
    assert np.array_equal(_host(Zs.view(torch.int16)), _host(Zf.view(torch.int16)))
    for amax in (16.0, 15.3):
        Qs = g5.act_quantize_e4m3(Zf, amax, _layout(M, N, kind, torch.uint8))
        Qf = g5.act_swiglu_e4m3(dG, dU, amax, _layout(M, N, kind, torch.uint8))
        assert np.array_equal(_host(Qs), _host(Qf)), f"amax={amax}"


def test_act_chain_layouts_agree():
    """The 16-byte-chunk kernels (contiguous and padded rows) and the
    element-by-element kernel (misaligned rows) give the same bits."""
    M, N = 96, 1024
    g = np.random.default_rng([gi.SEED_BASE + 3700])
    G = gi.to_bf16_bits(gi.normal(g, (M, N), 8.0))
    U = gi.to_bf16_bits(gi.normal(g, (M, N), 8.0))
    outs = {}
    for kind in ("contig", "padded", "odd"):
        dG, dU = _dev_like(G, kind), _dev_like(U, kind)
        outs[kind] = (_host(g5.act_swiglu(dG, dU, _layout(M, N, kind)).view(torch.int16)),
                      _host(g5.act_swiglu_e4m3(dG, dU, 20.0, _layout(M, N, kind, torch.uint8))),
                      _host(g5.act_silu(dG, _layout(M, N, kind)).view(torch.int16)))
    for kind in ("padded", "odd"):
        for a, b in zip(outs["contig"], outs[kind]):
            assert np.array_equal(a, b), kind


def test_act_chain_special_values(oracle_mod):
    """Infinities, NaN, signed zeros, saturation and ties of the
    quantization; SiLU of +-inf (inf and NaN) and of signed zeros."""
    vals = np.array([np.inf, -np.inf, np.nan, 0.0, -0.0, 500.0, -500.0, 1.0625, 1.1875, 448.0, -3.0, 2.0 ** -10,
                     3 * 2.0 ** -11, 2.0 ** -12, 88.0, -88.0], np.float32)
    Z = gi.to_bf16_bits(np.tile(vals, (8, 1)))
    for amax in (448.0, 447.3):
        Q = _host(g5.act_quantize_e4m3(dev_bf16(Z), amax))
        want = oracle_mod.quantize_fixed_e4m3(_vals(Z), np.float32(amax))
        assert np.array_equal(Q, want), f"amax={amax}: got {Q[0]} want {want[0]}"
    T = _vals(_host(g5.act_silu(dev_bf16(Z)).view(torch.int16)).view(np.uint16))
    t_ref, _ = oracle_mod.silu_mul_bf16(Z, Z)
    assert np.array_equal(np.isnan(T), np.isnan(t_ref))
    assert T[0, 0] == np.inf and np.isnan(T[0, 1]) and np.isnan(T[0, 2])
    assert T[0, 3] == 0.0 and math.copysign(1.0, T[0, 4]) < 0 and T[0, 4] == 0.0


def test_act_chain_empty_and_errors():
    G = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    assert g5.act_silu(G).shape == (0, 64)
    Gs = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(g5.GemmError):
        g5.act_quantize_e4m3(Gs, 0.0)
    with pytest.raises(g5.GemmError):
        g5.act_swiglu(Gs, Gs, Gs)                # the output overlaps an input
