"""Helpers shared by the GPU test modules: host <-> device marshalling of
bf16 bit patterns and the parity tolerances.  No GEMM arithmetic here."""
import math

import numpy as np
import torch

import gemm_inputs as gi


def dev_bf16(bits):
    """uint16 bf16 bit patterns (numpy) -> torch.bfloat16 on cuda:0."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def dev_f32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def host_bits(t):
    """torch.bfloat16 tensor -> uint16 numpy bit patterns."""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_values(t):
    """GPU result (bf16 or f32) -> float64 numpy values."""
    if t.dtype == torch.bfloat16:
        return gi.bf16_bits_to_f32(host_bits(t)).astype(np.float64)
    return t.float().cpu().numpy().astype(np.float64)


def tol_f32(K, amax, bmax):
    """FP32 bar: max |C - C_ref| <= 1e-5 * K * max|a| * max|b|."""
    return 1e-5 * max(K, 1) * amax * bmax


def check_f32(C, ref, K, amax, bmax, what=""):
    err = np.abs(C - ref)
    bound = tol_f32(K, amax, bmax)
    worst = float(err.max()) if err.size else 0.0
    assert np.all(np.isfinite(C)), f"{what}: non-finite output"
    assert worst <= bound, f"{what}: max err {worst:.3e} > bound {bound:.3e}"
    return worst / bound if bound > 0 else 0.0


def check_bf16(C, ref, K, what=""):
    """BF16-output bar: |C - C_ref| <= 2^-8 |C_ref| + 1e-3 sqrt(K), per element."""
    bound = 2.0 ** -8 * np.abs(ref) + 1e-3 * math.sqrt(max(K, 1))
    err = np.abs(C - ref)
    assert np.all(np.isfinite(C)), f"{what}: non-finite output"
    bad = err > bound
    if bad.any():
        idx = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} elements out of bound, first at {tuple(idx)}: "
                             f"got {C[tuple(idx)]!r} want {ref[tuple(idx)]!r}")
    return float((err / bound).max()) if err.size else 0.0


def amax_bf16(bits):
    return float(np.abs(gi.bf16_bits_to_f32(bits)).max()) if bits.size else 0.0


# Fused epilogues.  The kernel rounds its FP32 product g_k to bf16, the
# oracle rounds the exact product G; within the bf16 GEMM bar the two
# rounded values differ by at most
#     dg = 3 * 2^-9 |G| + 1e-3 sqrt(K)
# (the kernel's bf16 output is within 2^-8 |G| + 1e-3 sqrt(K) of G, the
# oracle's within 2^-9 |G|).  SiLU is Lipschitz with constant max|SiLU'| =
# 1.0998 < 1.1, and every further rounding to bf16 adds at most 2^-9 of the
# value (2^-8 is used to cover the FP32 evaluation of SiLU as well).

def _dg(G, K):
    return 3 * 2.0 ** -9 * np.abs(G) + 1e-3 * math.sqrt(max(K, 1))


def check_silu(Y, G, Yref, K, what=""):
    """|y - Y_ref| <= 1.1 dg (1 + 2^-9) + 2^-8 |Y_ref|, with G the exact product."""
    bound = 1.1 * _dg(G, K) * (1 + 2.0 ** -9) + 2.0 ** -8 * np.abs(Yref)
    return _check(Y, Yref, bound, what)


def check_swiglu(Z, G, U, t, u, Zref, K, what=""):
    """t = bf16(SiLU(g)) differs by dt = 1.1 dg (1 + 2^-9) + 2^-8 |t| and u by
    du = dg(U); the product by dt (|u| + du) + |t| du; the final rounding
    adds 2^-8 |Z_ref|."""
    dt = 1.1 * _dg(G, K) * (1 + 2.0 ** -9) + 2.0 ** -8 * np.abs(t)
    du = _dg(U, K)
    bound = (dt * (np.abs(u) + du) + np.abs(t) * du) * (1 + 2.0 ** -9) + 2.0 ** -8 * np.abs(Zref)
    return _check(Z, Zref, bound, what)


# E4M3FN codes of the SwiGLU output (fixed range amax).  A code has 3
# mantissa bits, so the bf16 GEMM bar above is far too loose to decide one;
# the check instead bounds what the kernel can have computed.  Its FP32 sum
# of K exact bf16 products is within K 2^-24 S of the exact sum (S the sum of
# the products' magnitudes; any order of K - 1 additions, each rounding at
# most 2^-24 of a partial sum no larger than S), so its bf16 g and u lie
# between the bf16 roundings of the interval's ends; SiLU in FP32 (exp and
# reciprocal of a few ulp, a relative error below 2^-17 for |g| < 100) and its
# bf16 rounding give t between the rounded ends of the SiLU image of that
# range (SiLU falls below x = -1.27846 and rises above it); t * u lies
# between the corner products and its bf16 rounding z (the value quantized)
# between their roundings; the binary32 quotient z * 448 / amax moves by at
# most 2^-22 relative.  The kernel's code must lie between the codes of the
# two ends, and equal them where they coincide.

SILU_ARGMIN = -1.2784645427610738


def swiglu_sums(oracle_mod, X, Wgu):
    """The exact gate and up sums G, U and the sums of their terms'
    magnitudes SG, SU (oracle products of bf16 bit patterns)."""
    N = Wgu.shape[1] // 2
    Wg, Wu = np.ascontiguousarray(Wgu[:, :N]), np.ascontiguousarray(Wgu[:, N:])
    Xa = X & 0x7fff
    return (oracle_mod.gemm_bf16(X, Wg), oracle_mod.gemm_bf16(X, Wu),
            oracle_mod.gemm_bf16(Xa, Wg & 0x7fff), oracle_mod.gemm_bf16(Xa, Wu & 0x7fff))


def swiglu_code_range(oracle_mod, X, Wgu, amax, sums=None):
    """(c_lo, c_hi): E4M3FN codes bracketing every code the kernel may give
    for SwiGLU(X, Wgu) against the range amax (bf16 bit patterns); `sums`:
    swiglu_sums of the same operands, when already computed."""
    K = X.shape[1]
    G, U, SG, SU = sums if sums is not None else swiglu_sums(oracle_mod, X, Wgu)
    e = 1.01 * K * 2.0 ** -24
    rb = oracle_mod.round_bf16_value
    g_lo, g_hi = rb(G - e * SG), rb(G + e * SG)
    u_lo, u_hi = rb(U - e * SU), rb(U + e * SU)
    s_lo, s_hi = oracle_mod.silu(g_lo), oracle_mod.silu(g_hi)
    tmin, tmax = np.minimum(s_lo, s_hi), np.maximum(s_lo, s_hi)
    tmin = np.where((g_lo < SILU_ARGMIN) & (g_hi > SILU_ARGMIN), oracle_mod.silu(np.array(SILU_ARGMIN)), tmin)
    t_lo = rb(tmin - 2.0 ** -17 * np.abs(tmin) - 1e-38)
    t_hi = rb(tmax + 2.0 ** -17 * np.abs(tmax) + 1e-38)
    corners = np.stack([t_lo * u_lo, t_lo * u_hi, t_hi * u_lo, t_hi * u_hi])
    s = 448.0 / float(np.float32(amax))
    y_lo, y_hi = rb(corners.min(0)) * s, rb(corners.max(0)) * s
    return (oracle_mod.e4m3_encode(y_lo - 2.0 ** -22 * np.abs(y_lo)),
            oracle_mod.e4m3_encode(y_hi + 2.0 ** -22 * np.abs(y_hi)))


def check_swiglu_codes(oracle_mod, Q, c_lo, c_hi, what="", min_unique=0.0):
    """Every code between c_lo and c_hi (by value), equal to them where they
    coincide; returns the fraction of such unique codes."""
    d = oracle_mod.e4m3_decode
    v, lo, hi = d(Q), d(c_lo), d(c_hi)
    assert not np.isnan(v).any(), f"{what}: NaN code"
    bad = (v < lo) | (v > hi)
    if bad.any():
        idx = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} codes outside their range, first at {idx}: "
                             f"got {int(Q[idx]):#04x} range [{int(c_lo[idx]):#04x}, {int(c_hi[idx]):#04x}]")
    uniq = c_lo == c_hi
    wrong = uniq & (Q != c_lo)
    if wrong.any():
        idx = tuple(np.argwhere(wrong)[0])
        raise AssertionError(f"{what}: {int(wrong.sum())} decided codes differ, first at {idx}: "
                             f"got {int(Q[idx]):#04x} want {int(c_lo[idx]):#04x}")
    frac = float(uniq.mean()) if uniq.size else 1.0
    assert frac >= min_unique, f"{what}: only {frac:.3f} of the codes are decided"
    return frac


def _check(C, ref, bound, what):
    err = np.abs(C - ref)
    assert np.all(np.isfinite(C)), f"{what}: non-finite output"
    bad = err > bound
    if bad.any():
        idx = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} elements out of bound, first at {idx}: "
                             f"got {C[idx]!r} want {ref[idx]!r} (bound {bound[idx]!r})")
    return float((err / bound).max()) if err.size else 0.0


# Affine epilogue C = alpha * S + bias + beta * C_old, evaluated by the kernel
# in FP32 from its FP32 sum S and rounded once.  S is within the accumulation
# part of the bf16 bar of the exact product P (2^-9 |P| + 1e-3 sqrt(K); the
# other 2^-9 |P| of that bar is the output rounding), scaled by |alpha|; the
# two FP32 fused multiply-adds add at most 2^-23 of the magnitudes they
# combine (2^-20 is used); the final rounding to bf16 at most 2^-9 |C_ref|
# (2^-8 is used), to float nothing beyond the FP32 bar.

def check_affine(C, ref, P, K, alpha, bias_vals, beta, old_vals, out_f32, amax=0.0, bmax=0.0, what=""):
    mags = np.abs(alpha * P) + np.abs(bias_vals)[None, :] + np.abs(beta * old_vals)
    if out_f32:
        acc = abs(alpha) * tol_f32(K, amax, bmax)
        bound = acc + 2.0 ** -20 * mags
    else:
        acc = abs(alpha) * (2.0 ** -9 * np.abs(P) + 1e-3 * math.sqrt(max(K, 1)))
        bound = 2.0 ** -8 * np.abs(ref) + acc + 2.0 ** -20 * mags
    return _check(C, ref, np.broadcast_to(bound, ref.shape), what)


_WS = None


def ws():
    """The test process's workspace (caller-owned scratch for gemm_run),
    created on first use on the current device and grown as calls need."""
    global _WS
    if _WS is None:
        import dense_gemm_05_amd as g5
        _WS = g5.Workspace()
    return _WS
