"""Seeded synthetic inputs for the dense-GEMM workloads.

This module is shared by the GPU tests, the benchmark and the CPU oracle's
callers.  It holds no GEMM arithmetic: only random draws, the float32 -> bf16
rounding that turns the draws into bf16 operands, and the shapes of the five
workloads.  It imports neither the GPU package nor the oracle.

Generator: numpy PCG64 via ``default_rng([seed, tensor_id])`` with
``seed = 20260 + workload index``.  Uniform[-1, 1] is ``2*u - 1`` with u a
float32 uniform draw; N(0, s^2) is a float32 standard normal times s (s=0.125
is exact for N(0, 1/64)).  bf16 operands are the float32 draws rounded to
nearest, ties to even.
"""
import numpy as np

SEED_BASE = 20260

# Workload indices (position in the list of five workloads).
W_SGEMM_SMALL = 0     # FP32 256^3
W_SGEMM_LARGE = 1     # FP32 4096^3
W_FFN = 2             # BF16 1024x4096 . 4096x12288 -> bf16
W_DECODE = 3          # BF16 M in {1,4,16} x 4096 . 4096x12288 -> bf16
W_BATCHED = 4         # 32 x (1024x128 . 128x1024) -> f32, plus ragged 1000x12280x4100


def rng(workload, tensor_id):
    return np.random.default_rng([SEED_BASE + int(workload), int(tensor_id)])


def uniform_pm1(g, shape):
    return (2.0 * g.random(shape, dtype=np.float32) - 1.0).astype(np.float32)


def normal(g, shape, scale=1.0):
    x = g.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


def to_bf16_bits(x):
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even.
    NaN inputs become a quiet NaN; the workloads never produce NaN/Inf."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    t = u >> np.uint32(16)
    t &= np.uint32(1)                 # lsb of the kept half
    t += np.uint32(0x7FFF)
    t += u                            # wraps only for NaN patterns, fixed below
    t >>= np.uint32(16)
    r = t.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
    return r


def bf16_bits_to_f32(b):
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---- the five workloads ---------------------------------------------------

def sgemm_inputs(n=256, workload=W_SGEMM_SMALL, m=None, k=None):
    """FP32 A[m,k], B[k,n] i.i.d. uniform[-1,1]."""
    m = n if m is None else m
    k = n if k is None else k
    A = uniform_pm1(rng(workload, 0), (m, k))
    B = uniform_pm1(rng(workload, 1), (k, n))
    return A, B


def ffn_inputs(M=1024, K=4096, N=12288, workload=W_FFN):
    """X ~ N(0,1) [M,K], W ~ N(0,1/64) [K,N], both bf16 bit patterns."""
    X = to_bf16_bits(normal(rng(workload, 0), (M, K)))
    W = to_bf16_bits(normal(rng(workload, 1), (K, N), 0.125))
    return X, W


def decode_inputs(M, K=4096, N=12288, workload=W_DECODE):
    """X ~ N(0,1) [M,K] (the first M rows of one 16-row draw, so smaller M are
    prefixes of larger M), W ~ N(0,1/64) [K,N]; bf16 bit patterns."""
    if not 1 <= M <= 16:
        raise ValueError("decode workload has 1 <= M <= 16")
    X16 = to_bf16_bits(normal(rng(workload, 0), (16, K)))
    W = to_bf16_bits(normal(rng(workload, 1), (K, N), 0.125))
    return np.ascontiguousarray(X16[:M]), W


def swiglu_inputs(M=1024, K=4096, N=12288, workload=W_FFN):
    """The FFN's two projections that share X, with a merged weight:
    X ~ N(0,1) [M,K] (the FFN projection's X), Wgu [K,2N] = [W_g | W_u] with
    W_g the FFN projection's weight and W_u a second N(0,1/64) draw (tensor
    id 4); bf16 bit patterns."""
    X, Wg = ffn_inputs(M, K, N, workload)
    Wu = to_bf16_bits(normal(rng(workload, 4), (K, N), 0.125))
    return X, np.ascontiguousarray(np.concatenate([Wg, Wu], axis=1))


def act_chain_inputs(M=1024, N=12288, workload=W_FFN):
    """The stored gate and up activations of the FFN, G and U [M, N], for the
    activation chain that follows the projections: each ~ N(0, 64), the
    distribution of X.W for X ~ N(0,1) and W ~ N(0,1/64) over K = 4096
    (tensor ids 6 and 7); bf16 bit patterns."""
    G = to_bf16_bits(normal(rng(workload, 6), (M, N), 8.0))
    U = to_bf16_bits(normal(rng(workload, 7), (M, N), 8.0))
    return G, U


def wgrad_inputs(tokens=1024, d_in=4096, d_out=12288, workload=W_FFN):
    """The weight gradient of the FFN projection, dW = X^T . dY: X ~ N(0,1)
    [tokens, d_in] (the FFN projection's X, given as At [K, M] with
    K = tokens, M = d_in) and dY ~ N(0, 1/64) [tokens, d_out] (tensor id 5);
    bf16 bit patterns."""
    X = to_bf16_bits(normal(rng(workload, 0), (tokens, d_in)))
    dY = to_bf16_bits(normal(rng(workload, 5), (tokens, d_out), 0.125))
    return X, dY


def batched_inputs(batch=32, M=1024, N=1024, K=128, workload=W_BATCHED):
    """Q ~ N(0,1) [batch,M,K] and Kmat ~ N(0,1) [batch,N,K] in bf16; the B
    operand is the materialised row-major transpose Kmat^T [batch,K,N]."""
    Q = to_bf16_bits(normal(rng(workload, 0), (batch, M, K)))
    Km = to_bf16_bits(normal(rng(workload, 1), (batch, N, K)))
    KT = np.ascontiguousarray(np.transpose(Km, (0, 2, 1)))
    return Q, KT


def ragged_inputs(M=1000, N=12280, K=4100, workload=W_BATCHED):
    """A ~ N(0,1) [M,K], B ~ N(0,1) [K,N], bf16 bit patterns."""
    A = to_bf16_bits(normal(rng(workload, 2), (M, K)))
    B = to_bf16_bits(normal(rng(workload, 3), (K, N)))
    return A, B


def small_case(kind, M, N, K, seed=0, scale_b=1.0):
    """Seeded small operands for parity sweeps: kind 'f32' gives uniform[-1,1]
    float32, kind 'bf16' gives N(0,1) bf16 bit patterns (B scaled by scale_b)."""
    g = np.random.default_rng([SEED_BASE + 1000 + int(seed), M, N, K])
    if kind == "f32":
        return uniform_pm1(g, (M, K)), uniform_pm1(g, (K, N))
    return to_bf16_bits(normal(g, (M, K))), to_bf16_bits(normal(g, (K, N), scale_b))
