"""ctypes wrapper around oracle_gemm.c -- test infrastructure only.

The C file holds the arithmetic (plain FP64 triple loop, bit-level bf16
rounding); this module only builds it with gcc, loads it and marshals numpy
arrays.  Nothing here imports the GPU package.
"""
import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle_gemm.c")
_LIB = os.path.join(_HERE, "liboracle_gemm.so")
_lib = None


def lib_path():
    return _LIB


def build(verbose=False):
    """Compile the oracle with gcc (-O2, OpenMP, no FP contraction)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-shared", "-fPIC", "-std=c11", "-Wall", "-o", _LIB + ".tmp", _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    i64, p = ctypes.c_int64, ctypes.c_void_p
    lib.oracle_gemm_f64_from_f32.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64]
    lib.oracle_gemm_f64_from_bf16.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64]
    lib.oracle_gemm_f64_batched_from_bf16.argtypes = [i64, i64, i64, i64, p, i64, i64,
                                                      p, i64, i64, p, i64, i64]
    lib.oracle_dot_f64_from_bf16.argtypes = [i64, p, p, i64, i64]
    lib.oracle_dot_f64_from_bf16.restype = ctypes.c_double
    lib.oracle_dot_f64_from_f32.argtypes = [i64, p, p, i64, i64]
    lib.oracle_dot_f64_from_f32.restype = ctypes.c_double
    lib.oracle_round_bf16_array.argtypes = [i64, p, p]
    lib.oracle_round_bf16_d_array.argtypes = [i64, p, p]
    lib.oracle_silu_array.argtypes = [i64, p, p]
    lib.oracle_gemm_bf16_silu.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64]
    lib.oracle_swiglu_bf16.argtypes = [i64, i64, i64, p, i64, p, i64, p, p, p, p, i64]
    lib.oracle_gemm_bf16_affine.argtypes = [i64, i64, i64, p, i64, p, i64, ctypes.c_double, p, ctypes.c_double,
                                            p, i64, ctypes.c_int, p, i64]
    lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_decode.restype = ctypes.c_double
    lib.oracle_e4m3_encode.argtypes = [ctypes.c_double]
    lib.oracle_e4m3_encode.restype = ctypes.c_uint8
    lib.oracle_e4m3_encode_array.argtypes = [i64, p, p]
    lib.oracle_quantize_fixed_e4m3.argtypes = [i64, p, ctypes.c_float, p]
    lib.oracle_quantize_fixed_e4m3.restype = None
    lib.oracle_silu_mul_bf16.argtypes = [i64, p, p, p, p]
    lib.oracle_silu_mul_bf16.restype = None
    lib.oracle_quantize_rows_e4m3.argtypes = [i64, i64, p, i64, p, i64, p]
    lib.oracle_gemm_fp8_nt.argtypes = [i64, i64, i64, p, i64, p, p, i64, p, p, i64]
    lib.oracle_gemm_fp8_nt_affine.argtypes = [i64, i64, i64, p, i64, p, p, i64, p, ctypes.c_double, p,
                                              ctypes.c_double, p, i64, ctypes.c_int, p, i64]
    lib.oracle_gemm_fp8_nt_affine.restype = None
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_num_threads.restype = None
    _lib = lib
    return lib


def _rows(a, dtype):
    """Return (array, leading dimension) for a 2-D row-major view with unit
    column stride (rows may be padded, e.g. a column slice of a wider array)."""
    if a.ndim != 2 or a.dtype != dtype:
        raise TypeError(f"expected a 2-D {dtype} array, got {a.dtype} {a.shape}")
    item = a.dtype.itemsize
    if a.size == 0:
        return a, max(a.shape[1], 1)
    if a.shape[1] > 1 and a.strides[1] != item:
        raise ValueError("column stride must be 1 element")
    if a.shape[0] > 1 and (a.strides[0] % item or a.strides[0] < a.shape[1] * item):
        raise ValueError("row stride must be a whole number of elements >= columns")
    ld = a.strides[0] // item if a.shape[0] > 1 else max(a.shape[1], 1)
    return a, ld


def gemm_f32(A, B):
    """C = A.B in double from float32 inputs (unrounded)."""
    A, lda = _rows(A, np.float32)
    B, ldb = _rows(B, np.float32)
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    C = np.empty((M, N), np.float64)
    _load().oracle_gemm_f64_from_f32(M, N, K, A.ctypes.data, lda, B.ctypes.data, ldb,
                                     C.ctypes.data, max(N, 1))
    return C


def gemm_bf16(A, B):
    """C = A.B in double from bf16 bit patterns (uint16 arrays)."""
    A, lda = _rows(A, np.uint16)
    B, ldb = _rows(B, np.uint16)
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    C = np.empty((M, N), np.float64)
    _load().oracle_gemm_f64_from_bf16(M, N, K, A.ctypes.data, lda, B.ctypes.data, ldb,
                                      C.ctypes.data, max(N, 1))
    return C


def gemm_bf16_batched(A, B):
    """C[b] = A[b].B[b] for contiguous 3-D uint16 stacks; returns double [batch,M,N]."""
    if A.ndim != 3 or B.ndim != 3 or A.dtype != np.uint16 or B.dtype != np.uint16:
        raise TypeError("expected 3-D uint16 stacks")
    A = np.ascontiguousarray(A)
    B = np.ascontiguousarray(B)
    batch, M, K = A.shape
    b2, K2, N = B.shape
    if batch != b2 or K != K2:
        raise ValueError("shape mismatch")
    C = np.empty((batch, M, N), np.float64)
    _load().oracle_gemm_f64_batched_from_bf16(batch, M, N, K, A.ctypes.data, K, M * K,
                                              B.ctypes.data, N, K * N,
                                              C.ctypes.data, N, M * N)
    return C


def dot_bf16(A, B, i, j):
    """One element C[i, j] of A.B (bf16 bit patterns), in double."""
    A, lda = _rows(A, np.uint16)
    B, ldb = _rows(B, np.uint16)
    K = A.shape[1]
    row = A[i]
    return _load().oracle_dot_f64_from_bf16(K, row.ctypes.data, B.ctypes.data, ldb, int(j))


def dot_f32(A, B, i, j):
    """One element C[i, j] of A.B (float32), in double."""
    A, lda = _rows(A, np.float32)
    B, ldb = _rows(B, np.float32)
    K = A.shape[1]
    row = A[i]
    return _load().oracle_dot_f64_from_f32(K, row.ctypes.data, B.ctypes.data, ldb, int(j))


def round_bf16(x):
    """float32 array -> bf16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(np.asarray(x, np.float32))
    out = np.empty(x.shape, np.uint16)
    _load().oracle_round_bf16_array(x.size, x.ctypes.data, out.ctypes.data)
    return out


def round_bf16_value(x):
    """Nearest bf16 value (ties to even) of each double, as doubles."""
    x = np.ascontiguousarray(np.asarray(x, np.float64))
    out = np.empty(x.shape, np.float64)
    _load().oracle_round_bf16_d_array(x.size, x.ctypes.data, out.ctypes.data)
    return out


def silu(x):
    """SiLU(x) = x / (1 + e^-x), elementwise in double."""
    x = np.ascontiguousarray(np.asarray(x, np.float64))
    out = np.empty(x.shape, np.float64)
    _load().oracle_silu_array(x.size, x.ctypes.data, out.ctypes.data)
    return out


def gemm_bf16_silu(A, B):
    """Y = SiLU(round_bf16(A.B)) in double from bf16 bit patterns."""
    A, lda = _rows(A, np.uint16)
    B, ldb = _rows(B, np.uint16)
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    Y = np.empty((M, N), np.float64)
    _load().oracle_gemm_bf16_silu(M, N, K, A.ctypes.data, lda, B.ctypes.data, ldb, Y.ctypes.data, max(N, 1))
    return Y


def swiglu_bf16(X, Wgu):
    """SwiGLU on a merged [K, 2N] gate/up weight (gate in the first N
    columns): returns (Z, g, u, t) in double, Z = t * u unrounded."""
    X, ldx = _rows(X, np.uint16)
    Wgu, ldw = _rows(Wgu, np.uint16)
    M, K = X.shape
    K2, N2 = Wgu.shape
    if K != K2 or N2 % 2:
        raise ValueError("expected X [M,K] and Wgu [K,2N]")
    N = N2 // 2
    Z, g, u, t = (np.empty((M, N), np.float64) for _ in range(4))
    _load().oracle_swiglu_bf16(M, N, K, X.ctypes.data, ldx, Wgu.ctypes.data, ldw, Z.ctypes.data,
                               g.ctypes.data, u.ctypes.data, t.ctypes.data, max(N, 1))
    return Z, g, u, t


def gemm_bf16_affine(A, B, alpha=1.0, bias=None, beta=0.0, C_old=None):
    """alpha * (A.B) + bias[j] + beta * C_old[i][j] in double; A, B, bias and a
    bf16 C_old as bf16 bit patterns (uint16), or a float32 C_old."""
    A, lda = _rows(A, np.uint16)
    B, ldb = _rows(B, np.uint16)
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    bias_p = None if bias is None else np.ascontiguousarray(bias, np.uint16)
    if beta != 0.0:
        old_f32 = C_old.dtype == np.float32
        C_old, ldo = _rows(C_old, np.float32 if old_f32 else np.uint16)
        old_p = C_old.ctypes.data
    else:
        old_f32, ldo, old_p = False, 1, None
    C = np.empty((M, N), np.float64)
    _load().oracle_gemm_bf16_affine(M, N, K, A.ctypes.data, lda, B.ctypes.data, ldb, float(alpha),
                                    None if bias_p is None else bias_p.ctypes.data, float(beta), old_p, ldo,
                                    int(old_f32), C.ctypes.data, max(N, 1))
    return C


def e4m3_decode(codes):
    """Values of E4M3FN codes (uint8), as doubles."""
    codes = np.asarray(codes, np.uint8)
    L = _load()
    return np.array([L.oracle_e4m3_decode(int(c)) for c in codes.ravel()], np.float64).reshape(codes.shape)


def e4m3_encode(x):
    """Nearest E4M3FN codes (ties to even, saturating at 448) of doubles."""
    x = np.ascontiguousarray(np.asarray(x, np.float64))
    out = np.empty(x.shape, np.uint8)
    _load().oracle_e4m3_encode_array(x.size, x.ctypes.data, out.ctypes.data)
    return out


def quantize_fixed_e4m3(v, amax):
    """Fixed-range E4M3FN codes of values v (doubles): the value nearest to
    fl32(fl32(fl32(v) * 448) / amax), saturating at 448."""
    amax = float(np.float32(amax))
    if not (math.isfinite(amax) and amax > 0):
        raise ValueError("amax must be finite and positive")
    v = np.ascontiguousarray(np.asarray(v, np.float64))
    out = np.empty(v.shape, np.uint8)
    _load().oracle_quantize_fixed_e4m3(v.size, v.ctypes.data, amax, out.ctypes.data)
    return out


def swiglu_e4m3(X, Wgu, amax):
    """SwiGLU on a merged [K, 2N] weight with its output quantized to E4M3FN
    codes against the fixed range amax (uint8 [M, N]): the codes of the bf16
    Z the unfused program stores."""
    Z, _, _, _ = swiglu_bf16(X, Wgu)
    return quantize_fixed_e4m3(round_bf16_value(Z), amax)


def silu_mul_bf16(G, U):
    """The activation chain on stored bf16 G and U (bit patterns, same
    shape): returns (t, z) in double, t = bf16(SiLU(g)), z = t * u
    unrounded."""
    G = np.ascontiguousarray(G, np.uint16)
    U = np.ascontiguousarray(U, np.uint16)
    if G.shape != U.shape:
        raise ValueError("G and U differ in shape")
    t, z = np.empty(G.shape, np.float64), np.empty(G.shape, np.float64)
    _load().oracle_silu_mul_bf16(G.size, G.ctypes.data, U.ctypes.data, t.ctypes.data, z.ctypes.data)
    return t, z


def quantize_rows_e4m3(X):
    """Per-row E4M3FN quantization of bf16 bit patterns X [rows, cols]:
    returns (codes uint8 [rows, cols], dequantization factors float32 [rows])."""
    X, ldx = _rows(X, np.uint16)
    rows, cols = X.shape
    Q = np.empty((rows, cols), np.uint8)
    s = np.empty(rows, np.float32)
    _load().oracle_quantize_rows_e4m3(rows, cols, X.ctypes.data, ldx, Q.ctypes.data, max(cols, 1), s.ctypes.data)
    return Q, s


def gemm_fp8_nt(A, sa, Bt, sb):
    """C = diag(sa) (dec(A) . dec(Bt)^T) diag(sb) in double; A [M,K], Bt [N,K]
    E4M3FN codes; sa [M], sb [N] float32 or None."""
    A, lda = _rows(A, np.uint8)
    Bt, ldb = _rows(Bt, np.uint8)
    M, K = A.shape
    N, K2 = Bt.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    sa_p = np.ascontiguousarray(sa, np.float32) if sa is not None else None
    sb_p = np.ascontiguousarray(sb, np.float32) if sb is not None else None
    C = np.empty((M, N), np.float64)
    _load().oracle_gemm_fp8_nt(M, N, K, A.ctypes.data, lda, None if sa_p is None else sa_p.ctypes.data,
                               Bt.ctypes.data, ldb, None if sb_p is None else sb_p.ctypes.data,
                               C.ctypes.data, max(N, 1))
    return C


def quantize_cols_e4m3(W):
    """Per-column E4M3FN quantization of bf16 bit patterns W [K, N] (a weight
    stored [in, out]): column j quantized with its own factor exactly as a
    row of quantize_rows_e4m3, returned transposed -- (codes uint8 [N, K],
    factors float32 [N]) -- the Bt operand of gemm_fp8_nt."""
    W = np.asarray(W, np.uint16)
    return quantize_rows_e4m3(np.ascontiguousarray(W.T))


def gemm_fp8_nt_affine(A, sa, Bt, sb, alpha=1.0, bias=None, beta=0.0, C_old=None):
    """alpha * D + bias[j] + beta * C_old[i][j] in double, D = gemm_fp8_nt(A,
    sa, Bt, sb); bias and a bf16 C_old as bf16 bit patterns, or a float32
    C_old."""
    A, lda = _rows(A, np.uint8)
    Bt, ldb = _rows(Bt, np.uint8)
    M, K = A.shape
    N, K2 = Bt.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    sa_p = np.ascontiguousarray(sa, np.float32) if sa is not None else None
    sb_p = np.ascontiguousarray(sb, np.float32) if sb is not None else None
    bias_p = None if bias is None else np.ascontiguousarray(bias, np.uint16)
    if beta != 0.0:
        old_f32 = C_old.dtype == np.float32
        C_old, ldo = _rows(C_old, np.float32 if old_f32 else np.uint16)
        old_p = C_old.ctypes.data
    else:
        old_f32, ldo, old_p = False, 1, None
    C = np.empty((M, N), np.float64)
    _load().oracle_gemm_fp8_nt_affine(M, N, K, A.ctypes.data, lda, None if sa_p is None else sa_p.ctypes.data,
                                      Bt.ctypes.data, ldb, None if sb_p is None else sb_p.ctypes.data, float(alpha),
                                      None if bias_p is None else bias_p.ctypes.data, float(beta), old_p, ldo,
                                      int(old_f32), C.ctypes.data, max(N, 1))
    return C


def num_threads():
    return int(_load().oracle_num_threads())


def set_num_threads(n):
    """Thread count of the oracle's parallel loops (results do not depend on it)."""
    _load().oracle_set_num_threads(int(n))
