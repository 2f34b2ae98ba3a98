"""Thin Python binding of the C ABI in include/gemm05.h.

Argument marshalling only: the functions read sizes, row strides and data
pointers from torch tensors (device memory owned by the caller), pass the
current HIP stream, and raise on a nonzero status.  All arithmetic runs in
the gfx950 kernels of libgemm05.so.

Every bf16 / fp8 product takes an optional ``workspace``: a ``Workspace``
(caller-owned scratch memory, allocated through torch) or a uint8 device
tensor.  With one the call goes through ``gemm_run`` and may use the paths
that need scratch memory (K split over workgroups, the split small-M path,
realigned row copies); without one it calls the named entry point, which
takes the paths that need none.
"""
import ctypes

import torch

from . import _lib
from ._lib import GEMM_ERR_WORKSPACE, GEMM_WORKSPACE_COUNTER_BYTES, GemmError, GemmPlan, lib

__all__ = ["gemm_sgemm", "gemm_bf16", "gemm_bf16_batched", "gemm_bf16_nt", "gemm_bf16_nt_batched",
           "gemm_bf16_tn", "gemm_bf16_tn_batched",
           "gemm_bf16_silu", "gemm_bf16_swiglu", "gemm_bf16_silu_batched", "gemm_bf16_swiglu_batched",
           "gemm_bf16_swiglu_e4m3", "gemm_bf16_swiglu_e4m3_batched",
           "act_chain", "act_silu", "act_mul", "act_swiglu", "act_quantize_e4m3", "act_swiglu_e4m3",
           "gemm_fp8_quantize_rows", "gemm_fp8_quantize_cols", "gemm_fp8_nt", "gemm_fp8_nt_affine",
           "gemm_fp8_nt_quant_a",
           "gemm_bf16_affine",
           "gemm_bf16_nt_affine", "gemm_bf16_tn_affine", "plan_query", "workspace_size", "Workspace",
           "GemmError"]


def _ld(t, inner):
    """Row stride of a 2-D (or trailing 2-D) operand; columns must be unit stride."""
    rows, cols = t.shape[-2], t.shape[-1]
    if cols > 1 and t.stride(-1) != 1:
        raise ValueError("operands must be row-major with unit column stride")
    ld = t.stride(-2)
    if rows <= 1 or ld < cols:
        ld = max(cols, 1) if rows <= 1 else ld
    return ld


# The raw handle of a device's current stream, without building a Stream
# object (a few microseconds per call otherwise, which is the whole kernel
# time of a small product).
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(idx):
    if _raw_stream is not None:
        return _raw_stream(idx)
    return torch.cuda.current_stream(idx).cuda_stream


def _check_dev(*ts):
    """Every tensor the kernels read or write (None entries skipped) must be a
    GPU tensor on one device; checked before anything is launched."""
    ts = [t for t in ts if t is not None]
    dev = ts[0].device
    if dev.type != "cuda":
        raise ValueError("operands must be GPU tensors")
    for t in ts[1:]:
        if t.device != dev:
            raise ValueError("every operand, output, scale, bias and workspace must be on one GPU")
    return dev


def _launch(fn, dev, *args):
    """Call `fn(*args, stream)` with `dev` current, on its current stream."""
    idx = dev.index if dev.index is not None else torch.cuda.current_device()
    if idx == torch.cuda.current_device():
        return fn(*args, _stream(idx))
    with torch.cuda.device(idx):
        return fn(*args, _stream(idx))


class Workspace:
    """Caller-owned scratch memory for the workspace paths of gemm_run.

    Device memory from torch (zero-filled when allocated: the first
    GEMM_WORKSPACE_COUNTER_BYTES hold arrival counters and exchange slots
    that every call leaves at zero).  ``reserve(n)``
    replaces the buffer with a larger one when a call needs more; the old
    one is released to torch's stream-ordered allocator.  One Workspace
    serves calls on one stream (calls that may overlap in time need separate
    workspaces)."""

    def __init__(self, device=None, nbytes=0):
        if device is None:
            device = torch.device("cuda", torch.cuda.current_device())
        self.device = torch.device(device)
        self.buf = None
        self._need = {}        # call shape -> bytes (the size query is host-only and deterministic)
        if nbytes:
            self.reserve(nbytes)

    def reserve(self, nbytes):
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=self.device)
        return self.buf


def workspace_size(op, batch, M, N, K, a_addr, lda, sA, b_addr, ldb, sB, c_addr, ldc, sC, c_type):
    """Host-only: bytes of workspace gemm_run needs for a call (0: none)."""
    n = ctypes.c_uint64(0)
    st = lib().gemm_workspace_size(op, batch, M, N, K, a_addr, lda, sA, b_addr, ldb, sB, c_addr, ldc, sC, c_type,
                                   ctypes.byref(n))
    if st != 0:
        raise GemmError(st, "gemm_workspace_size")
    return int(n.value)


def _gemm(what, named, named_args, workspace, dev, op, batch, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, code,
          alpha=1.0, bias=None, beta=0.0, scale_a=None, scale_b=None):
    """Run one call: the named entry point (`named`, its arguments
    `named_args`) without a workspace, else gemm_run with the workspace's
    memory."""
    if workspace is None:
        st = _launch(getattr(lib(), named), dev, *named_args)
    else:
        if isinstance(workspace, Workspace):
            if workspace.device != dev:
                raise ValueError("the workspace must be on the operands' GPU")
            pa, pb, pc = A.data_ptr(), B.data_ptr(), C.data_ptr()
            # the size depends on the pointers only through their alignment
            key = (op, batch, M, N, K, lda, sA, ldb, sB, ldc, sC, code, pa % 256, pb % 256, pc % 256)
            need = workspace._need.get(key)
            if need is None:
                need = workspace_size(op, batch, M, N, K, pa, lda, sA, pb, ldb, sB, pc, ldc, sC, code) if K > 0 else 0
                workspace._need[key] = need
            buf = workspace.reserve(need)
        else:
            buf = workspace
            if not isinstance(buf, torch.Tensor) or buf.dtype != torch.uint8 or buf.dim() != 1:
                raise ValueError("a workspace tensor must be a 1-D uint8 tensor")
            _check_dev(A, buf)
        def run(buf):
            return _launch(lib().gemm_run, dev, op, batch, M, N, K, A.data_ptr(), lda, sA, B.data_ptr(), ldb, sB,
                           C.data_ptr(), ldc, sC, code, float(alpha), None if bias is None else bias.data_ptr(),
                           float(beta), None if scale_a is None else scale_a.data_ptr(),
                           None if scale_b is None else scale_b.data_ptr(), buf.data_ptr(), buf.numel())
        st = run(buf)
        if st == GEMM_ERR_WORKSPACE and isinstance(workspace, Workspace):
            # The cached size went stale (the plan also follows the
            # library's environment overrides): a call refused for its
            # workspace has launched nothing, so ask again and retry once.
            need = workspace_size(op, batch, M, N, K, pa, lda, sA, pb, ldb, sB, pc, ldc, sC, code)
            workspace._need[key] = need
            st = run(workspace.reserve(need))
    if st != 0:
        raise GemmError(st, what)
    return C


def gemm_sgemm(A, B, C=None):
    """C[M,N] = A[M,K] . B[K,N] for float32 tensors (gemm_sgemm)."""
    if A.dtype != torch.float32 or B.dtype != torch.float32:
        raise TypeError("gemm_sgemm takes float32 operands")
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    dev = _check_dev(A, B, C)
    if C is None:
        C = torch.empty((M, N), dtype=torch.float32, device=dev)
    if C.shape != (M, N) or C.dtype != torch.float32:
        raise ValueError("C must be float32 [M, N]")
    st = _launch(lib().gemm_sgemm, dev, M, N, K, A.data_ptr(), _ld(A, K), B.data_ptr(), _ld(B, N),
                 C.data_ptr(), _ld(C, N))
    if st != 0:
        raise GemmError(st, "gemm_sgemm")
    return C


def _out_code(dtype):
    if dtype == torch.bfloat16:
        return _lib.GEMM_OUT_BF16
    if dtype == torch.float32:
        return _lib.GEMM_OUT_F32
    raise TypeError("output dtype must be bfloat16 or float32")


def _bstride(t):
    return t.stride(0) if t.shape[0] > 1 else 0


def gemm_bf16(A, B, C=None, out_dtype=torch.bfloat16, workspace=None):
    """C[M,N] = A[M,K] . B[K,N] for bfloat16 operands, FP32 accumulation,
    bf16 (round to nearest even) or float32 output (gemm_bf16)."""
    if A.dtype != torch.bfloat16 or B.dtype != torch.bfloat16:
        raise TypeError("gemm_bf16 takes bfloat16 operands")
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    dev = _check_dev(A, B, C)
    if C is None:
        C = torch.empty((M, N), dtype=out_dtype, device=dev)
    if C.shape != (M, N):
        raise ValueError("C must be [M, N]")
    code = _out_code(C.dtype)
    lda, ldb, ldc = _ld(A, K), _ld(B, N), _ld(C, N)
    return _gemm("gemm_bf16", "gemm_bf16",
                 (M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, C.data_ptr(), ldc, code), workspace, dev,
                 _lib.GEMM_OP_BF16, 1, M, N, K, A, lda, 0, B, ldb, 0, C, ldc, 0, code)


def gemm_bf16_batched(A, B, C=None, out_dtype=torch.bfloat16, workspace=None):
    """C[b] = A[b] . B[b] for bfloat16 stacks [batch, M, K] and [batch, K, N]
    (gemm_bf16_batched).  A batch stride of 0 (an expanded operand)
    broadcasts it."""
    if A.dtype != torch.bfloat16 or B.dtype != torch.bfloat16:
        raise TypeError("gemm_bf16_batched takes bfloat16 operands")
    batch, M, K = A.shape
    b2, K2, N = B.shape
    if batch != b2 or K != K2:
        raise ValueError("shape mismatch")
    dev = _check_dev(A, B, C)
    if C is None:
        C = torch.empty((batch, M, N), dtype=out_dtype, device=dev)
    if tuple(C.shape) != (batch, M, N):
        raise ValueError("C must be [batch, M, N]")
    code = _out_code(C.dtype)
    lda, ldb, ldc = _ld(A, K), _ld(B, N), _ld(C, N)
    sA, sB, sC = _bstride(A), _bstride(B), _bstride(C)
    return _gemm("gemm_bf16_batched", "gemm_bf16_batched",
                 (batch, M, N, K, A.data_ptr(), lda, sA, B.data_ptr(), ldb, sB, C.data_ptr(), ldc, sC, code),
                 workspace, dev, _lib.GEMM_OP_BF16, batch, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, code)


def gemm_bf16_nt(A, Bt, C=None, out_dtype=torch.bfloat16, workspace=None):
    """C[M,N] = A[M,K] . Bt[N,K]^T for bfloat16 operands (gemm_bf16_nt): B
    given transposed, as a linear layer's weight or attention's keys."""
    if A.dtype != torch.bfloat16 or Bt.dtype != torch.bfloat16:
        raise TypeError("gemm_bf16_nt takes bfloat16 operands")
    M, K = A.shape
    N, K2 = Bt.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    dev = _check_dev(A, Bt, C)
    if C is None:
        C = torch.empty((M, N), dtype=out_dtype, device=dev)
    if C.shape != (M, N):
        raise ValueError("C must be [M, N]")
    code = _out_code(C.dtype)
    lda, ldb, ldc = _ld(A, K), _ld(Bt, K), _ld(C, N)
    return _gemm("gemm_bf16_nt", "gemm_bf16_nt",
                 (M, N, K, A.data_ptr(), lda, Bt.data_ptr(), ldb, C.data_ptr(), ldc, code), workspace, dev,
                 _lib.GEMM_OP_BF16_NT, 1, M, N, K, A, lda, 0, Bt, ldb, 0, C, ldc, 0, code)


def gemm_bf16_nt_batched(A, Bt, C=None, out_dtype=torch.bfloat16, workspace=None):
    """C[b] = A[b] . Bt[b]^T for bfloat16 stacks [batch, M, K] and [batch, N, K]
    (gemm_bf16_nt_batched), e.g. attention scores Q . K^T; a batch stride of
    0 broadcasts an operand."""
    if A.dtype != torch.bfloat16 or Bt.dtype != torch.bfloat16:
        raise TypeError("gemm_bf16_nt_batched takes bfloat16 operands")
    batch, M, K = A.shape
    b2, N, K2 = Bt.shape
    if batch != b2 or K != K2:
        raise ValueError("shape mismatch")
    dev = _check_dev(A, Bt, C)
    if C is None:
        C = torch.empty((batch, M, N), dtype=out_dtype, device=dev)
    if tuple(C.shape) != (batch, M, N):
        raise ValueError("C must be [batch, M, N]")
    code = _out_code(C.dtype)
    lda, ldb, ldc = _ld(A, K), _ld(Bt, K), _ld(C, N)
    sA, sB, sC = _bstride(A), _bstride(Bt), _bstride(C)
    return _gemm("gemm_bf16_nt_batched", "gemm_bf16_nt_batched",
                 (batch, M, N, K, A.data_ptr(), lda, sA, Bt.data_ptr(), ldb, sB, C.data_ptr(), ldc, sC, code),
                 workspace, dev, _lib.GEMM_OP_BF16_NT, batch, M, N, K, A, lda, sA, Bt, ldb, sB, C, ldc, sC, code)


def gemm_bf16_tn(At, B, C=None, out_dtype=torch.bfloat16, workspace=None):
    """C[M,N] = At[K,M]^T . B[K,N] for bfloat16 operands (gemm_bf16_tn): A
    given transposed, e.g. the activations of a weight gradient X^T . dY."""
    if At.dtype != torch.bfloat16 or B.dtype != torch.bfloat16:
        raise TypeError("gemm_bf16_tn takes bfloat16 operands")
    K, M = At.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    dev = _check_dev(At, B, C)
    if C is None:
        C = torch.empty((M, N), dtype=out_dtype, device=dev)
    if C.shape != (M, N):
        raise ValueError("C must be [M, N]")
    code = _out_code(C.dtype)
    lda, ldb, ldc = _ld(At, M), _ld(B, N), _ld(C, N)
    return _gemm("gemm_bf16_tn", "gemm_bf16_tn",
                 (M, N, K, At.data_ptr(), lda, B.data_ptr(), ldb, C.data_ptr(), ldc, code), workspace, dev,
                 _lib.GEMM_OP_BF16_TN, 1, M, N, K, At, lda, 0, B, ldb, 0, C, ldc, 0, code)


def gemm_bf16_tn_batched(At, B, C=None, out_dtype=torch.bfloat16, workspace=None):
    """C[b] = At[b]^T . B[b] for bfloat16 stacks [batch, K, M] and [batch, K, N]
    (gemm_bf16_tn_batched); a batch stride of 0 broadcasts an operand."""
    if At.dtype != torch.bfloat16 or B.dtype != torch.bfloat16:
        raise TypeError("gemm_bf16_tn_batched takes bfloat16 operands")
    batch, K, M = At.shape
    b2, K2, N = B.shape
    if batch != b2 or K != K2:
        raise ValueError("shape mismatch")
    dev = _check_dev(At, B, C)
    if C is None:
        C = torch.empty((batch, M, N), dtype=out_dtype, device=dev)
    if tuple(C.shape) != (batch, M, N):
        raise ValueError("C must be [batch, M, N]")
    code = _out_code(C.dtype)
    lda, ldb, ldc = _ld(At, M), _ld(B, N), _ld(C, N)
    sA, sB, sC = _bstride(At), _bstride(B), _bstride(C)
    return _gemm("gemm_bf16_tn_batched", "gemm_bf16_tn_batched",
                 (batch, M, N, K, At.data_ptr(), lda, sA, B.data_ptr(), ldb, sB, C.data_ptr(), ldc, sC, code),
                 workspace, dev, _lib.GEMM_OP_BF16_TN, batch, M, N, K, At, lda, sA, B, ldb, sB, C, ldc, sC, code)


def _codes(t):
    """E4M3FN codes: a uint8 tensor or a float8_e4m3fn tensor viewed as bytes."""
    if t.dtype == torch.uint8:
        return t
    if str(t.dtype) == "torch.float8_e4m3fn":
        return t.view(torch.uint8)
    raise TypeError("fp8 operands are uint8 codes or float8_e4m3fn tensors")


def gemm_fp8_quantize_rows(X, Q=None, scale=None):
    """Per-row E4M3FN quantization of a bfloat16 [rows, cols] tensor
    (gemm_fp8_quantize_rows): returns (codes uint8 [rows, cols], float32
    dequantization factors [rows])."""
    if X.dtype != torch.bfloat16 or X.dim() != 2:
        raise TypeError("gemm_fp8_quantize_rows takes a 2-D bfloat16 tensor")
    rows, cols = X.shape
    dev = _check_dev(X, Q, scale)
    if Q is None:
        Q = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
    if scale is None:
        scale = torch.empty((rows,), dtype=torch.float32, device=dev)
    Q = _codes(Q)
    if tuple(Q.shape) != (rows, cols) or tuple(scale.shape) != (rows,) or scale.dtype != torch.float32:
        raise ValueError("Q must be [rows, cols] codes and scale float32 [rows]")
    if rows > 1 and scale.stride(0) != 1:
        raise ValueError("scale must be contiguous")
    st = _launch(lib().gemm_fp8_quantize_rows, dev, rows, cols, X.data_ptr(), _ld(X, cols), Q.data_ptr(),
                 _ld(Q, cols), scale.data_ptr())
    if st != 0:
        raise GemmError(st, "gemm_fp8_quantize_rows")
    return Q, scale


def gemm_fp8_quantize_cols(W, Qt=None, scale=None):
    """Per-column E4M3FN quantization of a bfloat16 weight W [K, N] stored as
    [in, out] (gemm_fp8_quantize_cols): returns (codes uint8 Qt [N, K], the
    Bt operand of the FP8 products, and float32 factors [N])."""
    if W.dtype != torch.bfloat16 or W.dim() != 2:
        raise TypeError("gemm_fp8_quantize_cols takes a 2-D bfloat16 tensor")
    K, N = W.shape
    dev = _check_dev(W, Qt, scale)
    if Qt is None:
        Qt = torch.empty((N, K), dtype=torch.uint8, device=dev)
    if scale is None:
        scale = torch.empty((N,), dtype=torch.float32, device=dev)
    Qt = _codes(Qt)
    if tuple(Qt.shape) != (N, K) or tuple(scale.shape) != (N,) or scale.dtype != torch.float32:
        raise ValueError("Qt must be [N, K] codes and scale float32 [N]")
    if N > 1 and scale.stride(0) != 1:
        raise ValueError("scale must be contiguous")
    st = _launch(lib().gemm_fp8_quantize_cols, dev, K, N, W.data_ptr(), _ld(W, N), Qt.data_ptr(), _ld(Qt, K),
                 scale.data_ptr())
    if st != 0:
        raise GemmError(st, "gemm_fp8_quantize_cols")
    return Qt, scale


def _fp8_scale(sc, shared, batch, n, what):
    """A factor vector: [n] for an operand shared by the batch entries (or a
    single product), else [batch, n], contiguous float32."""
    if sc is None:
        return None
    want = (n,) if shared else (batch, n)
    if sc.dtype != torch.float32 or (tuple(sc.shape) != want and not (shared and tuple(sc.shape) == (1, n))):
        raise ValueError(f"{what} must be float32 {list(want)}")
    if sc.numel() > 1 and not sc.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return sc


def _fp8(A, scale_a, Bt, scale_b, C, out_dtype, workspace, affine=None):
    """The FP8 products: 2-D operands, or stacks [batch, M, K] / [batch, N, K]
    (stride 0 along the batch broadcasts an operand, and its factors)."""
    A, Bt = _codes(A), _codes(Bt)
    if A.dim() != Bt.dim() or A.dim() not in (2, 3):
        raise ValueError("A and Bt must both be 2-D or both be 3-D")
    three = A.dim() == 3
    A3, B3 = (A, Bt) if three else (A.unsqueeze(0), Bt.unsqueeze(0))
    batch, M, K = A3.shape
    b2, N, K2 = B3.shape
    if batch != b2 or K != K2:
        raise ValueError(f"shape mismatch: A {tuple(A.shape)}, Bt {tuple(Bt.shape)}")
    dev = _check_dev(A, Bt, C, scale_a, scale_b, None if affine is None else affine[1])
    sA, sB = _bstride(A3), _bstride(B3)
    scale_a = _fp8_scale(scale_a, batch == 1 or sA == 0, batch, M, "scale_a")
    scale_b = _fp8_scale(scale_b, batch == 1 or sB == 0, batch, N, "scale_b")
    if C is None:
        if affine is not None:
            raise ValueError("the affine FP8 product updates a given C")
        C = torch.empty((batch, M, N) if three else (M, N), dtype=out_dtype, device=dev)
    C3 = C if three else C.unsqueeze(0)
    if tuple(C3.shape) != (batch, M, N):
        raise ValueError("C must be [M, N] (or [batch, M, N])")
    code = _out_code(C.dtype)
    lda, ldb, ldc = _ld(A3, K), _ld(B3, K), _ld(C3, N)
    sC = _bstride(C3)
    pa = None if scale_a is None else scale_a.data_ptr()
    pb = None if scale_b is None else scale_b.data_ptr()
    if affine is None:
        if three:
            named, args = "gemm_fp8_nt_batched", (batch, M, N, K, A3.data_ptr(), lda, sA, pa, B3.data_ptr(), ldb, sB,
                                                  pb, C3.data_ptr(), ldc, sC, code)
        else:
            named, args = "gemm_fp8_nt", (M, N, K, A.data_ptr(), lda, pa, Bt.data_ptr(), ldb, pb, C.data_ptr(), ldc,
                                          code)
        _gemm(named, named, args, workspace, dev, _lib.GEMM_OP_FP8_NT, batch, M, N, K, A3, lda, sA, B3, ldb, sB,
              C3, ldc, sC, code, scale_a=scale_a, scale_b=scale_b)
        return C
    alpha, bias, beta = affine
    if bias is not None and (bias.dtype != torch.bfloat16 or tuple(bias.shape) != (N,) or
                             (N > 1 and bias.stride(0) != 1)):
        raise ValueError("bias must be a contiguous bfloat16 vector of N elements")
    bp = None if bias is None else bias.data_ptr()
    _gemm("gemm_fp8_nt_affine", "gemm_fp8_nt_affine",
          (batch, M, N, K, A3.data_ptr(), lda, sA, pa, B3.data_ptr(), ldb, sB, pb, float(alpha), bp, float(beta),
           C3.data_ptr(), ldc, sC, code),
          workspace, dev, _lib.GEMM_OP_FP8_NT_AFFINE, batch, M, N, K, A3, lda, sA, B3, ldb, sB, C3, ldc, sC, code,
          alpha=alpha, bias=bias, beta=beta, scale_a=scale_a, scale_b=scale_b)
    return C


def gemm_fp8_nt(A, scale_a, Bt, scale_b, C=None, out_dtype=torch.bfloat16, workspace=None):
    """C[M,N] = (dec(A) . dec(Bt)^T) * scale_a[:, None] * scale_b[None, :] for
    E4M3FN codes A [M,K] and Bt [N,K] (gemm_fp8_nt); a scale may be None.
    Stacks A [batch, M, K], Bt [batch, N, K] (gemm_fp8_nt_batched) take
    factors [batch, M] / [batch, N], or [M] / [N] for an operand broadcast
    along the batch (stride 0)."""
    return _fp8(A, scale_a, Bt, scale_b, C, out_dtype, workspace)


def gemm_fp8_nt_quant_a(X, Bt, scale_b, C=None, scale_x=None, out_dtype=torch.bfloat16, workspace=None):
    """The FP8 product with X [M, K] (bfloat16) quantized inside the GEMM
    (gemm_fp8_nt_quant_a): returns (C [M, N], scale_x float32 [M], X's row
    factors).  Bt [N, K] codes with factors scale_b [N] (or None).  The
    workspace (a Workspace or a uint8 tensor) holds M floats after its first
    GEMM_WORKSPACE_COUNTER_BYTES (the counter region of gemm_run calls,
    left untouched); a
    Workspace is created for the call when None is given."""
    if X.dtype != torch.bfloat16 or X.dim() != 2:
        raise TypeError("gemm_fp8_nt_quant_a takes a 2-D bfloat16 X")
    Bt = _codes(Bt)
    M, K = X.shape
    N, K2 = Bt.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    dev = _check_dev(X, Bt, C, scale_b, scale_x)
    if scale_b is not None and (scale_b.dtype != torch.float32 or tuple(scale_b.shape) != (N,) or
                                (N > 1 and scale_b.stride(0) != 1)):
        raise ValueError(f"scale_b must be a contiguous float32 vector of {N}")
    if scale_x is None:
        scale_x = torch.empty((M,), dtype=torch.float32, device=dev)
    if scale_x.dtype != torch.float32 or tuple(scale_x.shape) != (M,) or (M > 1 and scale_x.stride(0) != 1):
        raise ValueError(f"scale_x must be a contiguous float32 vector of {M}")
    if C is None:
        C = torch.empty((M, N), dtype=out_dtype, device=dev)
    if C.shape != (M, N):
        raise ValueError("C must be [M, N]")
    if workspace is None:
        workspace = Workspace(dev)
    if isinstance(workspace, Workspace):
        if workspace.device != dev:
            raise ValueError("the workspace must be on the operands' GPU")
        buf = workspace.reserve(GEMM_WORKSPACE_COUNTER_BYTES + 4 * M)
    else:
        buf = workspace
        if not isinstance(buf, torch.Tensor) or buf.dtype != torch.uint8 or buf.dim() != 1:
            raise ValueError("a workspace tensor must be a 1-D uint8 tensor")
        _check_dev(X, buf)
    code = _out_code(C.dtype)
    st = _launch(lib().gemm_fp8_nt_quant_a, dev, M, N, K, X.data_ptr(), _ld(X, K), scale_x.data_ptr(), Bt.data_ptr(),
                 _ld(Bt, K), None if scale_b is None else scale_b.data_ptr(), C.data_ptr(), _ld(C, N), code,
                 buf.data_ptr(), buf.numel())
    if st != 0:
        raise GemmError(st, "gemm_fp8_nt_quant_a")
    return C, scale_x


def gemm_fp8_nt_affine(A, scale_a, Bt, scale_b, C, alpha=1.0, bias=None, beta=0.0, workspace=None):
    """C := alpha * (dec(A) . dec(Bt)^T * scale_a * scale_b) + bias + beta * C
    in place (gemm_fp8_nt_affine), 2-D or batched as gemm_fp8_nt; C bfloat16
    or float32 (read when beta != 0), bias a bfloat16 vector of N or None.
    Returns C."""
    return _fp8(A, scale_a, Bt, scale_b, C, C.dtype, workspace, affine=(alpha, bias, beta))


def gemm_bf16_silu(A, B, C=None, workspace=None):
    """C[M,N] = bf16(SiLU(bf16(A . B))) for bfloat16 operands (gemm_bf16_silu)."""
    if A.dtype != torch.bfloat16 or B.dtype != torch.bfloat16:
        raise TypeError("gemm_bf16_silu takes bfloat16 operands")
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    dev = _check_dev(A, B, C)
    if C is None:
        C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    if C.shape != (M, N) or C.dtype != torch.bfloat16:
        raise ValueError("C must be bfloat16 [M, N]")
    lda, ldb, ldc = _ld(A, K), _ld(B, N), _ld(C, N)
    return _gemm("gemm_bf16_silu", "gemm_bf16_silu",
                 (M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, C.data_ptr(), ldc), workspace, dev,
                 _lib.GEMM_OP_BF16_SILU, 1, M, N, K, A, lda, 0, B, ldb, 0, C, ldc, 0, _lib.GEMM_OUT_BF16)


def gemm_bf16_swiglu(X, Wgu, Z=None, workspace=None):
    """Z[M,N] = bf16(bf16(SiLU(bf16(X . W_g))) * bf16(X . W_u)) for a merged
    bfloat16 weight Wgu[K, 2N] = [W_g | W_u] (gemm_bf16_swiglu)."""
    if X.dtype != torch.bfloat16 or Wgu.dtype != torch.bfloat16:
        raise TypeError("gemm_bf16_swiglu takes bfloat16 operands")
    M, K = X.shape
    K2, N2 = Wgu.shape
    if K != K2 or N2 % 2:
        raise ValueError("expected X [M, K] and Wgu [K, 2N]")
    N = N2 // 2
    dev = _check_dev(X, Wgu, Z)
    if Z is None:
        Z = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    if Z.shape != (M, N) or Z.dtype != torch.bfloat16:
        raise ValueError("Z must be bfloat16 [M, N]")
    ldx, ldw, ldz = _ld(X, K), _ld(Wgu, N2), _ld(Z, N)
    return _gemm("gemm_bf16_swiglu", "gemm_bf16_swiglu",
                 (M, N, K, X.data_ptr(), ldx, Wgu.data_ptr(), ldw, Z.data_ptr(), ldz), workspace, dev,
                 _lib.GEMM_OP_BF16_SWIGLU, 1, M, N, K, X, ldx, 0, Wgu, ldw, 0, Z, ldz, 0, _lib.GEMM_OUT_BF16)


def gemm_bf16_silu_batched(A, B, C=None, workspace=None):
    """C[b] = bf16(SiLU(bf16(A[b] . B[b]))) for bfloat16 stacks [batch, M, K]
    and [batch, K, N] (gemm_bf16_silu_batched); a batch stride of 0
    broadcasts an operand."""
    if A.dtype != torch.bfloat16 or B.dtype != torch.bfloat16:
        raise TypeError("gemm_bf16_silu_batched takes bfloat16 operands")
    batch, M, K = A.shape
    b2, K2, N = B.shape
    if batch != b2 or K != K2:
        raise ValueError("shape mismatch")
    dev = _check_dev(A, B, C)
    if C is None:
        C = torch.empty((batch, M, N), dtype=torch.bfloat16, device=dev)
    if tuple(C.shape) != (batch, M, N) or C.dtype != torch.bfloat16:
        raise ValueError("C must be bfloat16 [batch, M, N]")
    lda, ldb, ldc = _ld(A, K), _ld(B, N), _ld(C, N)
    sA, sB, sC = _bstride(A), _bstride(B), _bstride(C)
    return _gemm("gemm_bf16_silu_batched", "gemm_bf16_silu_batched",
                 (batch, M, N, K, A.data_ptr(), lda, sA, B.data_ptr(), ldb, sB, C.data_ptr(), ldc, sC), workspace,
                 dev, _lib.GEMM_OP_BF16_SILU, batch, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, _lib.GEMM_OUT_BF16)


def gemm_bf16_swiglu_batched(X, Wgu, Z=None, workspace=None):
    """Z[b] = SwiGLU of X[b] with the merged gate|up weight Wgu[b] [K, 2N]
    (gemm_bf16_swiglu_batched), e.g. the experts of a mixture-of-experts FFN;
    a batch stride of 0 broadcasts an operand."""
    if X.dtype != torch.bfloat16 or Wgu.dtype != torch.bfloat16:
        raise TypeError("gemm_bf16_swiglu_batched takes bfloat16 operands")
    batch, M, K = X.shape
    b2, K2, N2 = Wgu.shape
    if batch != b2 or K != K2 or N2 % 2:
        raise ValueError("expected X [batch, M, K] and Wgu [batch, K, 2N]")
    N = N2 // 2
    dev = _check_dev(X, Wgu, Z)
    if Z is None:
        Z = torch.empty((batch, M, N), dtype=torch.bfloat16, device=dev)
    if tuple(Z.shape) != (batch, M, N) or Z.dtype != torch.bfloat16:
        raise ValueError("Z must be bfloat16 [batch, M, N]")
    ldx, ldw, ldz = _ld(X, K), _ld(Wgu, N2), _ld(Z, N)
    sA, sB, sC = _bstride(X), _bstride(Wgu), _bstride(Z)
    return _gemm("gemm_bf16_swiglu_batched", "gemm_bf16_swiglu_batched",
                 (batch, M, N, K, X.data_ptr(), ldx, sA, Wgu.data_ptr(), ldw, sB, Z.data_ptr(), ldz, sC), workspace,
                 dev, _lib.GEMM_OP_BF16_SWIGLU, batch, M, N, K, X, ldx, sA, Wgu, ldw, sB, Z, ldz, sC,
                 _lib.GEMM_OUT_BF16)


def _swiglu_e4m3_shapes(X, Wgu, Zq, what, batched):
    if X.dtype != torch.bfloat16 or Wgu.dtype != torch.bfloat16:
        raise TypeError(f"{what} takes bfloat16 operands")
    if batched:
        batch, M, K = X.shape
        b2, K2, N2 = Wgu.shape
        ok = batch == b2 and K == K2 and N2 % 2 == 0
    else:
        (M, K), (K2, N2), batch = X.shape, Wgu.shape, None
        ok = K == K2 and N2 % 2 == 0
    if not ok:
        raise ValueError(f"{what}: expected X [..., M, K] and Wgu [..., K, 2N]")
    N = N2 // 2
    dev = _check_dev(X, Wgu, Zq)
    shape = (M, N) if batch is None else (batch, M, N)
    if Zq is None:
        Zq = torch.empty(shape, dtype=torch.uint8, device=dev)
    if tuple(Zq.shape) != shape or Zq.dtype != torch.uint8:
        raise ValueError(f"{what}: Zq must be uint8 {list(shape)}")
    return batch, M, N, K, N2, dev, Zq


def gemm_bf16_swiglu_e4m3(X, Wgu, amax, Zq=None, workspace=None):
    """SwiGLU of X [M, K] with the merged weight Wgu [K, 2N], stored as
    E4M3FN codes (uint8 [M, N]) against the fixed range amax: the code
    nearest to z * 448 / amax for the bf16 output z, saturating at 448
    (gemm_bf16_swiglu_e4m3).
    The codes dequantize by amax / 448 (``Zq.view(torch.float8_e4m3fn)``
    reads them as float8)."""
    _, M, N, K, N2, dev, Zq = _swiglu_e4m3_shapes(X, Wgu, Zq, "gemm_bf16_swiglu_e4m3", False)
    ldx, ldw, ldz = _ld(X, K), _ld(Wgu, N2), _ld(Zq, N)
    amax = float(amax)
    return _gemm("gemm_bf16_swiglu_e4m3", "gemm_bf16_swiglu_e4m3",
                 (M, N, K, X.data_ptr(), ldx, Wgu.data_ptr(), ldw, Zq.data_ptr(), ldz, amax), workspace, dev,
                 _lib.GEMM_OP_BF16_SWIGLU, 1, M, N, K, X, ldx, 0, Wgu, ldw, 0, Zq, ldz, 0, _lib.GEMM_OUT_E4M3,
                 alpha=amax)


def gemm_bf16_swiglu_e4m3_batched(X, Wgu, amax, Zq=None, workspace=None):
    """The batched form of gemm_bf16_swiglu_e4m3: X [batch, M, K], Wgu
    [batch, K, 2N], codes uint8 [batch, M, N], one range for every entry; a
    batch stride of 0 broadcasts an operand."""
    batch, M, N, K, N2, dev, Zq = _swiglu_e4m3_shapes(X, Wgu, Zq, "gemm_bf16_swiglu_e4m3_batched", True)
    ldx, ldw, ldz = _ld(X, K), _ld(Wgu, N2), _ld(Zq, N)
    sA, sB, sC = _bstride(X), _bstride(Wgu), _bstride(Zq)
    amax = float(amax)
    return _gemm("gemm_bf16_swiglu_e4m3_batched", "gemm_bf16_swiglu_e4m3_batched",
                 (batch, M, N, K, X.data_ptr(), ldx, sA, Wgu.data_ptr(), ldw, sB, Zq.data_ptr(), ldz, sC, amax),
                 workspace, dev, _lib.GEMM_OP_BF16_SWIGLU, batch, M, N, K, X, ldx, sA, Wgu, ldw, sB, Zq, ldz, sC,
                 _lib.GEMM_OUT_E4M3, alpha=amax)


def act_chain(step, in0, in1=None, out=None, amax=None):
    """One step of the activation chain on stored bf16 tensors [M, N]
    (gemm_act_chain; step one of GEMM_ACT_*): SiLU, the product, SwiGLU, the
    fixed-range E4M3FN quantization, or SwiGLU and the quantization fused.
    Returns `out` (bfloat16, or uint8 codes for the quantizing steps)."""
    two = step in (_lib.GEMM_ACT_MUL, _lib.GEMM_ACT_SWIGLU, _lib.GEMM_ACT_SWIGLU_E4M3)
    codes = step in (_lib.GEMM_ACT_QUANT, _lib.GEMM_ACT_SWIGLU_E4M3)
    if step not in range(5):
        raise ValueError("unknown activation-chain step")
    if in0.dtype != torch.bfloat16 or in0.dim() != 2 or (two and (in1 is None or in1.dtype != torch.bfloat16)):
        raise TypeError("the activation chain takes bfloat16 [M, N] inputs")
    if two and tuple(in1.shape) != tuple(in0.shape):
        raise ValueError("in0 and in1 differ in shape")
    if codes and amax is None:
        raise ValueError("the quantizing steps take a range amax")
    M, N = in0.shape
    dev = _check_dev(in0, in1 if two else None, out)
    odt = torch.uint8 if codes else torch.bfloat16
    if out is None:
        out = torch.empty((M, N), dtype=odt, device=dev)
    if tuple(out.shape) != (M, N) or out.dtype != odt:
        raise ValueError(f"out must be {odt} [M, N]")
    st = _launch(lib().gemm_act_chain, dev, step, M, N, in0.data_ptr(), _ld(in0, N),
                 in1.data_ptr() if two else None, _ld(in1, N) if two else N, out.data_ptr(), _ld(out, N),
                 float(amax) if codes else 1.0)
    if st != 0:
        raise GemmError(st, "gemm_act_chain")
    return out


def act_silu(G, out=None):
    """T = bf16(SiLU(G)) element by element (the chain's first step)."""
    return act_chain(_lib.GEMM_ACT_SILU, G, None, out)


def act_mul(T, U, out=None):
    """Z = bf16(T * U) element by element (the chain's second step)."""
    return act_chain(_lib.GEMM_ACT_MUL, T, U, out)


def act_swiglu(G, U, out=None):
    """Z = bf16(bf16(SiLU(G)) * U), the first two steps fused."""
    return act_chain(_lib.GEMM_ACT_SWIGLU, G, U, out)


def act_quantize_e4m3(Z, amax, out=None):
    """E4M3FN codes of bf16 Z against the fixed range amax (the third step)."""
    return act_chain(_lib.GEMM_ACT_QUANT, Z, None, out, amax)


def act_swiglu_e4m3(G, U, amax, out=None):
    """The codes of bf16(bf16(SiLU(G)) * U), all three steps fused."""
    return act_chain(_lib.GEMM_ACT_SWIGLU_E4M3, G, U, out, amax)


def gemm_bf16_affine(A, B, C, alpha=1.0, bias=None, beta=0.0, workspace=None):
    """C := alpha * (A . B) + bias + beta * C in place (gemm_bf16_affine):
    bfloat16 A [M,K] / B [K,N] or stacks [batch, M, K] / [batch, K, N], C of
    the matching shape in bfloat16 or float32 (read when beta != 0), bias a
    bfloat16 vector of N elements or None.  Returns C."""
    return _affine(A, B, C, alpha, bias, beta, False, workspace=workspace)


def gemm_bf16_nt_affine(A, Bt, C, alpha=1.0, bias=None, beta=0.0, workspace=None):
    """C := alpha * (A . Bt^T) + bias + beta * C in place
    (gemm_bf16_nt_affine): Bt [N,K] (or [batch, N, K]) is a linear layer's
    [out, in] weight; otherwise as gemm_bf16_affine."""
    return _affine(A, Bt, C, alpha, bias, beta, True, workspace=workspace)


def gemm_bf16_tn_affine(At, B, C, alpha=1.0, bias=None, beta=0.0, workspace=None):
    """C := alpha * (At^T . B) + bias + beta * C in place
    (gemm_bf16_tn_affine): At [K,M] (or [batch, K, M]), e.g. the activations
    of a weight gradient accumulated with beta = 1; otherwise as
    gemm_bf16_affine."""
    return _affine(At, B, C, alpha, bias, beta, False, a_trans=True, workspace=workspace)


def _affine(A, B, C, alpha, bias, beta, b_trans, a_trans=False, workspace=None):
    what = "gemm_bf16_nt_affine" if b_trans else "gemm_bf16_tn_affine" if a_trans else "gemm_bf16_affine"
    if A.dtype != torch.bfloat16 or B.dtype != torch.bfloat16:
        raise TypeError(f"{what} takes bfloat16 operands")
    if A.dim() != B.dim() or A.dim() not in (2, 3):
        raise ValueError("A and B must both be 2-D or both be 3-D")
    A3, B3, C3 = (A, B, C) if A.dim() == 3 else (A.unsqueeze(0), B.unsqueeze(0), C.unsqueeze(0))
    if a_trans:
        batch, K, M = A3.shape
    else:
        batch, M, K = A3.shape
    if b_trans:
        b2, N, K2 = B3.shape
    else:
        b2, K2, N = B3.shape
    if batch != b2 or K != K2 or tuple(C3.shape) != (batch, M, N):
        raise ValueError("shape mismatch")
    dev = _check_dev(A, B, C, bias)
    if bias is not None and (bias.dtype != torch.bfloat16 or tuple(bias.shape) != (N,) or
                             (N > 1 and bias.stride(0) != 1)):
        raise ValueError("bias must be a contiguous bfloat16 vector of N elements")
    code = _out_code(C.dtype)
    op = (_lib.GEMM_OP_BF16_NT_AFFINE if b_trans else _lib.GEMM_OP_BF16_TN_AFFINE if a_trans
          else _lib.GEMM_OP_BF16_AFFINE)
    fn = "gemm_bf16_nt_affine" if b_trans else "gemm_bf16_tn_affine" if a_trans else "gemm_bf16_affine"
    lda, ldb, ldc = _ld(A3, M if a_trans else K), _ld(B3, K if b_trans else N), _ld(C3, N)
    sA, sB, sC = _bstride(A3), _bstride(B3), _bstride(C3)
    bp = None if bias is None else bias.data_ptr()
    _gemm(what, fn, (batch, M, N, K, A3.data_ptr(), lda, sA, B3.data_ptr(), ldb, sB, float(alpha), bp, float(beta),
                     C3.data_ptr(), ldc, sC, code),
          workspace, dev, op, batch, M, N, K, A3, lda, sA, B3, ldb, sB, C3, ldc, sC, code,
          alpha=alpha, bias=bias, beta=beta)
    return C


def _plan_args(op, M, N, K, batch, lda, ldb, ldc, sA, sB, sC):
    tn = op in (_lib.GEMM_OP_BF16_TN, _lib.GEMM_OP_BF16_TN_AFFINE)
    lda = (M if tn else K) if lda is None else lda
    nt = op in (_lib.GEMM_OP_BF16_NT, _lib.GEMM_OP_FP8_NT, _lib.GEMM_OP_BF16_NT_AFFINE, _lib.GEMM_OP_FP8_NT_AFFINE)
    ldb = (2 * N if op == _lib.GEMM_OP_BF16_SWIGLU else K if nt else N) if ldb is None else ldb
    ldc = N if ldc is None else ldc
    sA = (K if tn else M) * lda if sA is None else sA
    sB = (N if nt else K) * ldb if sB is None else sB
    sC = M * ldc if sC is None else sC
    return lda, ldb, ldc, sA, sB, sC


def plan_query(op, M, N, K, batch=1, lda=None, ldb=None, ldc=None, a_addr=0x10000, b_addr=0x20000000,
               c_addr=0x40000000, sA=None, sB=None, sC=None, c_type=_lib.GEMM_OUT_BF16, with_workspace=True):
    """Host-only: the status and plan a call would produce (no GPU work):
    through gemm_run with a workspace (default) or without one (the named
    entry points)."""
    lda, ldb, ldc, sA, sB, sC = _plan_args(op, M, N, K, batch, lda, ldb, ldc, sA, sB, sC)
    out = GemmPlan()
    st = lib().gemm_plan_query_ex(1 if with_workspace else 0, op, batch, M, N, K, a_addr, lda, sA, b_addr, ldb, sB,
                                  c_addr, ldc, sC, c_type, ctypes.byref(out))
    return st, out
