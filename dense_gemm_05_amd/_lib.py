"""Loads libgemm05.so and declares the C signatures of include/gemm05.h.

There is no fallback: if the library is missing or does not load, every
entry point raises.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgemm05.so")

GEMM_OK = 0
GEMM_ERR_INVALID_ARG = -1
GEMM_ERR_UNSUPPORTED = -2
GEMM_ERR_LAUNCH = -3
GEMM_ERR_NO_DEVICE = -4
GEMM_ERR_WORKSPACE = -5

# GEMM_WORKSPACE_COUNTER_BYTES: the zeroed counter region at the start of a workspace
GEMM_WORKSPACE_COUNTER_BYTES = 1 << 20

GEMM_OUT_BF16 = 0
GEMM_OUT_F32 = 1
GEMM_OUT_E4M3 = 2
GEMM_ACT_SILU, GEMM_ACT_MUL, GEMM_ACT_SWIGLU, GEMM_ACT_QUANT, GEMM_ACT_SWIGLU_E4M3 = range(5)

GEMM_OP_SGEMM = 0
GEMM_OP_BF16 = 1
GEMM_OP_BF16_SILU = 2
GEMM_OP_BF16_SWIGLU = 3
GEMM_OP_BF16_NT = 4
GEMM_OP_FP8_NT = 5
GEMM_OP_BF16_AFFINE = 6
GEMM_OP_BF16_TN = 7
GEMM_OP_BF16_NT_AFFINE = 8
GEMM_OP_BF16_TN_AFFINE = 9
GEMM_OP_FP8_NT_AFFINE = 10

GEMM_FAMILY = {0: "none", 1: "zero", 2: "bf16_mfma", 3: "f32_mfma", 4: "decode", 5: "generic"}

# Every symbol declared by include/gemm05.h.
EXPORTS = ("gemm_sgemm", "gemm_bf16", "gemm_bf16_batched", "gemm_bf16_nt", "gemm_bf16_nt_batched",
           "gemm_bf16_tn", "gemm_bf16_tn_batched",
           "gemm_bf16_silu", "gemm_bf16_swiglu", "gemm_bf16_silu_batched", "gemm_bf16_swiglu_batched",
           "gemm_bf16_swiglu_e4m3", "gemm_bf16_swiglu_e4m3_batched", "gemm_act_chain",
           "gemm_fp8_quantize_rows", "gemm_fp8_quantize_cols", "gemm_fp8_nt", "gemm_fp8_nt_batched",
           "gemm_fp8_nt_affine", "gemm_fp8_nt_quant_a", "gemm_bf16_affine", "gemm_bf16_nt_affine",
           "gemm_bf16_tn_affine", "gemm_run", "gemm_run_noalloc", "gemm_workspace_size",
           "gemm_status_string",
           "gemm_plan_query", "gemm_plan_query_ex", "gemm_model_local_bytes", "gemm_model_traffic_bytes", "gemm_model_quant_traffic", "gemm_model_act_chain_bytes",
           "gemm_tile_map")


class GemmPlan(ctypes.Structure):
    _fields_ = [("family", ctypes.c_int), ("config_id", ctypes.c_int),
                ("tile_m", ctypes.c_int), ("tile_n", ctypes.c_int), ("tile_k", ctypes.c_int),
                ("threads", ctypes.c_int), ("vec_a", ctypes.c_int), ("vec_b", ctypes.c_int),
                ("even", ctypes.c_int), ("variant", ctypes.c_int), ("grid", ctypes.c_int64), ("lds_bytes", ctypes.c_int64),
                ("model_bytes", ctypes.c_double), ("name", ctypes.c_char * 48),
                ("workspace_bytes", ctypes.c_int64), ("ksplit", ctypes.c_int), ("streamk", ctypes.c_int)]


class GemmError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


_lib = None


def lib():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run dense_gemm_05_amd.build.build_library()")
    L = ctypes.CDLL(LIB_PATH)
    i64, p, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    u64 = ctypes.c_uint64
    L.gemm_sgemm.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, p]
    L.gemm_sgemm.restype = i32
    L.gemm_bf16.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, i32, p]
    L.gemm_bf16.restype = i32
    L.gemm_bf16_batched.argtypes = [i64, i64, i64, i64, p, i64, i64, p, i64, i64, p, i64, i64, i32, p]
    L.gemm_bf16_batched.restype = i32
    L.gemm_bf16_nt.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, i32, p]
    L.gemm_bf16_nt.restype = i32
    L.gemm_bf16_nt_batched.argtypes = [i64, i64, i64, i64, p, i64, i64, p, i64, i64, p, i64, i64, i32, p]
    L.gemm_bf16_nt_batched.restype = i32
    L.gemm_bf16_tn.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, i32, p]
    L.gemm_bf16_tn.restype = i32
    L.gemm_bf16_tn_batched.argtypes = [i64, i64, i64, i64, p, i64, i64, p, i64, i64, p, i64, i64, i32, p]
    L.gemm_bf16_tn_batched.restype = i32
    L.gemm_fp8_quantize_rows.argtypes = [i64, i64, p, i64, p, i64, p, p]
    L.gemm_fp8_quantize_rows.restype = i32
    L.gemm_fp8_quantize_cols.argtypes = [i64, i64, p, i64, p, i64, p, p]
    L.gemm_fp8_quantize_cols.restype = i32
    L.gemm_fp8_nt.argtypes = [i64, i64, i64, p, i64, p, p, i64, p, p, i64, i32, p]
    L.gemm_fp8_nt.restype = i32
    L.gemm_fp8_nt_batched.argtypes = [i64, i64, i64, i64, p, i64, i64, p, p, i64, i64, p, p, i64, i64, i32, p]
    L.gemm_fp8_nt_batched.restype = i32
    L.gemm_fp8_nt_affine.argtypes = [i64, i64, i64, i64, p, i64, i64, p, p, i64, i64, p, ctypes.c_float, p,
                                     ctypes.c_float, p, i64, i64, i32, p]
    L.gemm_fp8_nt_affine.restype = i32
    L.gemm_fp8_nt_quant_a.argtypes = [i64, i64, i64, p, i64, p, p, i64, p, p, i64, i32, p, u64, p]
    L.gemm_fp8_nt_quant_a.restype = i32
    L.gemm_bf16_affine.argtypes = [i64, i64, i64, i64, p, i64, i64, p, i64, i64, ctypes.c_float, p, ctypes.c_float,
                                   p, i64, i64, i32, p]
    L.gemm_bf16_affine.restype = i32
    L.gemm_bf16_nt_affine.argtypes = L.gemm_bf16_affine.argtypes
    L.gemm_bf16_nt_affine.restype = i32
    L.gemm_bf16_tn_affine.argtypes = L.gemm_bf16_affine.argtypes
    L.gemm_bf16_tn_affine.restype = i32
    L.gemm_bf16_silu_batched.argtypes = [i64, i64, i64, i64, p, i64, i64, p, i64, i64, p, i64, i64, p]
    L.gemm_bf16_silu_batched.restype = i32
    L.gemm_bf16_swiglu_batched.argtypes = L.gemm_bf16_silu_batched.argtypes
    L.gemm_bf16_swiglu_batched.restype = i32
    L.gemm_bf16_silu.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, p]
    L.gemm_bf16_silu.restype = i32
    L.gemm_bf16_swiglu.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, p]
    L.gemm_bf16_swiglu.restype = i32
    L.gemm_bf16_swiglu_e4m3.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64, ctypes.c_float, p]
    L.gemm_bf16_swiglu_e4m3.restype = i32
    L.gemm_bf16_swiglu_e4m3_batched.argtypes = [i64, i64, i64, i64, p, i64, i64, p, i64, i64, p, i64, i64,
                                                ctypes.c_float, p]
    L.gemm_bf16_swiglu_e4m3_batched.restype = i32
    L.gemm_act_chain.argtypes = [i32, i64, i64, p, i64, p, i64, p, i64, ctypes.c_float, p]
    L.gemm_act_chain.restype = i32
    L.gemm_status_string.argtypes = [i32]
    L.gemm_status_string.restype = ctypes.c_char_p
    L.gemm_plan_query.argtypes = [i32, i64, i64, i64, i64, u64, i64, i64, u64, i64, i64, u64, i64, i64,
                                  i32, ctypes.POINTER(GemmPlan)]
    L.gemm_plan_query.restype = i32
    L.gemm_plan_query_ex.argtypes = [i32] + L.gemm_plan_query.argtypes
    L.gemm_plan_query_ex.restype = i32
    L.gemm_workspace_size.argtypes = [i32, i64, i64, i64, i64, u64, i64, i64, u64, i64, i64, u64, i64, i64,
                                      i32, ctypes.POINTER(u64)]
    L.gemm_workspace_size.restype = i32
    f32 = ctypes.c_float
    L.gemm_run.argtypes = [i32, i64, i64, i64, i64, p, i64, i64, p, i64, i64, p, i64, i64, i32,
                           f32, p, f32, p, p, p, u64, p]
    L.gemm_run.restype = i32
    L.gemm_run_noalloc.argtypes = L.gemm_run.argtypes[:20] + [p]
    L.gemm_run_noalloc.restype = i32
    L.gemm_model_local_bytes.argtypes = [i64, i64, i64, i64]
    L.gemm_model_local_bytes.restype = i64
    L.gemm_model_traffic_bytes.argtypes = [i64, i64, i64, i64, i64, i64]
    L.gemm_model_traffic_bytes.restype = ctypes.c_double
    L.gemm_model_quant_traffic.argtypes = [i64] * 9 + [ctypes.POINTER(ctypes.c_double)] * 2
    L.gemm_model_quant_traffic.restype = None
    L.gemm_model_act_chain_bytes.argtypes = [i32, i64, i64]
    L.gemm_model_act_chain_bytes.restype = ctypes.c_double
    L.gemm_tile_map.argtypes = [i64, i64, i64, i64, i64, ctypes.POINTER(i64), ctypes.POINTER(i64),
                                ctypes.POINTER(i64)]
    L.gemm_tile_map.restype = i32
    _lib = L
    return L


def status_string(status):
    return lib().gemm_status_string(int(status)).decode()
