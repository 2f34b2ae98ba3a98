"""Dense GEMM for AMD Instinct MI355X (gfx950): FP32 and BF16 (FP32
accumulation), single and batched, with fused SiLU, SwiGLU and affine
(alpha, beta, bias) epilogues (SwiGLU also with E4M3FN output),
behind the C ABI of include/gemm05.h."""
from ._lib import (  # noqa: F401
    GEMM_OK, GEMM_ERR_INVALID_ARG, GEMM_ERR_UNSUPPORTED, GEMM_ERR_LAUNCH, GEMM_ERR_NO_DEVICE, GEMM_ERR_WORKSPACE,
    GEMM_WORKSPACE_COUNTER_BYTES,
    GEMM_OUT_BF16, GEMM_OUT_F32, GEMM_OUT_E4M3, GEMM_ACT_SILU, GEMM_ACT_MUL, GEMM_ACT_SWIGLU, GEMM_ACT_QUANT,
    GEMM_ACT_SWIGLU_E4M3, GEMM_OP_SGEMM, GEMM_OP_BF16, GEMM_OP_BF16_SILU, GEMM_OP_BF16_SWIGLU, GEMM_OP_BF16_NT, GEMM_OP_FP8_NT,
    GEMM_OP_BF16_AFFINE, GEMM_OP_BF16_TN, GEMM_OP_BF16_NT_AFFINE,
    GEMM_OP_BF16_TN_AFFINE, GEMM_OP_FP8_NT_AFFINE,
    EXPORTS, LIB_PATH, GemmError, GemmPlan, lib, status_string,
)
from .gemm import (  # noqa: F401
    gemm_sgemm, gemm_bf16, gemm_bf16_batched, gemm_bf16_nt, gemm_bf16_nt_batched, gemm_bf16_tn,
    gemm_bf16_tn_batched, gemm_fp8_quantize_rows, gemm_fp8_quantize_cols, gemm_fp8_nt, gemm_fp8_nt_affine,
    gemm_fp8_nt_quant_a,
    gemm_bf16_silu, gemm_bf16_swiglu, gemm_bf16_silu_batched,
    gemm_bf16_swiglu_batched, gemm_bf16_swiglu_e4m3, gemm_bf16_swiglu_e4m3_batched, gemm_bf16_affine,
    act_chain, act_silu, act_mul, act_swiglu, act_quantize_e4m3, act_swiglu_e4m3,
    gemm_bf16_nt_affine, gemm_bf16_tn_affine, plan_query, workspace_size, Workspace,
)
