// g5_ring_epi.hip -- launchers of the bf16 LDS-ring kernel with a fused
// epilogue: SiLU and SwiGLU (page "Operator & Runtime" §5.3.1 and §5.4.2)
// and the affine epilogue alpha * (A.B) + bias + beta * C.
#include <hip/hip_runtime.h>

#include "g5_common.h"
#include "g5_device.h"
#include "g5_kernels.h"

namespace g5 {

template <int BM, int BN, int WGM, int WGN, int NSA, int NSB, int EPI>
static hipError_t launch_bf16_epi(const GemmArgs &a, int variant, int64_t grid, hipStream_t s)
{
    const dim3 g((unsigned)grid), b8(WGM * WGN * 64);
    switch (variant) {
    case 1: hipLaunchKernelGGL((k_bf16_ms<BM, BN, WGM, WGN, NSA, NSB, 16, false, EPI>), g, b8, 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_bf16_ms<BM, BN, WGM, WGN, NSA, NSB, 16, true, EPI>), g, b8, 0, s, a); break;
    case 3: hipLaunchKernelGGL((k_bf16_ms<BM, BN, WGM, WGN, NSA, NSB, 4, true, EPI>), g, b8, 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int EPI>
static hipError_t launch_fused_epi(int config_id, const GemmArgs &a, int variant, int64_t grid, hipStream_t s)
{
    switch (config_id) {
    case CFG_BF16_256x192: return launch_bf16_epi<256, 192, 2, 4, 4, 4, EPI>(a, variant, grid, s);
    case CFG_BF16_256x256: return launch_bf16_epi<256, 256, 2, 4, 4, 4, EPI>(a, variant, grid, s);
    case CFG_BF16_128x128:
        if constexpr (EPI == EPI_AFFINE) {
            // K split over workgroups: the last to arrive applies the epilogue
            if (a.ksplit > 1)
                return launch_ring<128, 128, 4, 2, 4, 4, EPI, true, false>(a, variant, dim3((unsigned)grid), dim3(512), s);
        }
        return launch_bf16_epi<128, 128, 4, 2, 4, 4, EPI>(a, variant, grid, s);
    default: return hipErrorInvalidValue;
    }
}

// The affine epilogue with B given transposed (Bt [N, K]).
static hipError_t launch_affine_bt(int config_id, const GemmArgs &a, int variant, int64_t grid, hipStream_t s)
{
    const dim3 g((unsigned)grid), b8(512);
    switch (config_id) {
    case CFG_BF16_256x192: return launch_ring<256, 192, 2, 4, 4, 4, EPI_AFFINE, false, true>(a, variant, g, b8, s);
    case CFG_BF16_256x256: return launch_ring<256, 256, 2, 4, 4, 4, EPI_AFFINE, false, true>(a, variant, g, b8, s);
    case CFG_BF16_128x128:
        if (a.ksplit > 1) return launch_ring<128, 128, 4, 2, 4, 4, EPI_AFFINE, true, true>(a, variant, g, b8, s);
        return launch_ring<128, 128, 4, 2, 4, 4, EPI_AFFINE, false, true>(a, variant, g, b8, s);
    default: return hipErrorInvalidValue;
    }
}

// The affine epilogue with A given transposed (At [K, M]): variants 1-2.
static hipError_t launch_affine_at(int config_id, const GemmArgs &a, int variant, int64_t grid, hipStream_t s)
{
    const dim3 g((unsigned)grid), b8(512);
    switch (config_id) {
    case CFG_BF16_256x192: return launch_ring<256, 192, 2, 4, 4, 4, EPI_AFFINE, false, false, false, true>(a, variant, g, b8, s);
    case CFG_BF16_256x256: return launch_ring<256, 256, 2, 4, 4, 4, EPI_AFFINE, false, false, false, true>(a, variant, g, b8, s);
    case CFG_BF16_128x128:
        if (a.ksplit > 1)
            return launch_ring<128, 128, 4, 2, 4, 4, EPI_AFFINE, true, false, false, true>(a, variant, g, b8, s);
        return launch_ring<128, 128, 4, 2, 4, 4, EPI_AFFINE, false, false, false, true>(a, variant, g, b8, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_fused(int config_id, int epi, const GemmArgs &a, int variant, int64_t grid, hipStream_t s)
{
    if (epi == EPI_SILU) return launch_fused_epi<EPI_SILU>(config_id, a, variant, grid, s);
    if (epi == EPI_SWIGLU) return launch_fused_epi<EPI_SWIGLU>(config_id, a, variant, grid, s);
    if (epi == EPI_AFFINE)
        return a.fp8       ? launch_ring_fp8_affine(config_id, a, variant, grid, s)
               : a.b_trans ? launch_affine_bt(config_id, a, variant, grid, s)
               : a.a_trans ? launch_affine_at(config_id, a, variant, grid, s)
                           : launch_fused_epi<EPI_AFFINE>(config_id, a, variant, grid, s);
    return hipErrorInvalidValue;
}

// The affine epilogue with nothing to multiply (K == 0, or alpha == 0, where
// A and B are not read): C := bias[n] + beta * C over batch x M x N, element
// by element (grid-stride); C is read only when beta != 0.
__global__ void __launch_bounds__(256) k_affine_no_product(GemmArgs p)
{
    const int64_t total = p.batch * p.M * p.N;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < total; q += stride) {
        const int64_t n = q % p.N, r = q / p.N;
        const int64_t b = r / p.M, m = r % p.M;
        const int64_t off = b * p.sC + m * p.ldc + n;
        float v = p.bias ? __uint_as_float((uint32_t)p.bias[n] << 16) : 0.f;
        if (p.out_f32) {
            float *c = (float *)p.C + off;
            if (p.beta != 0.f) v = __builtin_fmaf(p.beta, *c, v);
            *c = v;
        } else {
            uint16_t *c = (uint16_t *)p.C + off;
            if (p.beta != 0.f) v = __builtin_fmaf(p.beta, __uint_as_float((uint32_t)*c << 16), v);
            *c = (uint16_t)bf16_rne(v);
        }
    }
}

hipError_t launch_affine_no_product(const GemmArgs &a, int64_t grid, hipStream_t s)
{
    hipLaunchKernelGGL(k_affine_no_product, dim3((unsigned)grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace g5
