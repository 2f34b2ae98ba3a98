// g5_ring_epi.hip -- launchers of the bf16 LDS-ring kernel with a fused
// epilogue (SiLU, SwiGLU): page "Operator & Runtime" §5.3.1 and §5.4.2.
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
    case CFG_BF16_128x128: return launch_bf16_epi<128, 128, 4, 2, 4, 4, EPI>(a, variant, grid, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_fused(int config_id, int epi, const GemmArgs &a, int variant, int64_t grid, hipStream_t s)
{
    if (epi == EPI_SILU) return launch_fused_epi<EPI_SILU>(config_id, a, variant, grid, s);
    if (epi == EPI_SWIGLU) return launch_fused_epi<EPI_SWIGLU>(config_id, a, variant, grid, s);
    return hipErrorInvalidValue;
}

}  // namespace g5
