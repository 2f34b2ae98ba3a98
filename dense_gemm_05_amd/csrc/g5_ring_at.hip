// g5_ring_at.hip -- launchers of the bf16 LDS-ring kernel for A given
// transposed (At [K, M]): the layout of the activations in a weight
// gradient X^T.dY, which would otherwise need a transposed copy.
#include <hip/hip_runtime.h>

#include "g5_common.h"
#include "g5_device.h"
#include "g5_kernels.h"

namespace g5 {

template <int BM, int BN, int WGM, int WGN>
static hipError_t launch_at(const GemmArgs &a, int variant, int64_t grid, hipStream_t s)
{
    const dim3 g((unsigned)grid), b8(WGM * WGN * 64);
    if constexpr (BM == 128 && BN == 128) {
        if (a.ksplit > 1) return launch_ring<BM, BN, WGM, WGN, 4, 4, EPI_NONE, true, false, false, true>(a, variant, g, b8, s);
    }
    return launch_ring<BM, BN, WGM, WGN, 4, 4, EPI_NONE, false, false, false, true>(a, variant, g, b8, s);
}

hipError_t launch_ring_at(int config_id, const GemmArgs &a, int variant, int64_t grid, hipStream_t s)
{
    switch (config_id) {
    case CFG_BF16_256x192: return launch_at<256, 192, 2, 4>(a, variant, grid, s);
    case CFG_BF16_256x256: return launch_at<256, 256, 2, 4>(a, variant, grid, s);
    case CFG_BF16_128x128: return launch_at<128, 128, 4, 2>(a, variant, grid, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace g5
