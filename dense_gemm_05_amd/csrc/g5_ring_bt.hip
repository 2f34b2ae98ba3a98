// g5_ring_bt.hip -- launchers of the bf16 LDS-ring kernel for B given
// transposed (Bt [N, K]): the layout of a linear layer's weight and of the
// keys of attention scores.
#include <hip/hip_runtime.h>

#include "g5_common.h"
#include "g5_device.h"
#include "g5_kernels.h"

namespace g5 {

template <int BM, int BN, int WGM, int WGN>
static hipError_t launch_bt(const GemmArgs &a, int variant, int64_t grid, hipStream_t s)
{
    const dim3 g((unsigned)grid), b8(WGM * WGN * 64);
    if constexpr (BM == 128 && BN == 128) {
        if (a.ksplit > 1) return launch_ring<BM, BN, WGM, WGN, 4, 4, EPI_NONE, true, true>(a, variant, g, b8, s);
    }
    return launch_ring<BM, BN, WGM, WGN, 4, 4, EPI_NONE, false, true>(a, variant, g, b8, s);
}

hipError_t launch_ring_bt(int config_id, const GemmArgs &a, int variant, int64_t grid, hipStream_t s)
{
    switch (config_id) {
    case CFG_BF16_256x192: return launch_bt<256, 192, 2, 4>(a, variant, grid, s);
    case CFG_BF16_256x256: return launch_bt<256, 256, 2, 4>(a, variant, grid, s);
    case CFG_BF16_256x128: return launch_bt<256, 128, 4, 2>(a, variant, grid, s);
    case CFG_BF16_128x128: return launch_bt<128, 128, 4, 2>(a, variant, grid, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace g5
