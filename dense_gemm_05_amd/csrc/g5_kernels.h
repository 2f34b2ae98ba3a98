// g5_kernels.h -- launch entry of the gfx950 kernels (host side).
#pragma once

#include <hip/hip_runtime.h>

#include "g5_common.h"

namespace g5 {

// Enqueue compiled configuration `config_id` on stream `s` with `grid`
// workgroups.  `variant` selects the kernel variant (tiled configs: 0 fully
// general, 1 aligned without edge masking, 2/3 masked ring kernel with 16- or
// 8-byte A rows); the caller guarantees its preconditions.  Returns the
// launch status.
hipError_t launch_config(int config_id, bool f32_inputs, const GemmArgs &a, int variant, int64_t grid,
                         hipStream_t s);

}  // namespace g5
