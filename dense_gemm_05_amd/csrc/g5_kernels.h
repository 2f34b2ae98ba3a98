// g5_kernels.h -- launch entry of the gfx950 kernels (host side).
#pragma once

#include <hip/hip_runtime.h>

#include "g5_common.h"

namespace g5 {

// Enqueue compiled configuration `config_id` on stream `s` with `grid`
// workgroups.  `variant` selects the kernel variant (tiled configs: 0 fully
// general, 1 aligned without edge masking, 2/3 masked ring kernel copying A in
// 16- or 4-byte pieces); the caller guarantees its preconditions.  Returns the
// launch status.
hipError_t launch_config(int config_id, bool f32_inputs, const GemmArgs &a, int variant, int64_t grid,
                         hipStream_t s);

// Small-M path with K split over `ks` workgroups per 128-column strip
// (a.tiles_n strips): `ws` holds batch x strips x ks x 16 x 128 floats of
// partial sums, `cnt` batch x strips counters that are zero on entry and
// left zero on exit.  Requires N % 128 == 0, K % 32 == 0, 16-byte aligned
// rows of X and W.
hipError_t launch_decode_split(const GemmArgs &a, float *ws, unsigned *cnt, int ks, hipStream_t s);

}  // namespace g5
