// Launchers of the brick-binned kernels (host side).
#pragma once

#include <hip/hip_runtime.h>

#include "brick_grid.h"
#include "device_common.h"

namespace tproj {

// prefix[0..nb3] of the pose chunks of every brick (one workgroup).
hipError_t launch_brick_prefix(const BrickGrid& bg, int* prefix, hipStream_t st);
// forward: edge kernel (masked pixels, samples outside the active bricks)
// then the brick kernel; out is fully written.
hipError_t launch_fwd_brick(const KGeom& g, int interp, const BrickGrid& bg, const int* prefix, const float2* vol,
                            const float* rot, const float* shifts, float2* out, hipStream_t st);

}  // namespace tproj
