// Launchers of the brick-binned kernels (host side).
#pragma once

#include <hip/hip_runtime.h>

#include "brick_grid.h"
#include "device_common.h"
#include "timing.h"

namespace tproj {

// the work list of a brick plan: prefix[0..nb3] of the pose chunks of every
// brick, then the bricks' active ranks (one workgroup).
hipError_t launch_brick_prefix(const BrickGrid& bg, int* prefix, hipStream_t st);
// forward: edge kernel (masked pixels, samples outside the active bricks) on
// st_edge, hit lists and brick kernel on st; out is fully written once both
// are done.  wk: the plan's work area, its work list already built.
hipError_t launch_fwd_brick(const KGeom& g, int interp, const BrickGrid& bg, const BrickWork& wk, const float2* vol,
                            const float* rot, const float* shifts, float2* out, hipStream_t st, const EvPair* ev,
                            hipStream_t st_edge);
// same for a real volume (weight channel), no phase
hipError_t launch_fwd_brick_real(const KGeom& g, int interp, const BrickGrid& bg, const BrickWork& wk,
                                 const float* vol, const float* rot, float* out, hipStream_t st,
                                 const EvPair* ev = nullptr);
// rotation / shift gradients accumulated (atomically) into zeroed outputs
hipError_t launch_grad_brick(const KGeom& g, int interp, const BrickGrid& bg, const BrickWork& wk, const float2* volc,
                             const float* volr, const float2* U, const float* Ur, const float* rot,
                             const float* shifts, float* grad_rot, float* grad_s, hipStream_t st,
                             const EvPair* ev = nullptr);

}  // namespace tproj
