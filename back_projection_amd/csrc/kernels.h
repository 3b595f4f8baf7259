// Kernel launchers of libtproj (host side).  Each enqueues on `st` and returns
// hipGetLastError() of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"

namespace tproj {

hipError_t launch_zero(float* p, int64_t n, hipStream_t st);

// out = M * phi * I(vol, p)  (complex volume)
hipError_t launch_project(const KGeom& g, int interp, const float2* vol, const float* rot, const float* shifts,
                          float2* out, hipStream_t st);
// out = M * I(vol, p)  (real volume, no phase)
hipError_t launch_project_real(const KGeom& g, int interp, const float* vol, const float* rot, float* out,
                               hipStream_t st);
// rotation / shift gradients; volc+U (complex channel) and/or volr+Ur (real
// channel); outputs overwritten, except broadcast ones, which must be zeroed
// first and are accumulated.
hipError_t launch_rot_shift_grad(const KGeom& g, int interp, const float2* volc, const float* volr, const float2* U,
                                 const float* Ur, const float* rot, const float* shifts, float* grad_rot,
                                 float* grad_s, hipStream_t st);
// adjoint scatter into zeroed volumes with global float atomics
hipError_t launch_spread_atomic(const KGeom& g, int interp, const float2* Y, const float* Wimg, const float* rot,
                                const float* shifts, float2* Vd, float* Vw, hipStream_t st);

}  // namespace tproj
