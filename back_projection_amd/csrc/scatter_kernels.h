// Launchers of the brick-owned scatter (host side).
#pragma once

#include <hip/hip_runtime.h>

#include "device_common.h"
#include "scatter_grid.h"

namespace tproj {

// Workspace bytes of the scatter: work-list tables + partial tiles.
size_t scatter_ws_bytes(const ScatterGrid& sg, int Bv);
// Writes vol (and wvol when Wimg != NULL) completely: bricks, chunk reduction,
// then the edge pixels with global atomics.
hipError_t launch_scatter_brick(const KGeom& g, int interp, const ScatterGrid& sg, void* workspace, const float2* Y,
                                const float* Wimg, const float* rot, const float* shifts, float2* vol, float* wvol,
                                hipStream_t st);

}  // namespace tproj
