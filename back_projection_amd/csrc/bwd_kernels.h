// Launchers of the brick-binned back-projection / backward kernels (host side).
#pragma once

#include <hip/hip_runtime.h>

#include "brick_grid.h"
#include "device_common.h"
#include "timing.h"

namespace tproj {

struct BwdGrid {
  BrickGrid bg;       // tap-space bricks (as the forward gather)
  int npose;          // B * P images
  int nbands;         // radial bands of the per-image maxima (<= 128)
  float inv_band_w;   // 1 / band width (pixels)
};

// Brick edge S of the back-projection bricks for an interpolation kind.
int bwd_brick_edge(int interp);
// Workspace bytes: work list, band maxima, one partial tile per work item.
size_t bwd_ws_bytes(const BwdGrid& bw, int Bv, bool weights);

// Writes vol (and wvol when Wimg != NULL) completely with the adjoint of the
// forward (the back-projection of Y, and of the weight images Wimg).
// side (optional): a second stream and two events on which the band-maximum
// pass runs beside the work list and hit lists (st forks to it first and
// joins it before the brick kernels); the caller keeps each record / wait
// pair of the events together.
struct SideRef {
  hipStream_t s;
  hipEvent_t fork, join;
};
hipError_t launch_bwd(const KGeom& g, int interp, const BwdGrid& bw, void* workspace, const float2* Y,
                      const float* Wimg, const float* rot, const float* shifts, float2* vol, float* wvol,
                      hipStream_t st, const EvPair* ev_brick = nullptr, const EvPair* ev_fold = nullptr,
                      const SideRef* side = nullptr);

}  // namespace tproj
