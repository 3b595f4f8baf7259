// Launchers of the 2D -> 2D kernels (host side).  The geometry is the 3D one
// with D the box of the 2D source ([Bv][D][D/2+1]) and 2x2 maps
// ([Br][P][2][2], row-major).  E is the periodic Hermitian extension of a
// source, [Bv][e2_size(D)] (layout below).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "device_common.h"

namespace tproj {

// Layout of the periodic extension E: positions x, y in [-2, D + 2) (a margin
// of two beyond the box on every side, so that no tap of a sample reduced to
// [0, D) needs a wrap), row stride D + 5 entries.
__host__ __device__ inline int e2_rows(int D) { return D + 4; }
__host__ __device__ inline int e2_stride(int D) { return D + 5; }
__host__ __device__ inline int64_t e2_size(int D) { return (int64_t)e2_rows(D) * e2_stride(D); }

hipError_t launch_zero(float* p, int64_t n, hipStream_t st);

// Does an E of this box with bytes_per_entry bytes fit a workgroup's LDS?
int twod_lds_fits(const KGeom& g, size_t bytes_per_entry);
// Workgroups per volume of the 2D kernels (and partial Es of the accumulation).
int twod_parts(const KGeom& g);
// Bytes of partial Es the accumulation needs (data, plus weights).
size_t twod_bp_parts_bytes(const KGeom& g, bool weights);

// E from a stored source (complex / real weight channel).
hipError_t launch2_expand_c(const KGeom& g, const float2* X, float2* E, hipStream_t st);
hipError_t launch2_expand_r(const KGeom& g, const float* X, float* E, hipStream_t st);
// out = M * phi * I(E, p)  (complex), out = M * I(E, p) (real, no phase)
hipError_t launch2_gather_c(const KGeom& g, int interp, const float2* E, const float* rot, const float* shifts,
                            float2* out, hipStream_t st);
hipError_t launch2_gather_r(const KGeom& g, int interp, const float* E, const float* rot, float* out,
                            hipStream_t st);
// rotation / shift gradients added into zeroed grad_rot ([Br][P][2][2]) and
// grad_s; Ec + U (complex channel) and / or Er + Ur (real channel)
hipError_t launch2_grad(const KGeom& g, int interp, const float2* Ec, const float* Er, const float2* U,
                        const float* Ur, const float* rot, const float* shifts, float* grad_rot, float* grad_s,
                        hipStream_t st);
// accumulation of Y (and Wimg into wout when not NULL) into the stored
// half-spectra out / wout (overwritten); mx: B*P floats, parts:
// twod_bp_parts_bytes() bytes of scratch
hipError_t launch2_bp(const KGeom& g, int interp, const float2* Y, const float* Wimg, const float* rot,
                      const float* shifts, float* mx, void* parts, float2* out, float* wout, hipStream_t st);

}  // namespace tproj
