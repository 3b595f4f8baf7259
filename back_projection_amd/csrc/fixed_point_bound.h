// Bounds behind the fixed-point window scales of the back-projection kernels
// (3D: kernels_bwd.hip, 2D: kernels_2d.hip).  The same source is compiled for
// the GPU, where the kernels use it, and for the host, where the library
// exports it (include/tproj_bounds.h) so that the bounds can be checked
// against brute-force weight sums without a GPU.
//
// A window of poses adds its pixels' taps into fixed-point words whose scale
// is set before the window from the largest pixel value and from a bound on
// the sum of |interpolation weights| one voxel (tile entry) can receive from
// all pixels of one pose.  If such a bound ever fell short, a window's sums
// could overflow; the tests pin them against brute force.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>

namespace tproj {

// 1/x: the hardware reciprocal on the GPU (within one ulp), a division on the
// host.  The bounds below widen every quantity that goes through it by a
// factor 1.0001 (plus 1e-4), far more than that difference.
__host__ __device__ inline float bound_rcp(float x) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_rcpf(x);
#else
  return 1.0f / x;
#endif
}

// The cubic kernel's |value| summed over the unit cells of a plane, at most:
// the largest |K| over [0, 1) is 1 and over [1, 2) it is 0.0741 (at 4/3), so
// a cell of the (d_i, d_j) plane carries at most (2 + 2 * 0.0742)^2 (rounded
// up); the linear kernel's 2^2.
template <int NT>
constexpr float kernel_cells() {
  return NT == 4 ? 4.6152f : 4.0f;
}

// 3D, A = o [R_:0 R_:1] (R row-major 3x3): bound on the pixels of one pose
// that can reach one voxel.  The voxel's support box (edge NT) cuts the slice
// in a disc of radius NT sqrt(3) / 2 in sample space, an ellipse in pixel
// space whose semi-axes are that radius over the singular values of A;
// (2a + 1)^2 bounds its pixels.  Infinite for a degenerate map, NaN for a NaN
// map.
template <int NT>
__host__ __device__ inline float contrib_bound3(float o, const float* R) {
  float g00 = 0.f, g01 = 0.f, g11 = 0.f;
  for (int a = 0; a < 3; ++a) {
    const float c0 = o * R[3 * a], c1 = o * R[3 * a + 1];
    g00 = fmaf(c0, c0, g00);
    g01 = fmaf(c0, c1, g01);
    g11 = fmaf(c1, c1, g11);
  }
  const float d = g00 - g11;
  const float lam = 0.5f * (g00 + g11 - sqrtf(fmaf(d, d, 4.f * g01 * g01)));
  const float sig = sqrtf(fmaxf(lam, 0.f));
  const float a = (0.8660254f * NT) * bound_rcp(sig);
  const float c = 2.f * a + 1.f;
  return c * c;
}

// 3D: bound on the sum of |weights| one voxel receives from all pixels of one
// pose.  |w| = |K(d_x) K(d_y) K(d_z)| <= |K(d_i)| |K(d_j)| for any two axes
// i, j, and the pixels' (d_i, d_j) form the lattice M Z^2 + shift, with M the
// rows i, j of A.  Over each unit cell of the (d_i, d_j) plane |K| |K| sums to
// at most kernel_cells(), and a half-open unit cell holds at most
// (floor(w_1) + 1)(floor(w_2) + 1) lattice points, w_r the sum of |row r of
// M^-1| (the range of pixel coordinate r over the cell).  The best of the
// three axis pairs is taken; about 18.5 for a rotation.  Infinite for a
// rank-deficient map.
template <int NT>
__host__ __device__ inline float weight_sum_bound3(float o, const float* R) {
  float a0[3], a1[3];
  for (int a = 0; a < 3; ++a) {
    a0[a] = o * R[3 * a];
    a1[a] = o * R[3 * a + 1];
  }
  float best = 3.0e38f;
  for (int q = 0; q < 3; ++q) {
    const int i = q == 2 ? 1 : 0, j = q == 0 ? 1 : 2;
    const float d = fabsf(a0[i] * a1[j] - a1[i] * a0[j]);
    if (d > 1e-6f * (fabsf(a0[i]) + fabsf(a1[i])) * (fabsf(a0[j]) + fabsf(a1[j]))) {
      // rows of M^-1 = (1/d) [[a1_j, -a1_i], [-a0_j, a0_i]]; widths rounded up
      const float rd = bound_rcp(d);
      const float w1 = (fabsf(a1[j]) + fabsf(a1[i])) * rd * 1.0001f + 1e-4f;
      const float w2 = (fabsf(a0[j]) + fabsf(a0[i])) * rd * 1.0001f + 1e-4f;
      best = fminf(best, (floorf(w1) + 1.0f) * (floorf(w2) + 1.0f));
    }
  }
  return kernel_cells<NT>() * best;   // 3e38 * cells -> inf
}

// 2D, A = o R (R row-major 2x2): the same bound for one entry of the periodic
// D x D source.  The pixels' taps form the lattice A Z^2 + shift; a unit cell
// holds at most (floor(w1) + 1)(floor(w2) + 1) of them, w_r the sum of |row r
// of A^-1|.  The source is periodic, so an entry also collects the taps of
// its translates by D: the samples lie within |p| <= kmax sigma_max(A) and
// the taps within NT of them, so at most n = floor(2 (kmax sigma_max + NT) /
// D) + 1 translates per axis can be reached; the bound is multiplied by n^2.
// Infinite for a degenerate map.
template <int NT>
__host__ __device__ inline float weight_sum_bound_2d(float o, float kmax, int D, const float* R) {
  const float a00 = o * R[0], a01 = o * R[1], a10 = o * R[2], a11 = o * R[3];
  const float d = fabsf(a00 * a11 - a01 * a10);
  if (!(d > 1e-6f * (fabsf(a00) + fabsf(a01)) * (fabsf(a10) + fabsf(a11)))) return INFINITY;
  const float rd = bound_rcp(d);
  const float w1 = (fabsf(a11) + fabsf(a01)) * rd * 1.0001f + 1e-4f;
  const float w2 = (fabsf(a10) + fabsf(a00)) * rd * 1.0001f + 1e-4f;
  // largest singular value of A (columns (a00, a10), (a01, a11))
  const float g00 = fmaf(a00, a00, a10 * a10), g11 = fmaf(a01, a01, a11 * a11), g01 = fmaf(a00, a01, a10 * a11);
  const float dd = g00 - g11;
  const float smax = sqrtf(0.5f * (g00 + g11 + sqrtf(fmaf(dd, dd, 4.f * g01 * g01)))) * 1.0001f;
  const float nt = floorf(2.0f * (kmax * smax + (float)NT) / (float)D) + 1.0f;
  return kernel_cells<NT>() * (floorf(w1) + 1.0f) * (floorf(w2) + 1.0f) * nt * nt;
}

}  // namespace tproj
