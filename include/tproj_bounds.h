/* The bounds behind the back-projection's fixed-point accumulation
 * (libtproj.so), exported for checking.
 *
 * The back-projection (the adjoint of the rotated-central-slice forward, with
 * the weight channel: French page "Resume technique" 2; Dutch page,
 * Methodologie) adds every pixel's interpolation taps into fixed-point words.
 * A window of poses takes its scale from the largest pixel value it carries
 * and from a bound on the sum of |interpolation weights| that one voxel (or
 * one entry of the periodic 2D source) can receive from all pixels of one
 * pose; if that bound fell short, a window's sums could overflow.  The
 * kernels evaluate these bounds in device code; the functions below evaluate
 * the same source (back_projection_amd/csrc/fixed_point_bound.h) on the host,
 * and tp_bounds_device runs it on the GPU, so that tests can hold both against
 * brute-force weight sums.
 *
 * interp: 1 = cubic (Keys a = -1/2), 0 = linear.  oversampling > 0.
 * rot: a row-major 3x3 (3D) or 2x2 (2D) matrix, host memory, not retained.
 * A rank-deficient map gives +infinity.                                     */
#ifndef TPROJ_BOUNDS_H
#define TPROJ_BOUNDS_H

#include <stdint.h>

#include "tproj.h"

#ifdef __cplusplus
extern "C" {
#endif

/* 3D: bound on the sum over all pixels of one pose of |w|, the product of the
 * three 1D kernel weights, that one voxel receives (A = o [R_:0 R_:1]).      */
float tp_weight_sum_bound_3d(int interp, float oversampling, const float* rot);

/* 3D: bound on the number of pixels of one pose whose taps reach one voxel
 * (poses above 4096 take the direct kernel).                               */
float tp_contrib_bound_3d(int interp, float oversampling, const float* rot);

/* 2D: the weight-sum bound for one entry of the D x D periodic source,
 * periodic translates included, for in-mask pixels |k| <= kmax (A = o R).  */
float tp_weight_sum_bound_2d(int interp, float oversampling, float kmax, int D, const float* rot);

/* The same bounds evaluated by a kernel on the current HIP device, for n
 * maps: kind 0 = tp_weight_sum_bound_3d, 1 = tp_contrib_bound_3d (rot: n x 9
 * floats), 2 = tp_weight_sum_bound_2d (rot: n x 4 floats).  rot and out (n
 * floats) are host memory; the call allocates and frees its own device
 * buffers and returns when out is filled.  TP_E_VALUE for an unknown kind
 * or interp or n outside [0, 2^24], TP_E_NULL for NULL arrays with n > 0,
 * TP_E_DEVICE without a device, TP_E_LAUNCH if an allocation, copy or
 * launch fails.                                                            */
tp_status tp_bounds_device(int kind, int interp, float oversampling, float kmax, int D, const float* rot, int64_t n,
                           float* out);

#ifdef __cplusplus
}
#endif

#endif /* TPROJ_BOUNDS_H */
