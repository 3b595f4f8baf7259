// Brick decomposition of the stored volume for the adjoint scatter, shared by
// host and device code (integer arithmetic only, so both derive the same
// work list).
//
// A brick is an S^3 block of the stored half-spectrum volume (x in [0, D/2],
// y and z in [0, D)).  Through the Friedel rule and the DFT periodicity, each
// brick has a few preimage boxes in tap space: direct copies (x, y, z) + D j
// and, for 1 <= x <= D/2 - 1, mirrored copies (-x, -y, -z) + D j.  A
// workgroup owns one brick for a chunk of the pose list, serves every pixel
// whose taps reach one of these boxes and accumulates only the taps that land
// in its brick.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "brick_grid.h"

namespace tproj {

struct ScatterGrid {
  int S;              // brick edge (stored voxels)
  int nbx, nby, nbz;  // bricks per axis (x covers D/2 + 1)
  int nb3;
  int D, half, W;     // volume box, D/2, D/2 + 1
  int fmin, fmax;     // floor(p) range served by the bricks (all axes)
  int tmin, tmax;     // tap range it implies (inclusive)
  int list_len;       // poses per volume list
  int64_t target;     // pixel visits per work item
  int dens_q8;        // 256 / o^2
  int nwork;          // work items per volume
  int nslots;         // workspace partial tiles per volume (bricks with > 1 chunk)
  int weights;        // 1: the weight channel is accumulated too
  int npose;          // B * P images
  int nbands;         // radial bands of the per-image maxima (<= 128)
  float inv_band_w;   // 1 / band width (pixels)
};

__host__ __device__ inline void sbrick_coords(const ScatterGrid& g, int b, int& bi, int& bj, int& bk) {
  bi = b % g.nbx;
  bj = (b / g.nbx) % g.nby;
  bk = b / (g.nbx * g.nby);
}

// Signed frequency of a stored y/z index (fftfreq order).
__host__ __device__ inline int sfreq(int i, int D) { return i < D / 2 ? i : i - D; }

// Pose chunks of a stored brick: expected pixel visits over the pose list
// (two preimage boxes, each ~min(1.3 (S+3)^2, (S+3)^3 / (2 rho)) pixels per
// pose) divided by the per-item target.
__host__ __device__ inline int sbrick_chunks(const ScatterGrid& g, int bi, int bj, int bk) {
  const int64_t S = g.S, E = g.S + 3;
  const int64_t cx2 = 2 * (int64_t)bi * S + S;
  const int64_t cy2 = 2 * (int64_t)sfreq(bj * g.S, g.D) + S;
  const int64_t cz2 = 2 * (int64_t)sfreq(bk * g.S, g.D) + S;
  int64_t rho2 = isqrt64(cx2 * cx2 + cy2 * cy2 + cz2 * cz2);
  if (rho2 < 1) rho2 = 1;
  const int64_t per_pose_x10 = (13 * E * E * rho2 < 10 * E * E * E) ? 13 * E * E * rho2 : 10 * E * E * E;
  const int64_t num = (int64_t)g.list_len * 2 * per_pose_x10 * g.dens_q8;
  const int64_t den = 10 * rho2 * 256 * g.target;
  int64_t k = (num + den - 1) / den;
  if (k < 1) k = 1;
  if (k > g.list_len) k = g.list_len;
  return (int)k;
}

}  // namespace tproj
