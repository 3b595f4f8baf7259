// Brick decomposition of the sample space shared by host and device code.
//
// The gather kernels split tap space (the integer lattice of floor(p)) into
// cubic bricks of edge S.  A pixel belongs to the brick that holds floor(p);
// a workgroup stages the brick plus the interpolation halo of the volume in
// LDS and serves every pixel of a range of poses that falls in it.  Bricks
// that cannot hold a sample of an orthonormal map (|p| <= o * k_max) are
// inactive; pixels whose floor(p) lands in no active brick (maps that are not
// rotations) are served by an edge kernel directly from global memory.
//
// Everything here is integer arithmetic so that host and device derive the
// same work list.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tproj {

struct BrickGrid {
  int S;          // brick edge (floor(p) values per axis owned by a brick)
  int nb;         // bricks per axis
  int nb3;        // nb^3
  int origin;     // floor(p) value at the low corner of brick 0 (all axes)
  int pmax_i;     // integer bound on |p| for orthonormal maps (incl. margin)
  int list_len;   // poses served per volume: P, or B*P when Bv = 1
  int64_t target; // pixels per work item
  int dens_q8;    // 256 / o^2, pixel density in sample space (fixed point)
  int nwork;      // total work items per volume
  int nactive;    // bricks with at least one work item
};

__host__ __device__ inline int64_t isqrt64(int64_t v) {
  if (v <= 0) return 0;
  int64_t r = (int64_t)__builtin_sqrt((double)v);
  while (r * r > v) --r;
  while ((r + 1) * (r + 1) <= v) ++r;
  return r;
}

__host__ __device__ inline void brick_coords(const BrickGrid& g, int b, int& bi, int& bj, int& bk) {
  bi = b % g.nb;
  bj = (b / g.nb) % g.nb;
  bk = b / (g.nb * g.nb);
}

// Squared distance from the origin to the closest point of the brick's box
// [lo, lo + S) (integer corner bound).
__host__ __device__ inline int64_t brick_near_d2(const BrickGrid& g, int bi, int bj, int bk) {
  const int idx[3] = {bi, bj, bk};
  int64_t d2 = 0;
  for (int a = 0; a < 3; ++a) {
    const int64_t lo = g.origin + (int64_t)idx[a] * g.S, hi = lo + g.S;
    int64_t d = 0;
    if (lo > 0) d = lo;
    else if (hi < 0) d = -hi;
    d2 += d * d;
  }
  return d2;
}

__host__ __device__ inline bool brick_active(const BrickGrid& g, int bi, int bj, int bk) {
  return brick_near_d2(g, bi, bj, bk) <= (int64_t)g.pmax_i * g.pmax_i;
}

// Number of pose chunks (work items) of a brick: its expected pixel load over
// the pose list divided by the per-item target.  A random plane through the
// origin meets a brick at distance rho >> S with probability ~0.75 S / rho
// (the cube's mean half-width over rho); the slice is a half plane, which
// halves that, and a hit cuts ~0.67 S^2 pixels (the cube's volume over its
// mean width).  So the load per pose is ~min(0.67 S^2, S^3 / (4 rho)).
__host__ __device__ inline int brick_chunks(const BrickGrid& g, int bi, int bj, int bk) {
  if (!brick_active(g, bi, bj, bk)) return 0;
  const int idx[3] = {bi, bj, bk};
  int64_t c2 = 0;
  for (int a = 0; a < 3; ++a) {
    const int64_t twice_center = 2 * (g.origin + (int64_t)idx[a] * g.S) + g.S;
    c2 += twice_center * twice_center;
  }
  int64_t rho2 = isqrt64(c2);               // twice the centre distance
  if (rho2 < 1) rho2 = 1;
  const int64_t S = g.S;
  // 100 * rho2 * (pixels per pose) = min(67 S^2 rho2, 50 S^3 * ... ): S^3 / (4 rho) = S^3 / (2 rho2)
  const int64_t a1 = 67 * S * S * rho2, a2 = 50 * S * S * S;
  const int64_t per_pose_x100 = a1 < a2 ? a1 : a2;
  // expected pixels = list_len * per_pose_x100 / (100 * rho2) * dens_q8 / 256
  const int64_t num = (int64_t)g.list_len * per_pose_x100 * g.dens_q8;
  const int64_t den = 100 * rho2 * 256 * g.target;
  int64_t k = (num + den - 1) / den;
  if (k < 1) k = 1;
  // a chunk holds at most 65535 poses (hit lists store 16-bit offsets)
  const int64_t kmin = ((int64_t)g.list_len + 65534) / 65535;
  if (k < kmin) k = kmin;
  if (k > g.list_len) k = g.list_len;
  return (int)k;
}

// ---------------------------------------------------------------------------
// Work area of a brick plan (in the caller's workspace, 256-byte aligned
// parts): the work list -- prefix[0..nb3] of the chunk counts, then the active
// rank of every brick (bricks with chunks before it) -- the hit count of every
// work item and volume, and the hit lists.  The list of item (brick b, chunk
// [e0, e1)) of volume v starts at ((v * nactive + rank(b)) * list_len + e0)
// and holds up to e1 - e0 16-bit offsets e - e0.
// ---------------------------------------------------------------------------
struct BrickWork {
  int* prefix;              // nb3 + 1 chunk prefix sums, then nb3 active ranks
  int* counts;              // nvol * nwork hit counts
  unsigned short* hits;     // nvol * nactive * list_len offsets
};

__host__ __device__ inline size_t bw_align256(size_t n) { return (n + 255) / 256 * 256; }

inline size_t brick_work_bytes(const BrickGrid& g, int nvol) {
  return bw_align256((size_t)(2 * g.nb3 + 1) * sizeof(int)) + bw_align256((size_t)nvol * g.nwork * sizeof(int)) +
         bw_align256((size_t)nvol * g.nactive * g.list_len * sizeof(unsigned short));
}

inline BrickWork brick_work(const BrickGrid& g, int nvol, void* base) {
  BrickWork w;
  char* p = (char*)base;
  w.prefix = (int*)p;
  p += bw_align256((size_t)(2 * g.nb3 + 1) * sizeof(int));
  w.counts = (int*)p;
  p += bw_align256((size_t)nvol * g.nwork * sizeof(int));
  w.hits = (unsigned short*)p;
  return w;
}

}  // namespace tproj
