// Gather helpers shared by the direct and the brick-binned kernels:
// interpolation from global memory (value and derivatives), the slice
// coordinate, the LDS tile of a brick and the row-by-row enumeration of the
// pixels of a rotated central slice that fall in a box of sample space.
//
// The operation is the rotated central slice of the torch-projectors pages
// (Spanish "Resumen tecnico" 2, Dutch Methodologie, French "Resume technique"
// 2) with linear or Catmull-Rom interpolation and per-tap Friedel symmetry.
#pragma once

#include "brick_grid.h"
#include "device_common.h"

namespace tproj {

// p = o * R * (kx, ky, 0)^T.  Every kernel computes the slice coordinate with
// this one expression, so that all of them agree on floor(p).
__device__ __forceinline__ void slice_coord(const KGeom& g, const float* R, float kx, float ky, float p[3]) {
  p[0] = g.o * fmaf(R[1], ky, R[0] * kx);
  p[1] = g.o * fmaf(R[4], ky, R[3] * kx);
  p[2] = g.o * fmaf(R[7], ky, R[6] * kx);
}

// ---------------------------------------------------------------------------
// Interpolation of a complex volume at p (value and, optionally, the three
// partial derivatives).  Rows of taps along x are read contiguously when all
// x-taps are direct or all mirrored; otherwise each tap takes the full rule.
// ---------------------------------------------------------------------------
template <int NT, bool DERIV>
__device__ __forceinline__ void interp_c(const float2* __restrict__ V, const KGeom& g, float px, float py, float pz,
                                         float2& I, float2* dI) {
  const float flx = safe_floor(px), fly = safe_floor(py), flz = safe_floor(pz);
  float wx[NT], wy[NT], wz[NT], dx[NT], dy[NT], dz[NT];
  axis_weights<NT>(px - flx, wx);
  axis_weights<NT>(py - fly, wy);
  axis_weights<NT>(pz - flz, wz);
  if constexpr (DERIV) {
    axis_dweights<NT>(px - flx, dx);
    axis_dweights<NT>(py - fly, dy);
    axis_dweights<NT>(pz - flz, dz);
  }
  const int x0 = (int)flx + first_tap<NT>();
  const int y0 = (int)fly + first_tap<NT>();
  const int z0 = (int)flz + first_tap<NT>();
  // Taps of a sample with |p_a| < D - 3 stay in (-D, D), where one
  // conditional add/subtract wraps them; any other sample (large
  // oversampling, non-orthonormal or non-finite R) takes the general rule.
  const float lim = (float)(g.D - 3);
  const bool near = fabsf(px) < lim && fabsf(py) < lim && fabsf(pz) < lim;
  // 0: all x-taps direct; 1: all mirrored; 2: per-tap rule
  const int mode = !near ? 2 : ((x0 >= 0 && x0 <= g.half - (NT - 1)) ? 0
                                : ((x0 >= 1 - g.half && x0 <= -NT) ? 1 : 2));
  I = make_float2(0.f, 0.f);
  if constexpr (DERIV) { dI[0] = dI[1] = dI[2] = make_float2(0.f, 0.f); }
#pragma unroll
  for (int c = 0; c < NT; ++c) {
    const int tz = z0 + c;
#pragma unroll
    for (int b = 0; b < NT; ++b) {
      const int ty = y0 + b;
      float2 r = make_float2(0.f, 0.f), rx = make_float2(0.f, 0.f);
      if (mode == 0) {
        const float2* row = V + ((int64_t)wrap_fast(tz, g.D) * g.D + wrap_fast(ty, g.D)) * g.W + x0;
#pragma unroll
        for (int a = 0; a < NT; ++a) {
          const float2 v = row[a];
          r.x = fmaf(wx[a], v.x, r.x); r.y = fmaf(wx[a], v.y, r.y);
          if constexpr (DERIV) { rx.x = fmaf(dx[a], v.x, rx.x); rx.y = fmaf(dx[a], v.y, rx.y); }
        }
      } else if (mode == 1) {
        const float2* row = V + ((int64_t)wrap_fast(-tz, g.D) * g.D + wrap_fast(-ty, g.D)) * g.W + (-x0 - (NT - 1));
#pragma unroll
        for (int a = 0; a < NT; ++a) {
          const float2 v = row[NT - 1 - a];
          r.x = fmaf(wx[a], v.x, r.x); r.y = fmaf(-wx[a], v.y, r.y);
          if constexpr (DERIV) { rx.x = fmaf(dx[a], v.x, rx.x); rx.y = fmaf(-dx[a], v.y, rx.y); }
        }
      } else {
#pragma unroll
        for (int a = 0; a < NT; ++a) {
          bool cj;
          const int64_t idx = tap_index<true>(g, x0 + a, ty, tz, cj);
          float2 v = V[idx];
          if (cj) v.y = -v.y;
          r.x = fmaf(wx[a], v.x, r.x); r.y = fmaf(wx[a], v.y, r.y);
          if constexpr (DERIV) { rx.x = fmaf(dx[a], v.x, rx.x); rx.y = fmaf(dx[a], v.y, rx.y); }
        }
      }
      const float wyz = wy[b] * wz[c];
      I.x = fmaf(wyz, r.x, I.x); I.y = fmaf(wyz, r.y, I.y);
      if constexpr (DERIV) {
        dI[0].x = fmaf(wyz, rx.x, dI[0].x); dI[0].y = fmaf(wyz, rx.y, dI[0].y);
        const float gy = dy[b] * wz[c], gz = wy[b] * dz[c];
        dI[1].x = fmaf(gy, r.x, dI[1].x); dI[1].y = fmaf(gy, r.y, dI[1].y);
        dI[2].x = fmaf(gz, r.x, dI[2].x); dI[2].y = fmaf(gz, r.y, dI[2].y);
      }
    }
  }
}

// Same for a real volume; mirrored taps are not conjugated.
template <int NT, bool DERIV>
__device__ __forceinline__ void interp_r(const float* __restrict__ V, const KGeom& g, float px, float py, float pz,
                                         float& I, float* dI) {
  const float flx = safe_floor(px), fly = safe_floor(py), flz = safe_floor(pz);
  float wx[NT], wy[NT], wz[NT], dx[NT], dy[NT], dz[NT];
  axis_weights<NT>(px - flx, wx);
  axis_weights<NT>(py - fly, wy);
  axis_weights<NT>(pz - flz, wz);
  if constexpr (DERIV) {
    axis_dweights<NT>(px - flx, dx);
    axis_dweights<NT>(py - fly, dy);
    axis_dweights<NT>(pz - flz, dz);
  }
  const int x0 = (int)flx + first_tap<NT>();
  const int y0 = (int)fly + first_tap<NT>();
  const int z0 = (int)flz + first_tap<NT>();
  I = 0.f;
  if constexpr (DERIV) { dI[0] = dI[1] = dI[2] = 0.f; }
#pragma unroll
  for (int c = 0; c < NT; ++c) {
#pragma unroll
    for (int b = 0; b < NT; ++b) {
      float r = 0.f, rx = 0.f;
#pragma unroll
      for (int a = 0; a < NT; ++a) {
        bool cj;
        const float v = V[tap_index<true>(g, x0 + a, y0 + b, z0 + c, cj)];
        r = fmaf(wx[a], v, r);
        if constexpr (DERIV) rx = fmaf(dx[a], v, rx);
      }
      const float wyz = wy[b] * wz[c];
      I = fmaf(wyz, r, I);
      if constexpr (DERIV) {
        dI[0] = fmaf(wyz, rx, dI[0]);
        dI[1] = fmaf(dy[b] * wz[c], r, dI[1]);
        dI[2] = fmaf(wy[b] * dz[c], r, dI[2]);
      }
    }
  }
}


template <int NT>
__device__ __forceinline__ float2 interp_global(const float2* __restrict__ V, const KGeom& g, const float p[3]) {
  float2 I;
  interp_c<NT, false>(V, g, p[0], p[1], p[2], I, nullptr);
  return I;
}

// Value of the Hermitian-extended periodic volume at an integer tap.
__device__ __forceinline__ float2 tap_value(const float2* __restrict__ V, const KGeom& g, int tx, int ty, int tz) {
  bool cj;
  float2 v = V[tap_index<true>(g, tx, ty, tz, cj)];
  if (cj) v.y = -v.y;
  return v;
}

// ---------------------------------------------------------------------------
// LDS tile of one brick: the S^3 owned floor values plus the interpolation
// halo (1 below and 2 above for cubic, 1 above for linear), 16^3 entries.
//
// Cubic tiles use the bank-split layout: entry (x, y, z) sits at
//   (x & 3) + 16 (x >> 2) + 64 y + 4 (z & 3) + 1024 (z >> 2)
// (dense, 4096 entries), so that the bank pair of an 8-byte entry (address
// mod 16) is (x & 3) + 4 (z & 3), whatever y is.  A pixel's 4^3 taps cover
// every (x & 3, z & 3) pair once per y row, and a lane may visit its x taps
// and its z taps in any cyclic order: with the order chosen from the lane's
// slot in its group of 16 (SplitTaps), the 16 lanes of a group touch 16
// distinct bank pairs at every step of the tap loop, for any pixels they
// hold.  Measured on random footprints: the conflict-free LDS rate (15.3
// reads and 10.3 64-bit atomics per clock per CU, against 7.1 and 7.0 for
// padded strides with the lanes ranked by bank key).
// Linear tiles keep padded strides (rows of 17, planes of 276 entries) and the
// rank permutation of the lanes (spread_dest).
// ---------------------------------------------------------------------------
template <int NT>
struct Tile {
  static constexpr int S = 17 - NT;          // 13 (cubic) or 15 (linear)
  static constexpr int E = 16;               // tile edge = S + NT - 1
  static constexpr int HL = NT == 4 ? 1 : 0; // halo below
  static constexpr bool SPLIT = NT == 4;     // bank-split layout (cubic)
  static constexpr int SY = SPLIT ? 64 : 17;             // y stride
  static constexpr int SZ = 16 * 17 + 4;     // plane stride (padded layout)
  static constexpr int SIZE = SPLIT ? 4096 : E * SZ;
};

__device__ __forceinline__ int split_x(int x) { return (x & 3) + ((x >> 2) << 4); }
__device__ __forceinline__ int split_z(int z) { return ((z & 3) << 2) + ((z >> 2) << 10); }

// Address of tile entry (x, y, z) in [0, 16)^3.
template <int NT>
__device__ __forceinline__ int tile_addr(int x, int y, int z) {
  if constexpr (Tile<NT>::SPLIT) return split_x(x) + 64 * y + split_z(z);
  else return z * Tile<NT>::SZ + y * Tile<NT>::SY + x;
}

// The tap order of one lane in the bank-split tile, for the pixel whose first
// tap is tile entry l: its slot (lane & 3, (lane >> 2) & 3) fixes the
// rotations t (x) and r (z) that put the lane's step-(a, c) tap in bank pair
// ((lane + a) & 3) + 4 (((lane >> 2) + c) & 3).  Step (a, b, c) reads the tap
// (l0 + ((a + t) & 3), l1 + b, l2 + ((c + r) & 3)), whose x and z weights are
// those of index (a + t) & 3 and (c + r) & 3, at byte offset xo[a] + zo[c] +
// 512 b in a tile of 8-byte entries (zo includes l1; split_taps_lut).
struct SplitTaps {
  int xo[4], zo[4];
  int t, r;
};

// The offsets come from two lane tables in LDS (byte offsets of 8-byte
// entries), so that a pixel's 8 offsets cost two 16-byte LDS reads and a few
// adds instead of per-step residue arithmetic and selects (which issue at
// half the rate of FP32 FMAs).  The step-j x tap has x mod 4 = s = (u + j) & 3
// (u = lane & 3) and lies in [l0, l0 + 3], so x = 4 (l0 >> 2) + s + 4 [s < x4]
// with x4 = l0 & 3: table entry x[4 u + x4] holds 8 (s + 16 [s < x4]) for
// j = 0..3, added to 128 (l0 >> 2); z[4 v + z4] likewise holds
// 8 (4 s + 1024 [s < z4]) with s = (v + j) & 3, added to 8192 (l2 >> 2) +
// 512 l1.
struct SplitLut {
  int4 x[16];
  int4 z[16];
};

// Threads 0..31 write the tables; the caller's next barrier publishes them.
__device__ __forceinline__ void split_lut_fill(SplitLut& t) {
  const int i = (int)threadIdx.x;
  if (i < 32) {
    const int k = i & 15, u = k >> 2, r4 = k & 3;
    int e[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int sres = (u + j) & 3;
      e[j] = i < 16 ? 8 * (sres + (sres < r4 ? 16 : 0)) : 8 * (4 * sres + (sres < r4 ? 1024 : 0));
    }
    const int4 v = make_int4(e[0], e[1], e[2], e[3]);
    if (i < 16) t.x[k] = v;
    else t.z[k] = v;
  }
}

__device__ __forceinline__ void split_taps_lut(const SplitLut& lut, const int l[3], SplitTaps& s) {
  const int lane = (int)threadIdx.x;
  const int u = lane & 3, v = (lane >> 2) & 3;
  s.t = (u - l[0]) & 3;
  s.r = (v - l[2]) & 3;
  const int4 xr = lut.x[4 * u + (l[0] & 3)], zr = lut.z[4 * v + (l[2] & 3)];
  const int bx = (l[0] >> 2) * 128, bz = (l[2] >> 2) * 8192 + l[1] * 512;
  s.xo[0] = bx + xr.x;
  s.xo[1] = bx + xr.y;
  s.xo[2] = bx + xr.z;
  s.xo[3] = bx + xr.w;
  s.zo[0] = bz + zr.x;
  s.zo[1] = bz + zr.y;
  s.zo[2] = bz + zr.z;
  s.zo[3] = bz + zr.w;
}

// floor(p) relative to the brick's low corner; true if inside [0, S)^3.
__device__ __forceinline__ bool owned(const float p[3], const int lo[3], int S, int l[3]) {
  bool in = true;
#pragma unroll
  for (int a = 0; a < 3; ++a) {
    l[a] = (int)safe_floor(p[a]) - lo[a];
    in = in && (l[a] >= 0) && (l[a] < S);
  }
  return in;
}

// ---------------------------------------------------------------------------
// element helpers (complex tile with Friedel conjugation, or real tile)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float2 tap_load(const float2* __restrict__ V, const KGeom& g, int tx, int ty, int tz) {
  return tap_value(V, g, tx, ty, tz);
}
__device__ __forceinline__ float tap_load(const float* __restrict__ V, const KGeom& g, int tx, int ty, int tz) {
  bool cj;
  return V[tap_index<true>(g, tx, ty, tz, cj)];
}
__device__ __forceinline__ float2 zero_of(float2) { return make_float2(0.f, 0.f); }
__device__ __forceinline__ float zero_of(float) { return 0.f; }
__device__ __forceinline__ void fma_into(float w, float2 v, float2& a) { a.x = fmaf(w, v.x, a.x); a.y = fmaf(w, v.y, a.y); }
__device__ __forceinline__ void fma_into(float w, float v, float& a) { a = fmaf(w, v, a); }

// The brick's tile from global memory, THREADS threads: every thread's loads
// are issued before its LDS stores, so the tile costs one memory round trip.
template <int NT, int THREADS, typename T>
__device__ __forceinline__ void stage_tile_t(T* tile, const T* __restrict__ V, const KGeom& g, const int lo[3]) {
  using Tl = Tile<NT>;
  constexpr int N = Tl::E * Tl::E * Tl::E;
  static_assert(N % THREADS == 0, "the tile is a multiple of the workgroup");
  T v[N / THREADS];
#pragma unroll
  for (int k = 0; k < N / THREADS; ++k) {
    const int i = (int)threadIdx.x + k * THREADS;
    const int x = i & 15, y = (i >> 4) & 15, z = i >> 8;
    v[k] = tap_load(V, g, lo[0] - Tl::HL + x, lo[1] - Tl::HL + y, lo[2] - Tl::HL + z);
  }
#pragma unroll
  for (int k = 0; k < N / THREADS; ++k) {
    const int i = (int)threadIdx.x + k * THREADS;
    const int x = i & 15, y = (i >> 4) & 15, z = i >> 8;
    tile[tile_addr<NT>(x, y, z)] = v[k];
  }
}

// w[c] <- w[(c + r) mod 4], r in 0..3: two rounds of bitwise blends under
// all-ones / all-zero masks (one v_bfi each).  The masks are hidden from the
// optimiser, which would otherwise turn the blends into a compare per value.
__device__ __forceinline__ void rotate4(float w[4], int r) {
  int m1 = -(r & 1), m2 = -((r >> 1) & 1);
  asm volatile("" : "+v"(m1), "+v"(m2));
  int t[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) t[c] = (m1 & __float_as_int(w[(c + 1) & 3])) | (~m1 & __float_as_int(w[c]));
#pragma unroll
  for (int c = 0; c < 4; ++c) w[c] = __int_as_float((m2 & t[(c + 2) & 3]) | (~m2 & t[c]));
}

// Value (and, with DERIV, the partial derivatives along x, y, z) of the
// interpolant from a padded-stride tile (linear kernels), for the axis weights
// w* (and their derivatives d*) of the sample; l = floor(p) - lo.
template <int NT, bool DERIV, typename T, int SY = Tile<NT>::SY, int SZ = Tile<NT>::SZ>
__device__ __forceinline__ void interp_tile_w(const T* tile, const int l[3], const float wx[NT], const float wy[NT],
                                              const float wz[NT], const float dx[NT], const float dy[NT],
                                              const float dz[NT], T& I, T* dI) {
  static_assert(NT == 4 || NT == 2, "cubic or linear");
  static_assert(!Tile<NT>::SPLIT, "bank-split tiles are read with interp_split");
  const T* base = tile + l[2] * SZ + l[1] * SY + l[0];
  T z0 = zero_of(T{});
  I = z0;
  if constexpr (DERIV) { dI[0] = z0; dI[1] = z0; dI[2] = z0; }
  // contract x within each row, then y within each plane, then z
#pragma unroll
  for (int c = 0; c < NT; ++c) {
    T s = z0, sx = z0, sy = z0;   // plane sums: wy*r, wy*rx, dy*r
    const T* plane = base + c * SZ;
#pragma unroll
    for (int b = 0; b < NT; ++b) {
      const T* row = plane + b * SY;
      T r = z0, rx = z0;
#pragma unroll
      for (int a = 0; a < NT; ++a) {
        const T v = row[a];
        fma_into(wx[a], v, r);
        if constexpr (DERIV) fma_into(dx[a], v, rx);
      }
      fma_into(wy[b], r, s);
      if constexpr (DERIV) {
        fma_into(wy[b], rx, sx);
        fma_into(dy[b], r, sy);
      }
    }
    fma_into(wz[c], s, I);
    if constexpr (DERIV) {
      fma_into(wz[c], sx, dI[0]);
      fma_into(wz[c], sy, dI[1]);
      fma_into(dz[c], s, dI[2]);
    }
  }
}

// Value (and, with DERIV, the partial derivatives along x, y, z) of the
// cubic interpolant from a bank-split tile, in this lane's tap order
// (SplitTaps); l = floor(p) - lo is the tile entry of the first tap, w* / d*
// the axis weights (and derivatives) in tap order.  Contracts y within each
// column, then x within each plane, then z.
template <bool DERIV, typename T>
__device__ __forceinline__ void interp_split(const T* tile, const SplitLut& lut, const int l[3], const float wx_in[4],
                                             const float wy[4], const float wz_in[4], const float dx_in[4],
                                             const float dy[4], const float dz_in[4], T& I, T* dI) {
  // tap offsets in bytes from the lane tables (halved for 4-byte entries)
  static_assert(sizeof(T) == 8 || sizeof(T) == 4, "complex or real tile entries");
  SplitTaps st;
  split_taps_lut(lut, l, st);
  if constexpr (sizeof(T) == 4) {   // the tables hold offsets of 8-byte entries
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      st.xo[j] >>= 1;
      st.zo[j] >>= 1;
    }
  }
  float wx[4], wz[4], dx[4], dz[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    wx[j] = wx_in[j];
    wz[j] = wz_in[j];
    dx[j] = DERIV ? dx_in[j] : 0.f;
    dz[j] = DERIV ? dz_in[j] : 0.f;
  }
  rotate4(wx, st.t);
  rotate4(wz, st.r);
  if constexpr (DERIV) {
    rotate4(dx, st.t);
    rotate4(dz, st.r);
  }
  const T z0 = zero_of(T{});
  I = z0;
  if constexpr (DERIV) { dI[0] = z0; dI[1] = z0; dI[2] = z0; }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    T p = z0, px = z0, py = z0;   // plane sums: wx*q, dx*q, wx*qy
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const T* col = reinterpret_cast<const T*>(reinterpret_cast<const char*>(tile) + st.xo[a] + st.zo[c]);
      T q = z0, qy = z0;          // column sums: wy*v, dy*v
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const T v = col[64 * b];
        fma_into(wy[b], v, q);
        if constexpr (DERIV) fma_into(dy[b], v, qy);
      }
      fma_into(wx[a], q, p);
      if constexpr (DERIV) {
        fma_into(dx[a], q, px);
        fma_into(wx[a], qy, py);
      }
    }
    fma_into(wz[c], p, I);
    if constexpr (DERIV) {
      fma_into(wz[c], px, dI[0]);
      fma_into(wz[c], py, dI[1]);
      fma_into(dz[c], p, dI[2]);
    }
  }
}

// Largest |p| = |A k| over the in-mask pixels of a pose: kmax * sigma_max(A).
__device__ __forceinline__ float pose_pmax(const KGeom& g, const float* R) {
  float g00 = 0.f, g01 = 0.f, g11 = 0.f;
#pragma unroll
  for (int a = 0; a < 3; ++a) {
    const float c0 = g.o * R[3 * a], c1 = g.o * R[3 * a + 1];
    g00 = fmaf(c0, c0, g00); g01 = fmaf(c0, c1, g01); g11 = fmaf(c1, c1, g11);
  }
  const float d = g00 - g11;
  const float lmax = 0.5f * (g00 + g11 + sqrtf(fmaf(d, d, 4.f * g01 * g01)));
  return g.kmax * sqrtf(lmax) * 1.00001f;   // NaN for a NaN map
}

// Is floor(p) inside an active brick of the grid?
__device__ __forceinline__ bool in_active_brick(const BrickGrid& bg, const float p[3]) {
  int idx[3];
#pragma unroll
  for (int a = 0; a < 3; ++a) {
    const int rel = (int)safe_floor(p[a]) - bg.origin;
    if (rel < 0 || rel >= bg.nb * bg.S) return false;
    idx[a] = rel / bg.S;
  }
  return brick_active(bg, idx[0], idx[1], idx[2]);
}

// |p| <= pmax_i puts floor(p) in an active brick (the brick's nearest point to
// the origin is at most |p| away); only larger samples need the full test.
__device__ __forceinline__ bool served_by_bricks(const BrickGrid& bg, const float p[3]) {
  const float r2 = p[0] * p[0] + p[1] * p[1] + p[2] * p[2];
  const float pm = (float)bg.pmax_i;
  if (r2 <= pm * pm * 0.999f) return true;
  return in_active_brick(bg, p);
}

// Locate work item w: brick b with prefix[b] <= w < prefix[b + 1].
__device__ __forceinline__ int find_brick(const int* __restrict__ prefix, int nb3, int w) {
  int lo = 0, hi = nb3;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (prefix[mid] <= w) lo = mid; else hi = mid;
  }
  return lo;
}

// Pose list of one volume: all (b, n) when the volume is shared, else (v, n).
__device__ __forceinline__ void list_entry(const KGeom& g, int vsel, int e, int& bimg, int& n) {
  if (g.Bv == 1) { bimg = e / g.P; n = e - bimg * g.P; }
  else { bimg = vsel; n = e; }
}

__device__ __forceinline__ int64_t pixel_index(const KGeom& g, int kx, int ky) {
  return (int64_t)(ky >= 0 ? ky : ky + g.H) * g.Wi + kx;
}

// ---------------------------------------------------------------------------
// Enumeration of the pixels whose sample lies in a box [lo, lo + S)^3 of
// sample space.  The slice p = A k with A = o [R_:0 R_:1] cuts the box in a
// convex polygon; its ky extent is bounded through the pseudo-inverse of A,
// and each image row ky gets the kx interval of the three slab inequalities,
// widened by a margin.  The owner test on the exactly computed floor(p) then
// decides, so the enumeration only has to be a superset.
// ---------------------------------------------------------------------------
struct SliceRows {
  float a0[3], a1[3];     // columns of A
  float r0[3];            // approximate 1 / a0 (0 where |a0| is negligible)
  float bl[3], bh[3];     // box bounds in sample space
  int ky_lo, ky_hi;       // candidate rows
};

// Does the plane through the origin spanned by the columns of A meet the box
// [bl, bh]?  (Conservative by a small margin; a NaN map counts as a hit.)
__device__ __forceinline__ bool plane_meets_box(const KGeom& g, const float* R, const float bl[3], const float bh[3]) {
  float a0[3], a1[3];
#pragma unroll
  for (int a = 0; a < 3; ++a) { a0[a] = g.o * R[3 * a]; a1[a] = g.o * R[3 * a + 1]; }
  const float n0 = a0[1] * a1[2] - a0[2] * a1[1];
  const float n1 = a0[2] * a1[0] - a0[0] * a1[2];
  const float n2 = a0[0] * a1[1] - a0[1] * a1[0];
  const float c0 = 0.5f * (bl[0] + bh[0]), c1 = 0.5f * (bl[1] + bh[1]), c2 = 0.5f * (bl[2] + bh[2]);
  const float dist = n0 * c0 + n1 * c1 + n2 * c2;
  const float rad = 0.5f * (fabsf(n0) * (bh[0] - bl[0]) + fabsf(n1) * (bh[1] - bl[1]) + fabsf(n2) * (bh[2] - bl[2]));
  const bool miss = fabsf(dist) > rad * 1.001f + 1e-6f * (1.0f + fabsf(dist));
  return !miss;   // NaN compares false -> not a miss
}

// Can any image pixel (kx >= 0, |k| <= cutoff, inside the image) have its
// sample in the box [bl, bh]?  The plane must meet the box, and the box's
// image in pixel space -- bounded through the pseudo-inverse of A -- must meet
// the half disc of the image.  Conservative (margins; NaN -> true).
__device__ __forceinline__ bool slice_meets_box(const KGeom& g, const float* R, const float bl[3], const float bh[3]) {
  if (!plane_meets_box(g, R, bl, bh)) return false;
  float a0[3], a1[3];
#pragma unroll
  for (int a = 0; a < 3; ++a) { a0[a] = g.o * R[3 * a]; a1[a] = g.o * R[3 * a + 1]; }
  const float g00 = a0[0] * a0[0] + a0[1] * a0[1] + a0[2] * a0[2];
  const float g01 = a0[0] * a1[0] + a0[1] * a1[1] + a0[2] * a1[2];
  const float g11 = a1[0] * a1[0] + a1[1] * a1[1] + a1[2] * a1[2];
  const float det = g00 * g11 - g01 * g01;
  if (!(det > 1e-6f * g00 * g11)) return true;
  // (the hardware reciprocal's ulp is far inside the one-pixel margins below)
  const float rdet = __builtin_amdgcn_rcpf(det);
  float x0 = 0.f, x1 = 0.f, y0 = 0.f, y1 = 0.f;
#pragma unroll
  for (int a = 0; a < 3; ++a) {
    const float ux = (g11 * a0[a] - g01 * a1[a]) * rdet;   // kx = ux . p
    const float uy = (g00 * a1[a] - g01 * a0[a]) * rdet;   // ky = uy . p
    x0 += fminf(ux * bl[a], ux * bh[a]); x1 += fmaxf(ux * bl[a], ux * bh[a]);
    y0 += fminf(uy * bl[a], uy * bh[a]); y1 += fmaxf(uy * bl[a], uy * bh[a]);
  }
  x0 -= 1.0f; x1 += 1.0f; y0 -= 1.0f; y1 += 1.0f;
  const float hh = (float)(g.H >> 1);
  if (x1 < 0.0f || x0 > hh || y1 < -hh || y0 > hh) return false;
  if (g.r2 >= 0.0f) {
    const float nx = fminf(fmaxf(0.0f, x0), x1), ny = fminf(fmaxf(0.0f, y0), y1);
    if (nx * nx + ny * ny > g.r2 + 2.0f * sqrtf(g.r2) + 1.0f) return false;
  }
  return true;
}

// Candidate rows of the pixels whose sample lies in the box [bl, bh), for a
// map that passed slice_meets_box with this box.  Reciprocals are the
// hardware's (an ulp or so): the row bounds carry a margin of one row.
__device__ __forceinline__ bool slice_rows_box(const KGeom& g, const float* R, const float bl[3], const float bh[3],
                                               SliceRows& sr) {
#pragma unroll
  for (int a = 0; a < 3; ++a) {
    sr.a0[a] = g.o * R[3 * a];
    sr.a1[a] = g.o * R[3 * a + 1];
    sr.r0[a] = fabsf(sr.a0[a]) > 1e-20f ? __builtin_amdgcn_rcpf(sr.a0[a]) : 0.0f;
    sr.bl[a] = bl[a];
    sr.bh[a] = bh[a];
  }
  int lo_img = -(g.H >> 1), hi_img = (g.H >> 1) - 1;
  if (g.r2 >= 0.0f) {
    const int rr = (int)floorf(sqrtf(g.r2)) + 1;
    lo_img = max(lo_img, -rr);
    hi_img = min(hi_img, rr);
  }
  sr.ky_lo = lo_img;
  sr.ky_hi = hi_img;
  const float g00 = sr.a0[0] * sr.a0[0] + sr.a0[1] * sr.a0[1] + sr.a0[2] * sr.a0[2];
  const float g01 = sr.a0[0] * sr.a1[0] + sr.a0[1] * sr.a1[1] + sr.a0[2] * sr.a1[2];
  const float g11 = sr.a1[0] * sr.a1[0] + sr.a1[1] * sr.a1[1] + sr.a1[2] * sr.a1[2];
  const float det = g00 * g11 - g01 * g01;
  if (det > 1e-6f * g00 * g11 && det == det) {
    // ky = (row 1 of the pseudo-inverse of A) . p, bounded over the box
    const float rdet = __builtin_amdgcn_rcpf(det);
    float kmin = 0.f, kmax = 0.f;
#pragma unroll
    for (int a = 0; a < 3; ++a) {
      const float u = (g00 * sr.a1[a] - g01 * sr.a0[a]) * rdet;
      const float x = u * sr.bl[a], y = u * sr.bh[a];
      kmin += fminf(x, y);
      kmax += fmaxf(x, y);
    }
    // the box's shadow on the plane is larger than the section of the plane
    // by the box (a convex polygon whose corners each lie on the faces of two
    // different slabs bl_a <= A_a . k <= bh_a); its ky extent is the tighter
    // bound.  Used only when every pair of slab normals is well conditioned
    // (the corners then carry errors far below the one-row margin).
    float pmin = 3.0e38f, pmax = -3.0e38f;
    bool cond = true;
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      const int a = q == 2 ? 1 : 0, b = q == 0 ? 1 : 2, c = 3 - a - b;
      const float d = sr.a0[a] * sr.a1[b] - sr.a1[a] * sr.a0[b];
      const float na = fabsf(sr.a0[a]) + fabsf(sr.a1[a]), nb = fabsf(sr.a0[b]) + fabsf(sr.a1[b]);
      if (!(fabsf(d) > 1e-3f * na * nb)) {
        cond = false;
        continue;
      }
      const float inv = __builtin_amdgcn_rcpf(d);
      const float marg = 2e-2f + 1e-4f * (fabsf(sr.bl[c]) + fabsf(sr.bh[c]));
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const float va = (s & 1) ? sr.bh[a] : sr.bl[a], vb = (s & 2) ? sr.bh[b] : sr.bl[b];
        // [a0 a1; b0 b1] k = [va; vb]
        const float kx = (va * sr.a1[b] - vb * sr.a1[a]) * inv;
        const float ky = (vb * sr.a0[a] - va * sr.a0[b]) * inv;
        const float pc = fmaf(sr.a0[c], kx, sr.a1[c] * ky);
        if (pc >= sr.bl[c] - marg && pc <= sr.bh[c] + marg) {
          pmin = fminf(pmin, ky);
          pmax = fmaxf(pmax, ky);
        }
      }
    }
    if (cond && pmin <= pmax) {
      kmin = fmaxf(kmin, pmin);
      kmax = fminf(kmax, pmax);
    }
    kmin = fmaxf(kmin, (float)lo_img - 2.0f);
    kmax = fminf(kmax, (float)hi_img + 2.0f);
    sr.ky_lo = max(sr.ky_lo, (int)floorf(kmin) - 1);
    sr.ky_hi = min(sr.ky_hi, (int)ceilf(kmax) + 1);
  }
  return sr.ky_lo <= sr.ky_hi;
}

}  // namespace tproj
