// Block-wide enumeration of the pixels whose slice sample falls in one brick,
// shared by the brick kernels (forward gather, gradients, back-projection).
//
// A workgroup of 256 threads walks its brick's pose list in passes of 256
// poses.  Each pass:
//   1. one pose per thread is tested against the brick; the hit poses are
//      compacted into a list;
//   2. the hits are taken in windows of up to WIN; one thread per hit sets up
//      the hit's geometry in LDS and bounds its image rows (ky);
//   3. the rows of the window are laid out one after the other and handled
//      256 at a time, one per thread: each thread derives the kx interval of
//      its row from the slab inequalities of the brick and a block-wide scan
//      turns the interval lengths into candidate offsets;
//   4. the candidates (kx, ky, hit) of those rows are dealt to the four
//      wavefronts in chunks of 64, so the lanes stay full across row and hit
//      boundaries; each lane finds its row by binary search in LDS.
// The enumeration is a superset of the owned pixels (margins on the
// intervals); the owner test on floor(p), computed with the one slice_coord
// expression, decides.
#pragma once

#include "gather_common.h"

namespace tproj {

constexpr int EB_THREADS = 256;
constexpr int EB_ROWS = 256;
constexpr int EB_SENTINEL = 0x7fffffff;

template <int WIN>
struct EnumShared {
  int hits[EB_THREADS];      // list entries of the hit poses of this pass
  int wave_n[4];
  int wtot[4];
  float4 geo0[WIN];          // R[0] R[3] R[6] R[1]   (rotation columns 0 and 1)
  float4 geo1[WIN];          // R[4] R[7] sx sy
  int hpose[WIN];            // image index b * P + n
  int hrow[WIN + 1];         // first row of each hit; hrow[nw] = rows of the window
  int hky[WIN];              // ky of each hit's first row
  int rpre[EB_ROWS + 1];     // candidates before row r
  int rkx[EB_ROWS];          // first candidate kx of row r
  int rkh[EB_ROWS];          // (hit << 16) | (ky & 0xffff)
};

// Compact the hit flags of one pass (one pose per thread) into es.hits;
// returns the hit count (block-uniform) and this thread's slot (-1: no hit).
template <int WIN>
__device__ __forceinline__ int compact_hits(EnumShared<WIN>& es, bool hit, int e, int& slot) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const unsigned long long m = __ballot(hit);
  if (lane == 0) es.wave_n[wave] = __popcll(m);
  __syncthreads();
  int before = 0, nh = 0;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int c = es.wave_n[v];
    if (v < wave) before += c;
    nh += c;
  }
  slot = -1;
  if (hit) {
    slot = before + __popcll(m & ((1ull << lane) - 1ull));
    es.hits[slot] = e;
  }
  __syncthreads();
  return nh;
}

// Slice coordinate from the two rotation columns; the same arithmetic as
// slice_coord, so that every kernel agrees on floor(p).
__device__ __forceinline__ void slice_coord_cols(const KGeom& g, const float4& c0, const float4& c1, float kx,
                                                 float ky, float p[3]) {
  p[0] = g.o * fmaf(c0.w, ky, c0.x * kx);
  p[1] = g.o * fmaf(c1.x, ky, c0.y * kx);
  p[2] = g.o * fmaf(c1.y, ky, c0.z * kx);
}

// Window set-up: threads t < nw take hit hw + t.  Writes the geometry, the
// image index and the row range of every hit, then the row prefix.
template <int WIN>
__device__ __forceinline__ void window_setup(EnumShared<WIN>& es, const KGeom& g, const float* __restrict__ rot,
                                             const float* __restrict__ shifts, int vsel, int hw, int nw,
                                             const float bl[3], const float bh[3]) {
  static_assert(WIN <= 64, "one wavefront sets up a window");
  const int tid = threadIdx.x;
  if (tid < 64) {
    int nrows = 0;
    if (tid < nw) {
      int bimg, n;
      list_entry(g, vsel, es.hits[hw + tid], bimg, n);
      const float* R = rot + 9 * ((int64_t)(g.Br == 1 ? 0 : bimg) * g.P + n);
      float sx = 0.f, sy = 0.f;
      if (shifts) {
        const float* s = shifts + 2 * ((int64_t)(g.Bs == 1 ? 0 : bimg) * g.P + n);
        sx = s[0];
        sy = s[1];
      }
      es.geo0[tid] = make_float4(R[0], R[3], R[6], R[1]);
      es.geo1[tid] = make_float4(R[4], R[7], sx, sy);
      es.hpose[tid] = bimg * g.P + n;
      SliceRows sr;
      if (slice_rows_box(g, R, bl, bh, sr)) nrows = sr.ky_hi - sr.ky_lo + 1;
      es.hky[tid] = sr.ky_lo;
    }
    int v = nrows;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int u = __shfl_up(v, off, 64);
      if (tid >= off) v += u;
    }
    if (tid <= WIN) {
      if (tid == 0) es.hrow[0] = 0;
      if (tid < WIN) es.hrow[tid + 1] = v;
    }
  }
  __syncthreads();
}

// kx interval of image row ky whose samples may fall in the box [bl, bh]
// (a0, a1: columns of o R; r0: approximate reciprocals of a0).
__device__ __forceinline__ void row_interval(const KGeom& g, const float a0[3], const float a1[3], const float r0[3],
                                             const float bl[3], const float bh[3], int ky, int& kx0, int& cnt) {
  const float fky = (float)ky;
  float xlo = 0.0f, xhi = (float)(g.H >> 1);
  bool ok = true;
  if (g.r2 >= 0.0f) {
    const float rem = g.r2 - fky * fky;
    if (rem < 0.0f) ok = false;
    else xhi = fminf(xhi, floorf(sqrtf(rem)) + 1.0f);
  }
#pragma unroll
  for (int a = 0; a < 3; ++a) {
    // the approximate reciprocal is within a few ulp; the margin (in sample
    // units) and the owner test on the exact floor(p) absorb it
    const float marg = 1e-2f + 1e-4f * (fabsf(bl[a]) + fabsf(bh[a]) + fabsf(a1[a] * fky));
    const float rl = bl[a] - marg - a1[a] * fky;
    const float rh = bh[a] + marg - a1[a] * fky;
    const float c = a0[a], rc = r0[a];
    if (c > 1e-20f) { xlo = fmaxf(xlo, rl * rc); xhi = fminf(xhi, rh * rc); }
    else if (c < -1e-20f) { xlo = fmaxf(xlo, rh * rc); xhi = fminf(xhi, rl * rc); }
    else if (rl > 0.0f || rh < 0.0f) ok = false;
  }
  kx0 = 0;
  cnt = 0;
  if (ok && xlo <= xhi) {
    kx0 = (int)ceilf(xlo);
    const int kx1 = (int)floorf(xhi);
    cnt = kx1 >= kx0 ? kx1 - kx0 + 1 : 0;
  }
}

// Row stage: rows qb .. qb + 255 of the window, one per thread.  Returns the
// number of candidates of these rows (block-uniform).
template <int WIN>
__device__ __forceinline__ int row_stage(EnumShared<WIN>& es, const KGeom& g, int qb, int nrows, int nw,
                                         const float bl[3], const float bh[3]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = qb + tid;
  int cnt = 0, kx0 = 0, h = 0, ky = 0;
  if (q < nrows) {
    // hit of row q: the last h with hrow[h] <= q
#pragma unroll
    for (int step = WIN / 2; step >= 1; step >>= 1)
      if (h + step < nw && es.hrow[h + step] <= q) h += step;
    ky = es.hky[h] + (q - es.hrow[h]);
    const float4 c0 = es.geo0[h], c1 = es.geo1[h];
    const float a0[3] = {g.o * c0.x, g.o * c0.y, g.o * c0.z};
    const float a1[3] = {g.o * c0.w, g.o * c1.x, g.o * c1.y};
    float r0[3];
#pragma unroll
    for (int a = 0; a < 3; ++a) r0[a] = fabsf(a0[a]) > 1e-20f ? __builtin_amdgcn_rcpf(a0[a]) : 0.0f;
    row_interval(g, a0, a1, r0, bl, bh, ky, kx0, cnt);
  }
  int v = cnt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int u = __shfl_up(v, off, 64);
    if (lane >= off) v += u;
  }
  if (lane == 63) es.wtot[wave] = v;
  __syncthreads();
  int carry = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w)
    if (w < wave) carry += es.wtot[w];
  es.rpre[tid + 1] = carry + v;
  if (tid == 0) es.rpre[0] = 0;
  es.rkx[tid] = kx0;
  es.rkh[tid] = (h << 16) | (ky & 0xffff);
  __syncthreads();
  return es.rpre[EB_ROWS];
}

// Candidate i (< the row stage's count): its hit, kx and ky.
template <int WIN>
__device__ __forceinline__ void candidate_at(const EnumShared<WIN>& es, int i, int& h, int& kx, int& ky) {
  int r = 0;
#pragma unroll
  for (int step = EB_ROWS / 2; step >= 1; step >>= 1)
    if (es.rpre[r + step] <= i) r += step;
  const int hk = es.rkh[r];
  h = hk >> 16;
  ky = (int)(short)(hk & 0xffff);
  kx = es.rkx[r] + (i - es.rpre[r]);
}

// ---------------------------------------------------------------------------
// Segmented sums across a wavefront whose lanes carry sorted keys (the hit of
// the candidate; EB_SENTINEL past the end): after seg_scan, each lane holds
// the sum of its key's values from the key's first lane up to itself.  DPP
// row shifts, then the row broadcasts of lanes 15 and 31.
// ---------------------------------------------------------------------------
template <int CTRL, int RM>
__device__ __forceinline__ int dpp_int(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, RM, 0xf, false);
}

template <int CTRL, int RM, int N>
__device__ __forceinline__ void seg_step(float (&v)[N], int key) {
  const int ks = dpp_int<CTRL, RM>(-1, key);
  const float m = ks == key ? 1.0f : 0.0f;
#pragma unroll
  for (int q = 0; q < N; ++q) v[q] = fmaf(m, __int_as_float(dpp_int<CTRL, RM>(0, __float_as_int(v[q]))), v[q]);
}

template <int N>
__device__ __forceinline__ void seg_scan(float (&v)[N], int key) {
  seg_step<0x111, 0xf>(v, key);   // row_shr:1
  seg_step<0x112, 0xf>(v, key);   // row_shr:2
  seg_step<0x114, 0xf>(v, key);   // row_shr:4
  seg_step<0x118, 0xf>(v, key);   // row_shr:8
  seg_step<0x142, 0xa>(v, key);   // row_bcast:15 into rows 1 and 3
  seg_step<0x143, 0xc>(v, key);   // row_bcast:31 into rows 2 and 3
}

// Is this lane the last of its key's run?
__device__ __forceinline__ bool seg_tail(int key) {
  const int lane = threadIdx.x & 63;
  const int next = __shfl_down(key, 1, 64);
  return key != EB_SENTINEL && (lane == 63 || next != key);
}

// ---------------------------------------------------------------------------
// Per-hit rotation / shift gradient sums: a segmented sum over the lanes of
// one hit leaves the hit's partial in its last lane, which adds it to a
// per-wavefront, per-hit sum in LDS (no two lanes of a wavefront share a hit
// there, so no atomics).  At the end of a window the four wavefronts' sums go
// to the pose's gradient with global atomics, scaled by o (rotation) or
// 2 pi / H (shifts).
// ---------------------------------------------------------------------------
template <int WIN>
__device__ __forceinline__ void grad_flush(const KGeom& g, const EnumShared<WIN>& es, float (*gw)[WIN][8], int nw,
                                           float* __restrict__ grad_rot, float* __restrict__ grad_s) {
  const int tid = threadIdx.x;
  if (tid < nw * 8) {
    const int h = tid >> 3, q = tid & 7;
    const float v = gw[0][h][q] + gw[1][h][q] + gw[2][h][q] + gw[3][h][q];
#pragma unroll
    for (int w = 0; w < 4; ++w) gw[w][h][q] = 0.f;
    const int pose = es.hpose[h];
    const int bimg = pose / g.P, n = pose - bimg * g.P;
    if (q < 6) {
      if (grad_rot) atomicAdd(grad_rot + 9 * ((int64_t)(g.Br == 1 ? 0 : bimg) * g.P + n) + 3 * (q >> 1) + (q & 1), g.o * v);
    } else if (grad_s) {
      atomicAdd(grad_s + 2 * ((int64_t)(g.Bs == 1 ? 0 : bimg) * g.P + n) + (q - 6), 6.283185307179586f * g.inv_h * v);
    }
  }
}

// Per-lane terms -> per-hit sums (all 64 lanes of the wavefront call this).
template <int WIN>
__device__ __forceinline__ void grad_collect(float (&acc)[8], int key, float (*gw)[WIN][8]) {
  seg_scan(acc, key);
  if (seg_tail(key)) {
    float* d = gw[threadIdx.x >> 6][key];
#pragma unroll
    for (int q = 0; q < 8; ++q) d[q] += acc[q];
  }
}

}  // namespace tproj
