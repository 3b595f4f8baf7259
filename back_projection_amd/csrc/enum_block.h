// Block-wide enumeration of the pixels whose slice sample falls in one brick,
// shared by the brick kernels (forward gather, gradients, back-projection).
//
// A separate pass (k_hit_lists / k_bwd_hit_lists) has already listed, per
// work item (a brick and a chunk of its poses), the poses whose slice reaches
// the brick.  A workgroup of NW wavefronts walks that list:
//   1. the hits are taken in windows of up to WIN; one thread per hit sets up
//      the hit's geometry in LDS and bounds its image rows (ky);
//   2. the rows of the window are laid out one after the other and handled
//      one per thread: each thread derives the kx interval of its row from
//      the slab inequalities of the brick, a block-wide scan turns the
//      interval lengths into candidate offsets, and each row writes its index
//      into a per-candidate table (a stage takes rows while their candidates
//      fit the table);
//   3. the candidates (kx, ky, hit) are dealt to the wavefronts in chunks of
//      64, so the lanes stay full across row and hit boundaries; a lane finds
//      its row with one table read.
// The enumeration is a superset of the owned pixels (margins on the
// intervals); the owner test on floor(p), computed with the one slice_coord
// expression, decides.
#pragma once

#include <type_traits>

#include "gather_common.h"

namespace tproj {

constexpr int EB_CMAX = 2048;            // candidates per row stage (a row has at most H/2 + 1 <= 2048)
constexpr int EB_SENTINEL = 0x7fffffff;

// WIN hits per window, NW wavefronts per workgroup (one pose and one row per
// thread).
template <int WIN, int NW>
struct EnumShared {
  static constexpr int THREADS = NW * 64;
  static constexpr int ROWS = NW * 64;
  using RowIndex = std::conditional_t<(ROWS <= 256), unsigned char, unsigned short>;
  int wave_n[NW];
  int wtot[NW];
  int nr, nc;                      // rows and candidates of the current row stage
  float4 geo0[WIN];                // R[0] R[3] R[6] R[1]   (rotation columns 0 and 1)
  float4 geo1[WIN];                // R[4] R[7] sx sy
  int hpose[WIN];                  // image index b * P + n
  int hrow[WIN + 1];               // first row of each hit; hrow[nw] = rows of the window
  int hky[WIN];                    // ky of each hit's first row
  unsigned short rstart[ROWS];     // first candidate of row r (< EB_CMAX)
  int rinfo[ROWS];                 // kx0 | (ky & 0xfff) << 11 | hit << 23
  alignas(4) RowIndex crow[EB_CMAX];   // row of candidate i
};

// crow[j0 .. j1) = row: single entries up to a 4-byte boundary, then whole
// 32-bit words, then the tail (a row's run is about 15 entries).
template <typename RowIndex>
__device__ __forceinline__ void fill_rows(RowIndex* crow, int j0, int j1, int row) {
  constexpr int PER = 4 / (int)sizeof(RowIndex);
  int j = j0;
  for (; j < j1 && (j & (PER - 1)) != 0; ++j) crow[j] = (RowIndex)row;
  const unsigned rep = (unsigned)row * (PER == 4 ? 0x01010101u : 0x00010001u);
  unsigned* words = reinterpret_cast<unsigned*>(crow);
  for (; j + PER <= j1; j += PER) words[j / PER] = rep;
  for (; j < j1; ++j) crow[j] = (RowIndex)row;
}

// ---------------------------------------------------------------------------
// Hit lists.  Work item w of volume v is brick b with the pose chunk [e0, e1)
// of the volume's pose list.  A pass of its own (one workgroup of 256 threads
// per item, one pose per thread at a time) keeps the offsets e - e0 of the
// chunk's poses that pass the hit test, in order, in the item's list, and
// their number in counts; the brick kernels then set up windows of hits from
// the list, skip items without hits before staging their tile, and never test
// poses themselves.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int64_t hit_slot(const BrickGrid& bg, const int* __restrict__ prefix, int vsel, int b,
                                            int e0) {
  return ((int64_t)vsel * bg.nactive + prefix[bg.nb3 + 1 + b]) * bg.list_len + e0;
}

// The chunk [e0, e1) of work item w of brick b.
__device__ __forceinline__ void item_chunk(const BrickGrid& bg, const int* __restrict__ prefix, int b, int w, int& e0,
                                           int& e1) {
  const int chunk = w - prefix[b], nchunk = prefix[b + 1] - prefix[b];
  e0 = (int)((int64_t)bg.list_len * chunk / nchunk);
  e1 = (int)((int64_t)bg.list_len * (chunk + 1) / nchunk);
}

// Body of a hit-list kernel (grid: nwork x volumes, 256 threads).
// test(vsel, e, bl, bh): does pose e of the list reach the box [bl, bh)?
// Each thread tests HL_K poses per pass (pose eb + j * 256 + thread, tests
// issued together, so a long chunk costs few memory round trips); the hits
// of sub-pass j precede those of sub-pass j + 1, which keeps the list in
// pose order.
constexpr int HL_K = 8;
template <typename Test>
__device__ __forceinline__ void build_hit_list(const BrickGrid& bg, const int* __restrict__ prefix,
                                               unsigned short* __restrict__ hits, int* __restrict__ counts,
                                               Test test) {
  __shared__ int wcount[HL_K][4];
  const int w = blockIdx.x, vsel = blockIdx.y;
  if (w >= bg.nwork) return;
  const int b = find_brick(prefix, bg.nb3, w);
  int bi, bj, bk, e0, e1;
  brick_coords(bg, b, bi, bj, bk);
  item_chunk(bg, prefix, b, w, e0, e1);
  const int lo[3] = {bg.origin + bi * bg.S, bg.origin + bj * bg.S, bg.origin + bk * bg.S};
  const float bl[3] = {(float)lo[0], (float)lo[1], (float)lo[2]};
  const float bh[3] = {(float)(lo[0] + bg.S), (float)(lo[1] + bg.S), (float)(lo[2] + bg.S)};
  unsigned short* out = hits + hit_slot(bg, prefix, vsel, b, e0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const unsigned long long below = (1ull << lane) - 1ull;
  int cnt = 0;
  for (int eb = e0; eb < e1; eb += 256 * HL_K) {
    bool hit[HL_K];
#pragma unroll
    for (int j = 0; j < HL_K; ++j) {
      const int e = eb + j * 256 + tid;
      hit[j] = e < e1 && test(vsel, e, bl, bh);
    }
    unsigned long long m[HL_K];
#pragma unroll
    for (int j = 0; j < HL_K; ++j) {
      m[j] = __ballot(hit[j]);
      if (lane == 0) wcount[j][wave] = __popcll(m[j]);
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < HL_K; ++j) {
      int before = cnt, total = cnt;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int c = wcount[j][v];
        if (v < wave) before += c;
        total += c;
      }
      if (hit[j]) out[before + __popcll(m[j] & below)] = (unsigned short)(eb + j * 256 + tid - e0);
      cnt = total;
    }
    __syncthreads();   // every wavefront has read the counts before the next pass
  }
  if (tid == 0) counts[(int64_t)vsel * bg.nwork + w] = cnt;
}

// Slice coordinate from the two rotation columns; the same arithmetic as
// slice_coord, so that every kernel agrees on floor(p).
__device__ __forceinline__ void slice_coord_cols(const KGeom& g, const float4& c0, const float4& c1, float kx,
                                                 float ky, float p[3]) {
  p[0] = g.o * fmaf(c0.w, ky, c0.x * kx);
  p[1] = g.o * fmaf(c1.x, ky, c0.y * kx);
  p[2] = g.o * fmaf(c1.y, ky, c0.z * kx);
}

// The first two rotation columns as a row-major 3x3 array (column 2 unused).
__device__ __forceinline__ void cols_to_r9(const float4& c0, const float4& c1, float R[9]) {
  R[0] = c0.x; R[1] = c0.w; R[2] = 0.f;
  R[3] = c0.y; R[4] = c1.x; R[5] = 0.f;
  R[6] = c0.z; R[7] = c1.y; R[8] = 0.f;
}

// DPP move of v (lanes the control does not reach get old).
template <int CTRL, int RM>
__device__ __forceinline__ int dpp_int(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, RM, 0xf, false);
}

// Inclusive prefix sum across the wavefront: DPP row shifts within each row
// of 16 lanes, then the row broadcasts of lanes 15 and 31.
__device__ __forceinline__ int wave_scan_incl(int v) {
  v += dpp_int<0x111, 0xf>(0, v);   // row_shr:1
  v += dpp_int<0x112, 0xf>(0, v);   // row_shr:2
  v += dpp_int<0x114, 0xf>(0, v);   // row_shr:4
  v += dpp_int<0x118, 0xf>(0, v);   // row_shr:8
  v += dpp_int<0x142, 0xa>(0, v);   // row_bcast:15 into rows 1 and 3
  v += dpp_int<0x143, 0xc>(0, v);   // row_bcast:31 into rows 2 and 3
  return v;
}

// No per-hit work beyond the set-up.
struct NoHitHook {
  __device__ void operator()(bool, const float*, int) const {}
};

// Window set-up: threads t < nw take the hit at list entry e0 + hl[t] (hl:
// the window's part of the item's hit list).  Writes the geometry, the image
// index and the row range of every hit, then the row prefix.  hook(valid, R,
// pose) runs on every lane of wavefront 0 (valid: the lane holds a hit; R: its
// rotation, row-major), before the closing barrier, so what it writes to LDS
// is visible on return.
template <int WIN, int NW, typename Hook = NoHitHook>
__device__ __forceinline__ void window_setup(EnumShared<WIN, NW>& es, const KGeom& g, const float* __restrict__ rot,
                                             const float* __restrict__ shifts, int vsel, int e0,
                                             const unsigned short* __restrict__ hl, int nw, const float bl[3],
                                             const float bh[3], Hook hook = Hook()) {
  static_assert(WIN <= 64, "one wavefront sets up a window");
  const int tid = threadIdx.x;
  if (tid < 64) {
    int nrows = 0, pose = 0;
    float R[9];
#pragma unroll
    for (int a = 0; a < 9; ++a) R[a] = 0.f;
    if (tid < nw) {
      int bimg, n;
      list_entry(g, vsel, e0 + (int)hl[tid], bimg, n);
      const float* Rg = rot + 9 * ((int64_t)(g.Br == 1 ? 0 : bimg) * g.P + n);
#pragma unroll
      for (int a = 0; a < 9; ++a) R[a] = Rg[a];
      float sx = 0.f, sy = 0.f;
      if (shifts) {
        const float* s = shifts + 2 * ((int64_t)(g.Bs == 1 ? 0 : bimg) * g.P + n);
        sx = s[0];
        sy = s[1];
      }
      pose = bimg * g.P + n;
      es.geo0[tid] = make_float4(R[0], R[3], R[6], R[1]);
      es.geo1[tid] = make_float4(R[4], R[7], sx, sy);
      es.hpose[tid] = pose;
      SliceRows sr;
      if (slice_rows_box(g, R, bl, bh, sr)) nrows = sr.ky_hi - sr.ky_lo + 1;
      es.hky[tid] = sr.ky_lo;
    }
    const int v = wave_scan_incl(nrows);
    if (tid <= WIN) {
      if (tid == 0) es.hrow[0] = 0;
      if (tid < WIN) es.hrow[tid + 1] = v;
    }
    hook(tid < nw, R, pose);
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

// Row stage: rows qb, qb + 1, ... of the window, one per thread, as many as
// fit the workgroup's threads and EB_CMAX candidates.  Returns the candidate count and,
// in nr, the rows taken (both block-uniform; nr >= 1 while rows remain, as one
// row has at most H/2 + 1 <= EB_CMAX candidates).
template <int WIN, int NW>
__device__ __forceinline__ int row_stage(EnumShared<WIN, NW>& es, const KGeom& g, int qb, int nrows, int nw,
                                         const float bl[3], const float bh[3], int& nr) {
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
  const int v = wave_scan_incl(cnt);
  if (lane == 63) es.wtot[wave] = v;
  __syncthreads();
  int carry = 0, total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int t = es.wtot[w];
    if (w < wave) carry += t;
    total += t;
  }
  const int incl = carry + v, start = incl - cnt;
  // the rows whose candidates fit the table: a prefix of the rows, since the
  // inclusive counts grow (usually all of them: then every thread knows the
  // stage's counts without another round through LDS)
  const bool all = total <= EB_CMAX;   // block-uniform
  const bool take = q < nrows && incl <= EB_CMAX;
  if (!all) {
    const unsigned long long tm = __ballot(take);
    if (lane == 0) es.wave_n[wave] = __popcll(tm);
  }
  if (take) {
    es.rstart[tid] = start;
    es.rinfo[tid] = kx0 | ((ky & 0xfff) << 11) | (h << 23);
    fill_rows(es.crow, start, start + cnt, tid);
  }
  __syncthreads();
  if (all) {
    nr = min(NW * 64, nrows - qb);
    return total;
  }
  int n_taken = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) n_taken += es.wave_n[w];
  if (tid == n_taken - 1) es.nc = incl;
  __syncthreads();
  nr = n_taken;
  return es.nc;
}

// Candidate i (< the row stage's count): its hit, kx and ky.
template <int WIN, int NW>
__device__ __forceinline__ void candidate_at(const EnumShared<WIN, NW>& es, int i, int& h, int& kx, int& ky) {
  const int r = es.crow[i];
  const int info = es.rinfo[r];
  h = info >> 23;
  ky = (int)((unsigned)info << 9) >> 20;   // bits 11..22, sign-extended
  kx = (info & 0x7ff) + (i - es.rstart[r]);
}

// A candidate pixel with what the per-pixel work needs: its hit (key), whether
// the brick owns it and it lies in the mask (act), the sample p, floor(p)
// relative to the brick (l), the image element and the pose's shifts.
struct Cand {
  int key;
  bool act;
  float kx, ky;
  float p[3];
  int l[3];
  int64_t k;
  float sx, sy;
};

// Candidate i of the current row stage (i >= ncand: key = EB_SENTINEL).
template <int WIN, int NW>
__device__ __forceinline__ void cand_prep(const EnumShared<WIN, NW>& es, const KGeom& g, int i, int ncand, const int lo[3],
                                          int S, Cand& c) {
  c.key = EB_SENTINEL;
  c.act = false;
  c.k = 0;
  if (i < ncand) {
    int h, kx, ky;
    candidate_at(es, i, h, kx, ky);
    c.key = h;
    c.kx = (float)kx;
    c.ky = (float)ky;
    const float4 c0 = es.geo0[h], c1 = es.geo1[h];
    slice_coord_cols(g, c0, c1, c.kx, c.ky, c.p);
    c.sx = c1.z;
    c.sy = c1.w;
    c.act = owned(c.p, lo, S, c.l) && in_mask(g, c.kx, c.ky);
    c.k = (int64_t)es.hpose[h] * g.npix + pixel_index(g, kx, ky);
  }
}

// ---------------------------------------------------------------------------
// Bank-spreading lane permutation.  The LDS serves 64-bit reads and atomics
// for sixteen lanes at a time, and lanes of such a group whose addresses
// share a bank pair (16 pairs of 4-byte banks per 8-byte column) serialise.
// Every tap of a pixel sits at the same offset from the pixel's first tap, so
// the bank pair of the first tap (key 0..15) decides all of the pixel's
// conflicts.  The lanes are ranked by key and rank r moves to lane
// (r % 8) * 8 + r / 8, so that each group of eight consecutive lanes holds
// keys spread over the whole range (measured: as fast as spreading over the
// sixteen-lane groups, about twice the rate of unpermuted random keys; with
// random keys no assignment gets near the conflict-free rate, as the rarest
// keys are held by too few lanes).  Inactive lanes (key < 0) go last.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int spread_dest(int key) {
  const int lane = threadIdx.x & 63;
  const unsigned long long below = (1ull << lane) - 1ull;
  const unsigned long long act = __ballot(key >= 0);
  const bool a = key >= 0;
  unsigned long long less = 0ull, eq = act;
#pragma unroll
  for (int j = 3; j >= 0; --j) {
    const unsigned long long bj = __ballot(a && ((key >> j) & 1)) ;
    if (a && ((key >> j) & 1)) {
      less |= eq & ~bj;
      eq &= bj;
    } else {
      eq &= ~bj;
    }
  }
  const int r = a ? __popcll(less) + __popcll(eq & below) : __popcll(act) + __popcll(~act & below);
  return ((r & 7) << 3) | (r >> 3);
}

// Send v to lane dest (each lane a distinct dest), and fetch from lane src.
__device__ __forceinline__ int lane_send(int v, int dest) { return __builtin_amdgcn_ds_permute(dest << 2, v); }
__device__ __forceinline__ float lane_send(float v, int dest) {
  return __int_as_float(__builtin_amdgcn_ds_permute(dest << 2, __float_as_int(v)));
}
__device__ __forceinline__ float lane_fetch(float v, int src) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(v)));
}
__device__ __forceinline__ float2 lane_fetch(float2 v, int src) {
  return make_float2(lane_fetch(v.x, src), lane_fetch(v.y, src));
}

// ---------------------------------------------------------------------------
// Per-hit rotation / shift gradient sums: the wavefront sums of each hit
// (grad_collect, below) are added to the hit's sum in LDS (atomic adds whose
// results are not waited for).  At the end of a window the sums go to the
// pose's gradient with global atomics, scaled by o (rotation) or 2 pi / H
// (shifts).
// ---------------------------------------------------------------------------
template <int WIN, int NW>
__device__ __forceinline__ void grad_flush(const KGeom& g, const EnumShared<WIN, NW>& es, float (*gw)[8], int nw,
                                           float* __restrict__ grad_rot, float* __restrict__ grad_s) {
  static_assert(WIN * 8 <= NW * 64, "one thread per hit and term");
  const int tid = threadIdx.x;
  if (tid < nw * 8) {
    const int h = tid >> 3, q = tid & 7;
    const float v = gw[h][q];
    gw[h][q] = 0.f;
    const int pose = es.hpose[h];
    const int bimg = pose / g.P, n = pose - bimg * g.P;
    if (q < 6) {
      if (grad_rot) atomicAdd(grad_rot + 9 * ((int64_t)(g.Br == 1 ? 0 : bimg) * g.P + n) + 3 * (q >> 1) + (q & 1), g.o * v);
    } else if (grad_s) {
      atomicAdd(grad_s + 2 * ((int64_t)(g.Bs == 1 ? 0 : bimg) * g.P + n) + (q - 6), 6.283185307179586f * g.inv_h * v);
    }
  }
}

// Per-lane terms -> per-hit sums (all 64 lanes of the wavefront call this),
// added to gw[key][term] in LDS.  Keys rise along the lanes (candidates are
// ordered by hit; idle lanes hold EB_SENTINEL), so the wavefront holds one or
// a few runs of keys; each run is summed by a butterfly reduce-scatter with
// the other keys' terms masked out: in three steps a lane keeps half of its
// terms and adds its partner's share of them (lanes 1, 2 and 4 apart), after
// which lane i holds term 4 b0 + 2 b1 + b2 (b_j: bit j of i) summed over 8
// lanes; a step 8 lanes apart completes the row of 16, and two row swaps the
// wavefront.  Lanes 0-7 then add the 8 totals to LDS.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

__device__ __forceinline__ float wave_term_sum(const float (&t)[8]) {
  const int lane = threadIdx.x & 63;
  const bool b0 = lane & 1, b1 = lane & 2, b2 = lane & 4;
  float u[4], v[2];
#pragma unroll
  for (int j = 0; j < 4; ++j)   // partner lane ^ 1 (quad_perm 1,0,3,2)
    u[j] = (b0 ? t[j + 4] : t[j]) + dpp_f<0xB1>(b0 ? t[j] : t[j + 4]);
#pragma unroll
  for (int j = 0; j < 2; ++j)   // partner lane ^ 2 (quad_perm 2,3,0,1)
    v[j] = (b1 ? u[j + 2] : u[j]) + dpp_f<0x4E>(b1 ? u[j] : u[j + 2]);
  // partner 4 lanes away in the row (row_ror:4): opposite bit 2, same bits 0-1
  float w = (b2 ? v[1] : v[0]) + dpp_f<0x124>(b2 ? v[0] : v[1]);
  w += dpp_f<0x128>(w);         // 8 lanes away (row_ror:8): the same term
  // rows 0 + 1 and 2 + 3, then the two halves
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(w), __float_as_uint(w), false, false);
  w = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(w), __float_as_uint(w), false, false);
  return __uint_as_float(h[0]) + __uint_as_float(h[1]);
}

__device__ __forceinline__ void grad_collect(const float (&acc)[8], int key, float (*gw)[8]) {
  const int lane = threadIdx.x & 63;
  const int term = ((lane & 1) << 2) | (lane & 2) | ((lane >> 2) & 1);
  int k = __builtin_amdgcn_readfirstlane(key);
  if (k == EB_SENTINEL) return;
  if (k == __builtin_amdgcn_readlane(key, 63)) {   // one key: no masks
    const float s = wave_term_sum(acc);
    if (lane < 8) atomicAdd(&gw[k][term], s);
    return;
  }
  for (;;) {   // wave-uniform loop over the runs of keys
    float t[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) t[q] = key == k ? acc[q] : 0.f;
    const float s = wave_term_sum(t);
    if (lane < 8) atomicAdd(&gw[k][term], s);
    const unsigned long long later = __ballot(key > k && key != EB_SENTINEL);
    if (later == 0ull) break;
    k = __builtin_amdgcn_readlane(key, __builtin_ctzll(later));
  }
}

}  // namespace tproj
