// Back-projection kernels of libtproj for gfx950: the 2D->3D accumulation
// (with the weight channel), which is also the volume gradient of the 3D->2D
// forward.
//
// The back-projection is the exact adjoint of the rotated-central-slice
// forward: every in-mask pixel adds w * conj(phi) * Y to each of its taps
// (conjugated where the tap is a Friedel mate) and w * Wimg to the weight
// volume (French page, "Resume technique" 2: accumulation with weights for CTF
// correction; Dutch page, Methodologie: Friedel symmetry).
//
// Decomposition: the same tap-space bricks as the forward gather.  A pixel
// belongs to the brick holding floor(p), so every pixel is visited once and all
// its taps fall in the brick's 16^3 halo tile.  The workgroup accumulates the
// taps of its pixels in that tile in LDS and writes the tile to a workspace
// slot; a fold kernel then adds, for every stored voxel, the tile entries of
// all its preimages in tap space (direct copies, and conjugated Friedel mates)
// in a fixed order.  Float atomics in LDS are slow on this GPU while 64-bit
// integer ones are not, so the tile holds fixed-point words (re + im * 2^32,
// one ds_add_u64 per tap; the weight channel, in a launch of its own so that
// each launch holds one tile, one 32-bit word).  Taps are accumulated in
// windows of up to 32 poses
// whose scale is set, before the window, from per-image maxima in radial
// bands of |k| and a bound on the contributions a voxel can receive; no sum
// can overflow, and integer sums make the result deterministic.
#include <algorithm>

#include "brick_grid.h"
#include "brick_kernels.h"
#include "bwd_kernels.h"
#include "device_common.h"
#include "enum_block.h"
#include "fixed_point_bound.h"
#include "gather_common.h"

namespace tproj {

namespace {

#ifndef BWD_EDGE
#define BWD_EDGE 16
#endif
// Tile edge of the back-projection bricks: brick edge S = TE - NT + 1 plus the
// interpolation halo.  16^3 tiles use padded strides like the gather tile;
// 14^3 tiles (unpadded, S = 11 cubic) hold more workgroups per CU in LDS
// but measured slower in a kernel that also gathered the volume (more hits per
// pixel, and spills at the higher occupancy).
constexpr int TE = BWD_EDGE;
constexpr int TSY = TE == 16 ? 17 : TE;
constexpr int TSZ = TE == 16 ? 16 * 17 + 4 : TE * TE;
constexpr int TSIZE = TE * TSZ;            // padded entries
constexpr int TLOG = TE * TE * TE;         // logical entries
#ifndef BWD_NW
#define BWD_NW 4
#endif
constexpr int BNW = BWD_NW;                 // wavefronts per workgroup of the brick kernel
constexpr int BTHREADS = BNW * 64;
constexpr int PER_LANE = (TLOG + BTHREADS - 1) / BTHREADS;   // partial-tile entries per thread
constexpr int WINDOW = 32;                 // poses per fixed-point window
constexpr int SCALE_BATCH = BTHREADS / WINDOW;   // windows whose scales one pass sets
static_assert(WINDOW == 32, "a window's scale is reduced over a half wavefront");
constexpr float FIX_RANGE = 0.9f * 2147483648.0f;
constexpr int MAX_BANDS = 128;

// Fixed-point conversion by the magic-number trick: for |w u| < 2^22,
// fma(w, u, 1.5 * 2^23) rounds w * u to the nearest integer k in one
// instruction and its bit pattern is 0x4B400000 + k.
constexpr float MAGIC = 12582912.0f;
constexpr int MAGIC_BITS = 0x4B400000;

__device__ __forceinline__ int fixed_round(float w, float u) {
  return __float_as_int(fmaf(w, u, MAGIC)) - MAGIC_BITS;
}

// One 64-bit word holding re + im * 2^32 (re signed): sums of such words keep
// both parts exact as long as each partial sum stays within 31 bits.  The two
// magic-number results side by side are (0x4B400000 + re) + 2^32 (0x4B400000
// + im); one 64-bit subtraction of the two offsets leaves re + 2^32 im in
// two's complement (the borrow of a negative re lands in the high word).
constexpr unsigned long long MAGIC_PAIR = 0x4B4000004B400000ull;

__device__ __forceinline__ unsigned long long fixed_pair(float w, float ur, float ui) {
  const unsigned long long lo = __float_as_uint(fmaf(w, ur, MAGIC));
  const unsigned long long hi = __float_as_uint(fmaf(w, ui, MAGIC));
  return ((hi << 32) | lo) - MAGIC_PAIR;
}

__device__ __forceinline__ void unpack_fixed(unsigned long long w, float& re, float& im) {
  const long long v = (long long)w;
  const int r = (int)(unsigned int)(w & 0xffffffffull);
  const int i = (int)((v - (long long)r) >> 32);
  re = (float)r;
  im = (float)i;
}

// Accumulator tile layout: cubic 16^3 tiles use the bank-split layout of the
// gather tiles (gather_common.h), each lane adding its pixel's taps in its
// slot's rotated order (conflict-free for any pixels); other tiles use the
// padded strides with the lanes ranked by bank key.
template <int NT>
struct AccTile {
  static constexpr bool SPLIT = NT == 4 && TE == 16;
  static constexpr int SIZE = SPLIT ? TLOG : TSIZE;
};

// Accumulator address of logical tile entry idx = x + TE (y + TE z).
template <int NT>
__device__ __forceinline__ int acc_index(int idx) {
  const int x = idx % TE, y = (idx / TE) % TE, z = idx / (TE * TE);
  if constexpr (AccTile<NT>::SPLIT) return split_x(x) + 64 * y + split_z(z);
  else return z * TSZ + y * TSY + x;
}

// The bounds behind the window scales (fixed_point_bound.h): the pixels of
// one pose that can reach a voxel (contrib_bound3) and the sum of |weights|
// a voxel receives from one pose (weight_sum_bound3).
template <int NT>
__device__ __forceinline__ float contrib_bound(const KGeom& g, const float* R) {
  return contrib_bound3<NT>(g.o, R);
}
template <int NT>
__device__ __forceinline__ float weight_sum_bound(const KGeom& g, const float* R) {
  return weight_sum_bound3<NT>(g.o, R);
}

// Poses with a larger bound (degenerate maps) go to the edge kernel.
__device__ __forceinline__ bool pose_ok(float cb) { return cb <= 4096.0f; }

// Hit lists of the back-projection bricks: the slice of pose e reaches the
// box and the map is not degenerate.
template <int NT>
__global__ void __launch_bounds__(256) k_bwd_hit_lists(const float* __restrict__ rot, KGeom g, BrickGrid bg,
                                                       const int* __restrict__ prefix,
                                                       unsigned short* __restrict__ hits, int* __restrict__ counts) {
  build_hit_list(bg, prefix, hits, counts, [&](int vsel, int e, const float* bl, const float* bh) {
    int bimg, n;
    list_entry(g, vsel, e, bimg, n);
    const float* R = rot + 9 * ((int64_t)(g.Br == 1 ? 0 : bimg) * g.P + n);
    return pose_ok(contrib_bound<NT>(g, R)) && slice_meets_box(g, R, bl, bh);
  });
}

// Largest value a pose can put into the brick [bl, bh): the bands of the pixel
// radii |k| in [|p| / sigma_max, |p| / sigma_min] for p in the brick.
__device__ __forceinline__ float box_band_max(const KGeom& g, const BwdGrid& bw, const float* R,
                                              const float* __restrict__ table, int64_t pose, const float bl[3],
                                              const float bh[3]) {
  float g00 = 0.f, g01 = 0.f, g11 = 0.f;
#pragma unroll
  for (int a = 0; a < 3; ++a) {
    const float c0 = g.o * R[3 * a], c1 = g.o * R[3 * a + 1];
    g00 = fmaf(c0, c0, g00); g01 = fmaf(c0, c1, g01); g11 = fmaf(c1, c1, g11);
  }
  const float d = g00 - g11, rt = sqrtf(fmaf(d, d, 4.f * g01 * g01));
  const float smax = sqrtf(fmaxf(0.5f * (g00 + g11 + rt), 0.f)), smin = sqrtf(fmaxf(0.5f * (g00 + g11 - rt), 0.f));
  float dn = 0.f, df = 0.f;
#pragma unroll
  for (int a = 0; a < 3; ++a) {
    const float n = fmaxf(0.f, fmaxf(bl[a], -bh[a]));
    const float f = fmaxf(fabsf(bl[a]), fabsf(bh[a]));
    dn = fmaf(n, n, dn);
    df = fmaf(f, f, df);
  }
  // (the one-pixel margins cover the hardware reciprocal's ulp)
  const float kmin = sqrtf(dn) * __builtin_amdgcn_rcpf(smax) - 1.0f, kmax = sqrtf(df) * __builtin_amdgcn_rcpf(smin) + 1.0f;
  int b0 = (int)fmaxf(0.f, kmin * bw.inv_band_w);
  if (!(kmin == kmin)) b0 = 0;
  const int b1 = (kmax * bw.inv_band_w < (float)bw.nbands) ? (int)(kmax * bw.inv_band_w) : bw.nbands - 1;
  // the first 16 bands of the range as independent loads (one memory round
  // trip instead of one per band); longer ranges finish in a loop
  const float* t = table + pose * bw.nbands;
  float m = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j)
    if (b0 + j <= b1) m = fmaxf(m, t[b0 + j]);
  for (int i = b0 + 16; i <= b1; ++i) m = fmaxf(m, t[i]);
  return m;
}

// Sum of c and maximum of m (m >= 0) over each 32-lane half of the wavefront:
// inclusive DPP scans (row shifts, then the broadcast of lane 15 into rows 1
// and 3) leave lanes 31 and 63 with their half's totals.
__device__ __forceinline__ void half_sum_max(float& c, float& m) {
#define TP_SCAN_STEP(CTRL, RM)                                                      \
  c += __int_as_float(dpp_int<CTRL, RM>(0, __float_as_int(c)));                  \
  m = fmaxf(m, __int_as_float(dpp_int<CTRL, RM>(0, __float_as_int(m))));
  TP_SCAN_STEP(0x111, 0xf)
  TP_SCAN_STEP(0x112, 0xf)
  TP_SCAN_STEP(0x114, 0xf)
  TP_SCAN_STEP(0x118, 0xf)
  TP_SCAN_STEP(0x142, 0xa)
#undef TP_SCAN_STEP
}

__host__ __device__ inline int floor_div(int a, int b) {  // b > 0
  return a >= 0 ? a / b : -((-a + b - 1) / b);
}

}  // namespace

// ---------------------------------------------------------------------------
// Largest |Re|, |Im| (and |Wimg|) of every image per band of pixel radius
// |k| in [bw * i, bw * (i + 1)).
// ---------------------------------------------------------------------------
template <bool WEIGHTS>
__global__ void __launch_bounds__(256) k_band_max(const float2* __restrict__ Y, const float* __restrict__ Wimg,
                                                  float* __restrict__ ymax, float* __restrict__ wmax, KGeom g,
                                                  BwdGrid bw) {
  __shared__ unsigned int bm[MAX_BANDS], bwm[MAX_BANDS];
  for (int bn = blockIdx.x; bn < g.B * g.P; bn += gridDim.x) {
    for (int i = threadIdx.x; i < bw.nbands; i += blockDim.x) { bm[i] = 0u; bwm[i] = 0u; }
    __syncthreads();
    const float2* Yb = Y + (int64_t)bn * g.npix;
    const float* Wb = WEIGHTS ? Wimg + (int64_t)bn * g.npix : nullptr;
    // pixel pix = threadIdx.x + 256 j: its row and column are stepped from the
    // previous ones (no division per pixel); four pixels' loads are issued
    // before their maxima go to LDS
    constexpr int STEP = 256, U = 4;
    const int drow = STEP / g.Wi, dcol = STEP - drow * g.Wi;
    int iy = (int)threadIdx.x / g.Wi, ix = (int)threadIdx.x - iy * g.Wi;
    for (int pix0 = threadIdx.x; pix0 < g.npix; pix0 += U * STEP) {
      float2 v[U];
      float wv[U];
      int band[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int pix = pix0 + u * STEP;
        band[u] = -1;
        if (pix < g.npix) {
          const float kx = (float)ix, ky = (float)(iy < (g.H >> 1) ? iy : iy - g.H);
          if (in_mask(g, kx, ky)) {
            band[u] = min((int)(sqrtf(fmaf(kx, kx, ky * ky)) * bw.inv_band_w), bw.nbands - 1);
            v[u] = Yb[pix];
            if constexpr (WEIGHTS) wv[u] = Wb[pix];
          }
        }
        ix += dcol;
        iy += drow;
        if (ix >= g.Wi) {
          ix -= g.Wi;
          ++iy;
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (band[u] < 0) continue;
        atomicMax(&bm[band[u]], __float_as_uint(fmaxf(fabsf(v[u].x), fabsf(v[u].y))));
        if constexpr (WEIGHTS) atomicMax(&bwm[band[u]], __float_as_uint(fabsf(wv[u])));
      }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < bw.nbands; i += blockDim.x) {
      ymax[(int64_t)bn * bw.nbands + i] = __uint_as_float(bm[i]);
      if constexpr (WEIGHTS) wmax[(int64_t)bn * bw.nbands + i] = __uint_as_float(bwm[i]);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// the brick kernel: the taps of every pixel the brick owns into its LDS tile
// ---------------------------------------------------------------------------
#ifndef BWD_UNROLL
#define BWD_UNROLL 2
#endif
#ifndef BWD_MIN_WAVES
#define BWD_MIN_WAVES 4   // wavefronts per SIMD for the data channel (127 VGPRs, 40 KB LDS)
#endif
#ifndef BWD_MIN_WAVES_W
#define BWD_MIN_WAVES_W 4   // for the weight channel (107 VGPRs; five would spill)
#endif

// The channels of the brick kernel: the complex data (conj(phi) Y into a
// fixed-point pair per tap) or the real weights (Wimg into one fixed-point
// word per tap).  A call with weights runs one launch per channel, so that
// each holds one tile in LDS.
constexpr int CH_DATA = 1, CH_WEIGHTS = 2;

// One pixel, in the lane the bank-spreading permutation gave it (padded
// tiles): pk packs (active, l) with l = floor(p) - lo; f holds the fractional
// parts of p; v is c = conj(phi) Y (data) or (Wimg, 0) (weights).  Adds v
// with the taps' weights to the accumulator tile.
template <int NT, int CH>
__device__ __forceinline__ void bwd_scatter(int pk, float fx, float fy, float fz, float2 v,
                                            unsigned long long* acc_t, unsigned int* acc_w, float scale) {
  if (!(pk & 1)) return;
  const int l[3] = {(pk >> 1) & 15, (pk >> 5) & 15, (pk >> 9) & 15};
  float wx[NT], wy[NT], wz[NT];
  axis_weights<NT>(fx, wx);
  axis_weights<NT>(fy, wy);
  axis_weights<NT>(fz, wz);
  const float cr = v.x * scale, ci = v.y * scale;
#pragma unroll
  for (int jc = 0; jc < NT; ++jc)
#pragma unroll
    for (int jb = 0; jb < NT; ++jb) {
      const float wyz = wy[jb] * wz[jc];
      const float ur = wyz * cr, ui = wyz * ci;
      const int rowb = (l[2] + jc) * TSZ + (l[1] + jb) * TSY + l[0];
#pragma unroll
      for (int ja = 0; ja < NT; ++ja) {
        if constexpr (CH == CH_DATA) atomicAdd(&acc_t[rowb + ja], fixed_pair(wx[ja], ur, ui));
        else atomicAdd(&acc_w[rowb + ja], (unsigned int)fixed_round(wx[ja], ur));
      }
    }
}

// One cubic pixel into a bank-split accumulator tile, in this lane's own tap
// order (SplitTaps): l = floor(p) - lo, f the fractional parts of p, v as
// above.  The y weights are folded into the value once per row, the x and z
// weights once per column.
template <int CH>
__device__ __forceinline__ void bwd_scatter_split(const SplitLut& lut, const int l[3], float fx, float fy, float fz,
                                                  float2 v, unsigned long long* acc_t, unsigned int* acc_w,
                                                  float scale) {
  float wx[4], wy[4], wz[4];
  axis_weights<4>(fx, wx);
  axis_weights<4>(fy, wy);
  axis_weights<4>(fz, wz);
  SplitTaps st;
  split_taps_lut(lut, l, st);   // byte offsets of 8-byte entries
  rotate4(wx, st.t);
  rotate4(wz, st.r);
  const float cr = v.x * scale, ci = v.y * scale;
  // 4-byte weight words: two interleaved copies of the tile, one per 16-lane
  // half of each 32-lane LDS pass, so that the halves use the even and the
  // odd banks (the flush adds the two copies)
  const int half = (((int)threadIdx.x >> 4) & 1) * 4;   // bytes
  float yr[4], yi[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    yr[b] = wy[b] * cr;
    yi[b] = wy[b] * ci;
  }
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const float wxz = wx[a] * wz[c];
      const int col = st.xo[a] + st.zo[c];   // bytes: entry 8 col of the data tile, word pair of the weights
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        if constexpr (CH == CH_DATA)
          atomicAdd(reinterpret_cast<unsigned long long*>(reinterpret_cast<char*>(acc_t) + col) + 64 * b,
                    fixed_pair(wxz, yr[b], yi[b]));
        else
          atomicAdd(reinterpret_cast<unsigned int*>(reinterpret_cast<char*>(acc_w) + col + half) + 128 * b,
                    (unsigned int)fixed_round(wxz, yr[b]));
      }
    }
}

template <int NT, int CH>
__global__ void __launch_bounds__(BTHREADS, CH == CH_DATA ? BWD_MIN_WAVES : BWD_MIN_WAVES_W)
    k_bwd_brick(const float2* __restrict__ Y, const float* __restrict__ Wimg, const float* __restrict__ rot,
                const float* __restrict__ shifts, float2* __restrict__ part_c, float* __restrict__ part_w, KGeom g,
                BwdGrid bw, const int* __restrict__ prefix, const unsigned short* __restrict__ hits,
                const int* __restrict__ counts, const float* __restrict__ vmax) {
  constexpr bool DATA = CH == CH_DATA;
  constexpr bool SPLIT = AccTile<NT>::SPLIT;
  constexpr int ASIZE = AccTile<NT>::SIZE;
  const BrickGrid& bg = bw.bg;
  constexpr int WSIZE = SPLIT ? 2 * ASIZE : ASIZE;   // bank-split weight tiles: two copies
  __shared__ unsigned long long acc_t[DATA ? ASIZE : 1];
  __shared__ unsigned int acc_w[DATA ? 1 : WSIZE];
  __shared__ EnumShared<WINDOW, BNW> es;
  __shared__ float win_scale[SCALE_BATCH];
  __shared__ std::conditional_t<SPLIT, SplitLut, char> lut;   // tap tables of the bank-split tile

  const int w = blockIdx.x, vsel = blockIdx.y;
  if (w >= bg.nwork) return;
  const int nh = counts[(int64_t)vsel * bg.nwork + w];
  const int b = find_brick(prefix, bg.nb3, w);
  int e0, e1;
  item_chunk(bg, prefix, b, w, e0, e1);
  const unsigned short* hl = hits + hit_slot(bg, prefix, vsel, b, e0);
  int bi, bj, bk;
  brick_coords(bg, b, bi, bj, bk);
  const int lo[3] = {bg.origin + bi * bg.S, bg.origin + bj * bg.S, bg.origin + bk * bg.S};
  const float bl[3] = {(float)lo[0], (float)lo[1], (float)lo[2]};
  const float bh[3] = {(float)(lo[0] + bg.S), (float)(lo[1] + bg.S), (float)(lo[2] + bg.S)};
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t slot0 = ((int64_t)vsel * bg.nwork + w) * TLOG;
  if (nh == 0) {
    // no hits: the partial tile is zero (the fold reads every slot)
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) {
      if (TLOG % BTHREADS != 0 && tid + BTHREADS * i >= TLOG) break;
      if constexpr (DATA) part_c[slot0 + tid + BTHREADS * i] = make_float2(0.f, 0.f);
      else part_w[slot0 + tid + BTHREADS * i] = 0.f;
    }
    return;
  }

  float2 acc[PER_LANE];
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) acc[i] = make_float2(0.f, 0.f);
  for (int i = tid; i < (DATA ? ASIZE : WSIZE); i += BTHREADS) {
    if constexpr (DATA) acc_t[i] = 0ull;
    else acc_w[i] = 0u;
  }
  if constexpr (SPLIT) split_lut_fill(lut);
  __syncthreads();

  {
    for (int hb = 0; hb < nh; hb += WINDOW) {
      const int nw = min(WINDOW, nh - hb);
      const int wslot = (hb / WINDOW) % SCALE_BATCH;
      if (wslot == 0) {
        // the fixed-point scales of the next SCALE_BATCH windows, one hit per
        // thread: every hit's bound on the contributions to one tap and the
        // largest value it can bring to this brick, summed and maximised over
        // each window's 32 hits (a half wavefront)
        const int i = hb + tid;
        float c = 0.f, m = 0.f;
        if (i < nh) {
          int bimg, n;
          list_entry(g, vsel, e0 + (int)hl[i], bimg, n);
          const float* Rg = rot + 9 * ((int64_t)(g.Br == 1 ? 0 : bimg) * g.P + n);
          float R[9];
#pragma unroll
          for (int a = 0; a < 9; ++a) R[a] = Rg[a];
          c = weight_sum_bound<NT>(g, R);
          m = box_band_max(g, bw, R, vmax, (int64_t)bimg * g.P + n, bl, bh);
        }
        half_sum_max(c, m);
        if ((lane & 31) == 31 && i - 31 < nh) {
          // data: |re|, |im| <= sqrt(2) M per unit weight (the phase
          // rotates), so no sum exceeds lim; every single contribution (weight
          // <= 1) also stays below 2^22 for the magic rounding; the 10 %
          // headroom of FIX_RANGE absorbs the rounding of the window's at most
          // a few thousand contributions per tap
          const float lim = fminf(FIX_RANGE, 0.99f * 4194304.0f * c);
          win_scale[tid >> 5] = m > 0.f ? lim / ((DATA ? 1.41421356f : 1.0f) * m * c) : 0.f;
        }
        // (window_setup's closing barrier publishes the scales)
      }
      window_setup(es, g, rot, DATA ? shifts : nullptr, vsel, e0, hl + hb, nw, bl, bh);
      const float scale = win_scale[wslot];
      const int nrows = es.hrow[nw];
      for (int qb = 0; qb < nrows;) {
        int nr;
        const int ncand = row_stage(es, g, qb, nrows, nw, bl, bh, nr);
        for (int c0 = wave * 64; c0 < ncand; c0 += BWD_UNROLL * BTHREADS) {   // wave-uniform (lane permutes)
          constexpr int U = BWD_UNROLL;
          int mpk[U];
          float mf[U][3];
          float2 mv[U], mph[U];
          // look up each pixel and issue its load (and, for padded tiles, move
          // it to its bank-spreading lane) ...
#pragma unroll
          for (int u = 0; u < U; ++u) {
            Cand cu;
            cand_prep(es, g, c0 + u * BTHREADS + lane, ncand, lo, bg.S, cu);
            // every candidate's element index is in range (0 past the
            // stage's end), so the load needs no branch: the tap code then
            // waits for this pixel's value only, not for the next one's
            float2 v = make_float2(0.f, 0.f), ph = make_float2(1.f, 0.f);
            if constexpr (DATA) v = Y[cu.k];
            else v.x = Wimg[cu.k];
            float f[3] = {0.f, 0.f, 0.f};
            int pk = 0, key = -1;
            if (cu.act) {
              if (DATA && shifts) ph = shift_phase(cu.kx, cu.ky, cu.sx, cu.sy, g.inv_h);
#pragma unroll
              for (int a = 0; a < 3; ++a) f[a] = frac_of(cu.p[a]);
              pk = 1 | (cu.l[0] << 1) | (cu.l[1] << 5) | (cu.l[2] << 9);
              key = (cu.l[0] + cu.l[1] * TSY + cu.l[2] * TSZ) & 15;
            }
            if constexpr (SPLIT) {
              // the phase is applied when the taps need the value, so that the
              // next pixel's lookup and load overlap this one's memory latency
              mpk[u] = pk;
#pragma unroll
              for (int a = 0; a < 3; ++a) mf[u][a] = f[a];
              mv[u] = v;
              mph[u] = ph;
            } else {
              if (DATA && shifts) v = cmulc(ph, v);   // conj(phi) * Y
              const int dest = spread_dest(key);
              mpk[u] = lane_send(pk, dest);
#pragma unroll
              for (int a = 0; a < 3; ++a) mf[u][a] = lane_send(f[a], dest);
              mv[u].x = lane_send(v.x, dest);
              mv[u].y = DATA ? lane_send(v.y, dest) : 0.f;
            }
          }
          // ... then all the taps (nothing waits on these atomics)
#pragma unroll
          for (int u = 0; u < U; ++u) {
            if constexpr (SPLIT) {
              if (mpk[u] & 1) {
                const int l[3] = {(mpk[u] >> 1) & 15, (mpk[u] >> 5) & 15, (mpk[u] >> 9) & 15};
                const float2 v = DATA && shifts ? cmulc(mph[u], mv[u]) : mv[u];   // conj(phi) * Y
                bwd_scatter_split<CH>(lut, l, mf[u][0], mf[u][1], mf[u][2], v, acc_t, acc_w, scale);
              }
            } else {
              bwd_scatter<NT, CH>(mpk[u], mf[u][0], mf[u][1], mf[u][2], mv[u], acc_t, acc_w, scale);
            }
          }
        }
        __syncthreads();
        qb += nr;
      }
      // ---- flush the window into the float accumulators ----
      const float inv = scale > 0.f ? 1.0f / scale : 0.f;
#pragma unroll
      for (int i = 0; i < PER_LANE; ++i) {
        if (TLOG % BTHREADS != 0 && tid + BTHREADS * i >= TLOG) break;
        const int pi = acc_index<NT>(tid + BTHREADS * i);
        if constexpr (DATA) {
          const unsigned long long v = acc_t[pi];
          if (v != 0ull) {
            float re, im;
            unpack_fixed(v, re, im);
            acc[i].x = fmaf(re, inv, acc[i].x);
            acc[i].y = fmaf(im, inv, acc[i].y);
            acc_t[pi] = 0ull;
          }
        } else if constexpr (SPLIT) {
          const unsigned int u0 = acc_w[2 * pi], u1 = acc_w[2 * pi + 1];
          if ((u0 | u1) != 0u) {
            acc[i].x = fmaf((float)((int)u0 + (int)u1), inv, acc[i].x);
            acc_w[2 * pi] = 0u;
            acc_w[2 * pi + 1] = 0u;
          }
        } else {
          const unsigned int u = acc_w[pi];
          if (u != 0u) {
            acc[i].x = fmaf((float)(int)u, inv, acc[i].x);
            acc_w[pi] = 0u;
          }
        }
      }
      __syncthreads();
    }
  }

  // ---- this work item's partial tile (tap space, logical order) ----
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) {
    if (TLOG % BTHREADS != 0 && tid + BTHREADS * i >= TLOG) break;
    if constexpr (DATA) part_c[slot0 + tid + BTHREADS * i] = acc[i];
    else part_w[slot0 + tid + BTHREADS * i] = acc[i].x;
  }
}

// ---------------------------------------------------------------------------
// Every brick's chunks (work items) wrote partial tiles of the same tap
// region; this pass sums them, in chunk order, into the first chunk's tile,
// so that the fold reads one tile per brick.  One workgroup per (brick, 256
// tile entries); bricks with fewer than two chunks have nothing to do.
// ---------------------------------------------------------------------------
constexpr int REDUCE_BLOCKS = (TLOG + 255) / 256;   // entry blocks per brick

template <bool WEIGHTS>
__global__ void __launch_bounds__(256) k_bwd_reduce(float2* __restrict__ part_c, float* __restrict__ part_w,
                                                    BrickGrid bg, const int* __restrict__ prefix) {
  const int b = blockIdx.x / REDUCE_BLOCKS, vsel = blockIdx.y;
  const int k0 = prefix[b], k1 = prefix[b + 1];
  if (k1 - k0 < 2) return;
  const int64_t e = (int64_t)(blockIdx.x % REDUCE_BLOCKS) * 256 + threadIdx.x;
  if (e >= TLOG) return;
  float2* pc = part_c + (int64_t)vsel * bg.nwork * TLOG;
  float* pw = WEIGHTS ? part_w + (int64_t)vsel * bg.nwork * TLOG : nullptr;
  float2 s = make_float2(0.f, 0.f);
  float sw = 0.f;
  // four chunks at a time, so that several loads are in flight
  int c = k0;
  for (; c + 4 <= k1; c += 4) {
    float2 t[4];
    float tw[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      t[j] = pc[(int64_t)(c + j) * TLOG + e];
      if constexpr (WEIGHTS) tw[j] = pw[(int64_t)(c + j) * TLOG + e];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      s.x += t[j].x;
      s.y += t[j].y;
      if constexpr (WEIGHTS) sw += tw[j];
    }
  }
  for (; c < k1; ++c) {
    const float2 t = pc[(int64_t)c * TLOG + e];
    s.x += t.x;
    s.y += t.y;
    if constexpr (WEIGHTS) sw += pw[(int64_t)c * TLOG + e];
  }
  pc[(int64_t)k0 * TLOG + e] = s;
  if constexpr (WEIGHTS) pw[(int64_t)k0 * TLOG + e] = sw;
}

// ---------------------------------------------------------------------------
// Fold: every stored voxel sums the tile entries of all its tap-space
// preimages -- direct copies (x, y, z) + D j and, for 1 <= x <= D/2 - 1, the
// conjugated Friedel mates (-x, -y, -z) + D j -- over every brick tile and
// chunk that holds them, in a fixed order.
// ---------------------------------------------------------------------------
template <int NT, bool WEIGHTS>
__global__ void __launch_bounds__(256) k_bwd_fold(float2* __restrict__ vol, float* __restrict__ wvol,
                                                  const float2* __restrict__ part_c, const float* __restrict__ part_w,
                                                  KGeom g, BwdGrid bw, const int* __restrict__ prefix, bool reduced) {
  const BrickGrid& bg = bw.bg;
  constexpr int HL = NT == 4 ? 1 : 0;
  constexpr int SB = TE - NT + 1;   // brick edge (bg.S)
  const int nvol = g.D * g.D * g.W;
  const int vsel = blockIdx.y;
  const int tlo = bg.origin - HL, thi = bg.origin + (bg.nb - 1) * SB - HL + TE - 1;   // covered taps
  const float2* pc = part_c + (int64_t)vsel * bg.nwork * TLOG;
  const float* pw = WEIGHTS ? part_w + (int64_t)vsel * bg.nwork * TLOG : nullptr;
  for (int v = blockIdx.x * blockDim.x + threadIdx.x; v < nvol; v += gridDim.x * blockDim.x) {
    const int xy = v % (g.W * g.D), z = v / (g.W * g.D);
    const int x = xy % g.W, y = xy / g.W;
    float2 a = make_float2(0.f, 0.f);
    float aw = 0.f;
    for (int kind = 0; kind < 2; ++kind) {
      if (kind == 1 && !(x >= 1 && x <= g.half - 1)) break;
      const int sx = kind ? -x : x, sy = kind ? -y : y, sz = kind ? -z : z;
      float2 part = make_float2(0.f, 0.f);
      float partw = 0.f;
      for (int tz = sz + g.D * floor_div(tlo - sz + g.D - 1, g.D); tz <= thi; tz += g.D) {
        const int iz0 = max(0, floor_div(tz - bg.origin + HL - TE, SB) + 1), iz1 = min(bg.nb - 1, floor_div(tz - bg.origin + HL, SB));
        for (int ty = sy + g.D * floor_div(tlo - sy + g.D - 1, g.D); ty <= thi; ty += g.D) {
          const int iy0 = max(0, floor_div(ty - bg.origin + HL - TE, SB) + 1), iy1 = min(bg.nb - 1, floor_div(ty - bg.origin + HL, SB));
          for (int tx = sx + g.D * floor_div(tlo - sx + g.D - 1, g.D); tx <= thi; tx += g.D) {
            const int ix0 = max(0, floor_div(tx - bg.origin + HL - TE, SB) + 1), ix1 = min(bg.nb - 1, floor_div(tx - bg.origin + HL, SB));
            for (int iz = iz0; iz <= iz1; ++iz)
              for (int iy = iy0; iy <= iy1; ++iy)
                for (int ix = ix0; ix <= ix1; ++ix) {
                  const int bb = (iz * bg.nb + iy) * bg.nb + ix;
                  const int k0 = prefix[bb], k1 = reduced ? min(prefix[bb + 1], k0 + 1) : prefix[bb + 1];
                  const int lx = tx - (bg.origin + ix * SB - HL), ly = ty - (bg.origin + iy * SB - HL),
                            lz = tz - (bg.origin + iz * SB - HL);
                  const int64_t li = (int64_t)lz * (TE * TE) + ly * TE + lx;
                  // four chunks at a time, so that several loads are in flight
                  int c = k0;
                  for (; c + 4 <= k1; c += 4) {
                    float2 t[4];
                    float tw[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                      t[j] = pc[(int64_t)(c + j) * TLOG + li];
                      if constexpr (WEIGHTS) tw[j] = pw[(int64_t)(c + j) * TLOG + li];
                    }
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                      part.x += t[j].x;
                      part.y += t[j].y;
                      if constexpr (WEIGHTS) partw += tw[j];
                    }
                  }
                  for (; c < k1; ++c) {
                    const float2 t = pc[(int64_t)c * TLOG + li];
                    part.x += t.x;
                    part.y += t.y;
                    if constexpr (WEIGHTS) partw += pw[(int64_t)c * TLOG + li];
                  }
                }
          }
        }
      }
      a.x += part.x;
      a.y += kind ? -part.y : part.y;
      aw += partw;
    }
    vol[(int64_t)nvol * vsel + v] = a;
    if constexpr (WEIGHTS) wvol[(int64_t)nvol * vsel + v] = aw;
  }
}

// ---------------------------------------------------------------------------
// The same fold driven by a per-axis table.  All three axes share one brick
// grid and the period D, so the tap-space preimages of a voxel factor into
// per-axis lists: for every coordinate c in [0, D), the (brick index, tile
// offset) pairs of the taps t = c (mod D) that some brick's tile holds,
// translates ascending, bricks ascending.  Each workgroup builds the table in
// LDS (D x FOLD_K entries); a voxel then walks the product of its three lists
// (Friedel mates: the lists of -x, -y, -z) with no division in the loop.
// Used when no coordinate has more than FOLD_K pairs (the launcher checks).
// ---------------------------------------------------------------------------
constexpr int FOLD_K = 8;

template <int NT, bool WEIGHTS>
__global__ void __launch_bounds__(256) k_bwd_fold_map(float2* __restrict__ vol, float* __restrict__ wvol,
                                                      const float2* __restrict__ part_c,
                                                      const float* __restrict__ part_w, KGeom g, BwdGrid bw,
                                                      const int* __restrict__ prefix, bool reduced) {
  extern __shared__ unsigned short fmap[];   // [D][FOLD_K] entries brick * 16 + offset, then [D] counts
  unsigned short* fcnt = fmap + g.D * FOLD_K;
  const BrickGrid& bg = bw.bg;
  constexpr int HL = NT == 4 ? 1 : 0;
  constexpr int SB = TE - NT + 1;   // brick edge (bg.S)
  const int tlo = bg.origin - HL, thi = bg.origin + (bg.nb - 1) * SB - HL + TE - 1;   // covered taps
  for (int c = threadIdx.x; c < g.D; c += blockDim.x) {
    int n = 0;
    for (int t = c + g.D * floor_div(tlo - c + g.D - 1, g.D); t <= thi; t += g.D) {
      const int i0 = max(0, floor_div(t - bg.origin + HL - TE, SB) + 1), i1 = min(bg.nb - 1, floor_div(t - bg.origin + HL, SB));
      for (int i = i0; i <= i1 && n < FOLD_K; ++i)
        fmap[c * FOLD_K + n++] = (unsigned short)(i * 16 + (t - (bg.origin + i * SB - HL)));
    }
    fcnt[c] = (unsigned short)n;
  }
  __syncthreads();
  const int nvol = g.D * g.D * g.W;
  const int vsel = blockIdx.y;
  const float2* pc = part_c + (int64_t)vsel * bg.nwork * TLOG;
  const float* pw = WEIGHTS ? part_w + (int64_t)vsel * bg.nwork * TLOG : nullptr;
  for (int v = blockIdx.x * blockDim.x + threadIdx.x; v < nvol; v += gridDim.x * blockDim.x) {
    const int xy = v % (g.W * g.D), z = v / (g.W * g.D);
    const int x = xy % g.W, y = xy / g.W;
    float2 a = make_float2(0.f, 0.f);
    float aw = 0.f;
    for (int kind = 0; kind < 2; ++kind) {
      if (kind == 1 && !(x >= 1 && x <= g.half - 1)) break;
      const int cx = kind ? g.D - x : x, cy = kind ? (g.D - y) % g.D : y, cz = kind ? (g.D - z) % g.D : z;
      const unsigned short* mx = fmap + cx * FOLD_K;
      const unsigned short* my = fmap + cy * FOLD_K;
      const unsigned short* mz = fmap + cz * FOLD_K;
      const int nx = fcnt[cx], ny = fcnt[cy], nz = fcnt[cz];
      float2 part = make_float2(0.f, 0.f);
      float partw = 0.f;
      for (int jz = 0; jz < nz; ++jz) {
        const int ez = mz[jz];
        for (int jy = 0; jy < ny; ++jy) {
          const int ey = my[jy];
          const int bzy = ((ez >> 4) * bg.nb + (ey >> 4)) * bg.nb;
          const int lzy = (ez & 15) * (TE * TE) + (ey & 15) * TE;
          for (int jx = 0; jx < nx; ++jx) {
            const int ex = mx[jx];
            const int bb = bzy + (ex >> 4);
            const int k0 = prefix[bb], k1 = reduced ? min(prefix[bb + 1], k0 + 1) : prefix[bb + 1];
            const int64_t li = lzy + (ex & 15);
            // four chunks at a time, so that several loads are in flight
            int c = k0;
            for (; c + 4 <= k1; c += 4) {
              float2 t[4];
              float tw[4];
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                t[j] = pc[(int64_t)(c + j) * TLOG + li];
                if constexpr (WEIGHTS) tw[j] = pw[(int64_t)(c + j) * TLOG + li];
              }
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                part.x += t[j].x;
                part.y += t[j].y;
                if constexpr (WEIGHTS) partw += tw[j];
              }
            }
            for (; c < k1; ++c) {
              const float2 t = pc[(int64_t)c * TLOG + li];
              part.x += t.x;
              part.y += t.y;
              if constexpr (WEIGHTS) partw += pw[(int64_t)c * TLOG + li];
            }
          }
        }
      }
      a.x += part.x;
      a.y += kind ? -part.y : part.y;
      aw += partw;
    }
    vol[(int64_t)nvol * vsel + v] = a;
    if constexpr (WEIGHTS) wvol[(int64_t)nvol * vsel + v] = aw;
  }
}

// ---------------------------------------------------------------------------
// Pixels the bricks do not serve (degenerate maps, samples outside every
// active brick): their taps with global atomics, after the fold.  One
// workgroup per pose; a pose served whole by the bricks is skipped.
// ---------------------------------------------------------------------------
template <int NT, bool WEIGHTS>
__global__ void __launch_bounds__(256) k_bwd_edge(const float2* __restrict__ Y, const float* __restrict__ Wimg,
                                                  const float* __restrict__ rot, const float* __restrict__ shifts,
                                                  float2* __restrict__ vol, float* __restrict__ wvol, KGeom g,
                                                  BwdGrid bw) {
  const BrickGrid& bg = bw.bg;
  const int64_t nvol = (int64_t)g.D * g.D * g.W;
  for (int bn = blockIdx.x; bn < g.B * g.P; bn += gridDim.x) {
    const int bimg = bn / g.P, n = bn - bimg * g.P;
    const float* R = rot + 9 * ((int64_t)(g.Br == 1 ? 0 : bimg) * g.P + n);
    const bool ok = pose_ok(contrib_bound<NT>(g, R));
    if (ok && pose_pmax(g, R) <= 0.9995f * (float)bg.pmax_i) continue;
    for (PixelWalk pw(g, threadIdx.x, blockDim.x); pw.pix < g.npix; pw.step(g, blockDim.x)) {
      const int pix = pw.pix;
      const float kx = (float)pw.kx(), ky = (float)pw.ky(g);
      if (!in_mask(g, kx, ky)) continue;
      float p[3];
      slice_coord(g, R, kx, ky, p);
      if (ok && served_by_bricks(bg, p)) continue;
      float2 c = Y[(int64_t)bn * g.npix + pix];
      if (shifts) {
        const float* s = shifts + 2 * ((int64_t)(g.Bs == 1 ? 0 : bimg) * g.P + n);
        c = cmulc(shift_phase(kx, ky, s[0], s[1], g.inv_h), c);   // conj(phi) * Y
      }
      const float wimg = WEIGHTS ? Wimg[(int64_t)bn * g.npix + pix] : 0.f;
      float2* V = vol + nvol * (g.Bv == 1 ? 0 : bimg);
      float* VW = WEIGHTS ? wvol + nvol * (g.Bv == 1 ? 0 : bimg) : nullptr;
      const float flx = safe_floor(p[0]), fly = safe_floor(p[1]), flz = safe_floor(p[2]);
      float wx[NT], wy[NT], wz[NT];
      axis_weights<NT>(p[0] - flx, wx);
      axis_weights<NT>(p[1] - fly, wy);
      axis_weights<NT>(p[2] - flz, wz);
      const int x0 = (int)flx + first_tap<NT>(), y0 = (int)fly + first_tap<NT>(), z0 = (int)flz + first_tap<NT>();
      for (int cc = 0; cc < NT; ++cc)
        for (int bb = 0; bb < NT; ++bb)
          for (int aa = 0; aa < NT; ++aa) {
            bool cj;
            const int64_t idx = tap_index<true>(g, x0 + aa, y0 + bb, z0 + cc, cj);
            const float wt = wx[aa] * wy[bb] * wz[cc];
            float* dst = reinterpret_cast<float*>(V + idx);
            unsafeAtomicAdd(dst, wt * c.x);
            unsafeAtomicAdd(dst + 1, cj ? -wt * c.y : wt * c.y);
            if constexpr (WEIGHTS) unsafeAtomicAdd(VW + idx, wt * wimg);
          }
    }
  }
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------
static size_t align256(size_t n) { return (n + 255) / 256 * 256; }

int bwd_brick_edge(int interp) { return TE - (interp == 1 ? 4 : 2) + 1; }

// Does every coordinate of the per-axis fold table hold at most FOLD_K
// (brick, offset) pairs?  (The same count k_bwd_fold_map's table makes.)
static bool fold_table_fits(const KGeom& g, const BwdGrid& bw, int interp) {
  const BrickGrid& bg = bw.bg;
  const int NT = interp == 1 ? 4 : 2, HL = interp == 1 ? 1 : 0, SB = TE - NT + 1;
  if (bg.S != SB || g.D > 4096) return false;
  const int tlo = bg.origin - HL, thi = bg.origin + (bg.nb - 1) * SB - HL + TE - 1;
  for (int c = 0; c < g.D; ++c) {
    int n = 0;
    for (int t = c + g.D * floor_div(tlo - c + g.D - 1, g.D); t <= thi; t += g.D) {
      const int i0 = std::max(0, floor_div(t - bg.origin + HL - TE, SB) + 1);
      const int i1 = std::min(bg.nb - 1, floor_div(t - bg.origin + HL, SB));
      n += i1 >= i0 ? i1 - i0 + 1 : 0;
    }
    if (n > FOLD_K) return false;
  }
  return true;
}

size_t bwd_ws_bytes(const BwdGrid& bw, int Bv, bool weights) {
  const size_t work = brick_work_bytes(bw.bg, Bv);
  const size_t bands = align256((size_t)bw.npose * bw.nbands * sizeof(float) * (weights ? 2 : 1));
  const size_t parts = (size_t)bw.bg.nwork * Bv * TLOG * (sizeof(float2) + (weights ? sizeof(float) : 0));
  return work + bands + parts;
}

hipError_t launch_bwd(const KGeom& g, int interp, const BwdGrid& bw, void* workspace, const float2* Y,
                      const float* Wimg, const float* rot, const float* shifts, float2* vol, float* wvol,
                      hipStream_t st, const EvPair* ev_brick, const EvPair* ev_fold, const SideRef* side) {
  const bool weights = Wimg != nullptr;
  const BrickWork wk = brick_work(bw.bg, g.Bv, workspace);
  int* prefix = wk.prefix;
  const size_t off_b = brick_work_bytes(bw.bg, g.Bv);
  float* ymax = (float*)((char*)workspace + off_b);
  float* wmax = ymax + (size_t)bw.npose * bw.nbands;
  const size_t off_p = off_b + align256((size_t)bw.npose * bw.nbands * sizeof(float) * (weights ? 2 : 1));
  float2* part_c = (float2*)((char*)workspace + off_p);
  float* part_w = (float*)(part_c + (size_t)bw.bg.nwork * g.Bv * TLOG);
  hipError_t e = hipSuccess;
  // the band maxima read only the images: on the side stream they overlap the
  // work list and the hit lists (HBM-bound beside latency-bound work)
  hipStream_t sb = st;
  if (side) {
    e = hipEventRecord(side->fork, st);
    if (e == hipSuccess) e = hipStreamWaitEvent(side->s, side->fork, 0);
    if (e != hipSuccess) return e;
    sb = side->s;
  }
  const int nb = bw.npose < 65535 ? bw.npose : 65535;
  if (weights) hipLaunchKernelGGL((k_band_max<true>), dim3(nb), dim3(256), 0, sb, Y, Wimg, ymax, wmax, g, bw);
  else hipLaunchKernelGGL((k_band_max<false>), dim3(nb), dim3(256), 0, sb, Y, Wimg, ymax, wmax, g, bw);
  e = hipGetLastError();
  if (e == hipSuccess && side) e = hipEventRecord(side->join, side->s);
  if (e != hipSuccess) return e;
  e = launch_brick_prefix(bw.bg, prefix, st);
  if (e != hipSuccess) return e;
  if (bw.bg.nwork > 0) {
    const dim3 grid(bw.bg.nwork, g.Bv);
    if (interp == 1) hipLaunchKernelGGL((k_bwd_hit_lists<4>), grid, dim3(256), 0, st, rot, g, bw.bg, prefix, wk.hits, wk.counts);
    else hipLaunchKernelGGL((k_bwd_hit_lists<2>), grid, dim3(256), 0, st, rot, g, bw.bg, prefix, wk.hits, wk.counts);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (side) {
    e = hipStreamWaitEvent(st, side->join, 0);
    if (e != hipSuccess) return e;
  }
  const dim3 blk(256);
  ev_begin(ev_brick, st);   // recorded even when no brick kernel runs
  if (bw.bg.nwork > 0) {
    const dim3 grid(bw.bg.nwork, g.Bv);
#define TP_BWD(NT_, CH_, VMAX)                                                                              \
  hipLaunchKernelGGL((k_bwd_brick<NT_, CH_>), grid, dim3(BTHREADS), 0, st, Y, Wimg, rot, shifts, part_c, part_w, g, \
                     bw, prefix, wk.hits, wk.counts, VMAX)
    // the data channel, then (with weights) the weight channel
    if (interp == 1) {
      TP_BWD(4, CH_DATA, ymax);
      if (weights) TP_BWD(4, CH_WEIGHTS, wmax);
    } else {
      TP_BWD(2, CH_DATA, ymax);
      if (weights) TP_BWD(2, CH_WEIGHTS, wmax);
    }
    e = hipGetLastError();
#undef TP_BWD
  }
  ev_end(ev_brick, st);
  if (e != hipSuccess) return e;
  {
    const int64_t nvol = (int64_t)g.D * g.D * g.W;
    const int blocks = (int)((nvol + 255) / 256 < 8192 ? (nvol + 255) / 256 : 8192);
    const dim3 fg(blocks, g.Bv);
    ev_begin(ev_fold, st);
    // with two or more chunks per active brick on average, sum each brick's
    // chunks first (the fold then reads one tile per brick); with fewer the
    // pass costs more than it saves (measured: D=128 step fold 0.27 -> 0.21 ms,
    // D=256 weighted back-projection with mostly single-chunk bricks 5.41 ->
    // 5.59 ms when always run)
    const bool reduced = bw.bg.nwork >= 2 * bw.bg.nactive;
    if (reduced) {
      const dim3 rg(bw.bg.nb3 * REDUCE_BLOCKS, g.Bv);
      if (weights) hipLaunchKernelGGL((k_bwd_reduce<true>), rg, blk, 0, st, part_c, part_w, bw.bg, prefix);
      else hipLaunchKernelGGL((k_bwd_reduce<false>), rg, blk, 0, st, part_c, part_w, bw.bg, prefix);
    }
    if (fold_table_fits(g, bw, interp)) {
      const size_t shm = (size_t)g.D * (FOLD_K + 1) * sizeof(unsigned short);
      if (interp == 1) {
        if (weights) hipLaunchKernelGGL((k_bwd_fold_map<4, true>), fg, blk, shm, st, vol, wvol, part_c, part_w, g, bw, prefix, reduced);
        else hipLaunchKernelGGL((k_bwd_fold_map<4, false>), fg, blk, shm, st, vol, wvol, part_c, part_w, g, bw, prefix, reduced);
      } else {
        if (weights) hipLaunchKernelGGL((k_bwd_fold_map<2, true>), fg, blk, shm, st, vol, wvol, part_c, part_w, g, bw, prefix, reduced);
        else hipLaunchKernelGGL((k_bwd_fold_map<2, false>), fg, blk, shm, st, vol, wvol, part_c, part_w, g, bw, prefix, reduced);
      }
    } else if (interp == 1) {
      if (weights) hipLaunchKernelGGL((k_bwd_fold<4, true>), fg, blk, 0, st, vol, wvol, part_c, part_w, g, bw, prefix, reduced);
      else hipLaunchKernelGGL((k_bwd_fold<4, false>), fg, blk, 0, st, vol, wvol, part_c, part_w, g, bw, prefix, reduced);
    } else {
      if (weights) hipLaunchKernelGGL((k_bwd_fold<2, true>), fg, blk, 0, st, vol, wvol, part_c, part_w, g, bw, prefix, reduced);
      else hipLaunchKernelGGL((k_bwd_fold<2, false>), fg, blk, 0, st, vol, wvol, part_c, part_w, g, bw, prefix, reduced);
    }
    ev_end(ev_fold, st);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 eg(g.B * g.P < 16384 ? g.B * g.P : 16384);   // one workgroup per pose
  if (interp == 1) {
    if (weights) hipLaunchKernelGGL((k_bwd_edge<4, true>), eg, blk, 0, st, Y, Wimg, rot, shifts, vol, wvol, g, bw);
    else hipLaunchKernelGGL((k_bwd_edge<4, false>), eg, blk, 0, st, Y, Wimg, rot, shifts, vol, wvol, g, bw);
  } else {
    if (weights) hipLaunchKernelGGL((k_bwd_edge<2, true>), eg, blk, 0, st, Y, Wimg, rot, shifts, vol, wvol, g, bw);
    else hipLaunchKernelGGL((k_bwd_edge<2, false>), eg, blk, 0, st, Y, Wimg, rot, shifts, vol, wvol, g, bw);
  }
  return hipGetLastError();
}

}  // namespace tproj
