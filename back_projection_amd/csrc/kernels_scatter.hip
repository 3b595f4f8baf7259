// Brick-owned adjoint scatter (2D->3D back-projection and the volume gradient
// of the forward) for gfx950.
//
// The back-projection is the exact adjoint of the rotated-central-slice
// forward: every in-mask pixel adds w * conj(phi) * Y to each of its taps
// (conjugated where the tap is a Friedel mate) and w * Wimg to the weight
// volume (French page, "Resume technique" 2: accumulation with weights for CTF
// correction; Dutch page, Methodologie: Friedel symmetry).
//
// A workgroup owns one S^3 brick of the stored volume for a chunk of the pose
// list.  For every preimage box of the brick in tap space it detects the poses
// whose slice crosses the box (256 poses at a time, one per lane), enumerates
// the pixels that reach the box, and adds their in-box taps into an LDS tile.
// Floating-point atomics in LDS are slow on this GPU while 64-bit integer ones
// are not, so the tile holds fixed-point integers: re and im of a tap share one
// 64-bit word (im * 2^32 + re), added with a single ds_add_u64.  Taps are
// accumulated in windows of up to 16 poses; a first pass over the window
// finds the largest |value| and a bound on the contributions per voxel, which
// fix a scale that cannot overflow 31 bits; after the window the tile is
// decoded into float registers and cleared.  Integer sums do not depend on the
// order of the atomics, so the result is deterministic.
#include "device_common.h"
#include "gather_common.h"
#include "scatter_grid.h"
#include "scatter_kernels.h"

namespace tproj {

namespace {

constexpr int SB = 16;                     // stored brick edge
constexpr int TSY = 17;                    // tile row stride (u64 entries)
constexpr int TSZ = 16 * 17 + 8;           // tile plane stride
constexpr int TSIZE = SB * TSZ;            // 4480 entries
constexpr int TGUARD = 4;                  // guard entries below index 0
constexpr int PER_LANE = (TSIZE + 255) / 256;
constexpr int WINDOW = 16;                 // poses per fixed-point window
constexpr float FIX_RANGE = 0.9f * 2147483648.0f;
constexpr int MAX_BANDS = 128;

// Copies of a stored interval [lo, hi) in tap space.  Direct: t = s + D j;
// mirrored: t = D j - s.  Each copy is clipped to the tap range [tmin, tmax].
struct AxisCopies {
  int n;
  int qlo[5], qhi[5], add[5];   // local = sgn * t + add
};

__device__ __forceinline__ void axis_copies(int lo, int hi, int brick_lo, int D, int tmin, int tmax, bool mirror,
                                            AxisCopies& c) {
  c.n = 0;
  if (lo >= hi) return;
  for (int j = -2; j <= 2; ++j) {
    int a, b, add;
    if (!mirror) { a = lo + D * j; b = hi + D * j; add = -(D * j) - brick_lo; }
    else { a = D * j - hi + 1; b = D * j - lo + 1; add = D * j - brick_lo; }
    a = max(a, tmin);
    b = min(b, tmax + 1);
    if (a < b) { c.qlo[c.n] = a; c.qhi[c.n] = b; c.add[c.n] = add; ++c.n; }
  }
}

struct TBox {
  int qlo[3], qhi[3], add[3];
  int sgn;
};

// Bound on the pixels of one pose that can reach one voxel: the voxel's
// support box (edge NT) cuts the slice in a disc of radius NT*sqrt(3)/2 in
// sample space, i.e. an ellipse in pixel space whose semi-axes are that radius
// over the singular values of A = o [R_:0 R_:1]; (2a+1)^2 bounds its pixels.
template <int NT>
__device__ __forceinline__ float contrib_bound(const KGeom& g, const float* R) {
  float g00 = 0.f, g01 = 0.f, g11 = 0.f;
#pragma unroll
  for (int a = 0; a < 3; ++a) {
    const float c0 = g.o * R[3 * a], c1 = g.o * R[3 * a + 1];
    g00 = fmaf(c0, c0, g00); g01 = fmaf(c0, c1, g01); g11 = fmaf(c1, c1, g11);
  }
  const float d = g00 - g11;
  const float lam = 0.5f * (g00 + g11 - sqrtf(fmaf(d, d, 4.f * g01 * g01)));
  const float sig = sqrtf(fmaxf(lam, 0.f));
  const float a = (0.8660254f * NT) / sig;   // inf for a degenerate map
  const float c = 2.f * a + 1.f;
  return c * c;                              // NaN map -> NaN
}
// Poses whose bound is too large (degenerate maps) go to the edge kernel.
__device__ __forceinline__ bool scatter_pose_ok(float cb) { return cb <= 4096.0f; }

__device__ __forceinline__ int floor_i(float p) { return (int)safe_floor(p); }

__device__ __forceinline__ bool floor_in(const float p[3], const int lo[3], const int hi[3], int f[3]) {
  bool in = true;
#pragma unroll
  for (int a = 0; a < 3; ++a) {
    f[a] = floor_i(p[a]);
    in = in && f[a] >= lo[a] && f[a] < hi[a];
  }
  return in;
}

// Fixed-point conversion by the magic-number trick: for |x| < 2^22,
// fma(w, u, 1.5 * 2^23) rounds w * u to the nearest integer k in one
// instruction and its bit pattern is 0x4B400000 + k.
constexpr float MAGIC = 12582912.0f;
constexpr int MAGIC_BITS = 0x4B400000;

__device__ __forceinline__ int fixed_round(float w, float u) {
  return __float_as_int(fmaf(w, u, MAGIC)) - MAGIC_BITS;
}

// One 64-bit word holding re + im * 2^32 (re signed): sums of such words
// keep both parts exact as long as each partial sum stays within 31 bits.
__device__ __forceinline__ unsigned long long pack_fixed(int re, int im) {
  const unsigned int lo = (unsigned int)re;
  const unsigned int hi = (unsigned int)(im + (re >> 31));
  return ((unsigned long long)hi << 32) | lo;
}

__device__ __forceinline__ void unpack_fixed(unsigned long long w, float& re, float& im) {
  const long long v = (long long)w;
  const int r = (int)(unsigned int)(w & 0xffffffffull);
  const int i = (int)((v - (long long)r) >> 32);
  re = (float)r;
  im = (float)i;
}

}  // namespace

// ---------------------------------------------------------------------------
// work list of the stored bricks: prefix[] of the pose chunks, slot[] of the
// workspace tiles (bricks with more than one chunk)
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(1024) k_sbrick_prefix(ScatterGrid sg, int* __restrict__ prefix,
                                                        int* __restrict__ slot) {
  __shared__ int tot_k[16], tot_s[16];
  __shared__ int carry_k, carry_s;
  if (threadIdx.x == 0) { carry_k = 0; carry_s = 0; prefix[0] = 0; slot[0] = 0; }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int base = 0; base < sg.nb3; base += 1024) {
    const int b = base + threadIdx.x;
    int k = 0;
    if (b < sg.nb3) {
      int bi, bj, bk;
      sbrick_coords(sg, b, bi, bj, bk);
      k = sbrick_chunks(sg, bi, bj, bk);
    }
    int s = k > 1 ? k : 0;
    int vk = k, vs = s;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int uk = __shfl_up(vk, off, 64), us = __shfl_up(vs, off, 64);
      if (lane >= off) { vk += uk; vs += us; }
    }
    if (lane == 63) { tot_k[wave] = vk; tot_s[wave] = vs; }
    __syncthreads();
    int bk_ = carry_k, bs_ = carry_s;
    for (int w = 0; w < wave; ++w) { bk_ += tot_k[w]; bs_ += tot_s[w]; }
    if (b < sg.nb3) { prefix[b + 1] = bk_ + vk; slot[b + 1] = bs_ + vs; }
    __syncthreads();
    if (threadIdx.x == 1023) { carry_k = bk_ + vk; carry_s = bs_ + vs; }
    __syncthreads();
  }
}

__device__ __forceinline__ int find_sbrick(const int* __restrict__ prefix, int nb3, int w) {
  int lo = 0, hi = nb3;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (prefix[mid] <= w) lo = mid; else hi = mid;
  }
  return lo;
}

// Add the in-box taps of one pixel.  Rows outside the box along y or z are
// skipped; along x the out-of-box taps carry weight 0.  SGN = +1 for a direct
// box (local x = t + add), -1 for a mirrored one (local x = add - t).
template <int NT, bool WEIGHTS, int SGN>
__device__ __forceinline__ void scatter_taps(unsigned long long* tile, unsigned int* wtile, const TBox& box,
                                             const int f[3], const float wx[NT], const float wy[NT],
                                             const float wz[NT], float2 c, float wv) {
  constexpr int HL = NT == 4 ? 1 : 0;
  const int lx0 = SGN * (f[0] - HL) + box.add[0];   // local x of tap ja = 0
#pragma unroll
  for (int jc = 0; jc < NT; ++jc) {
    const int tz = f[2] - HL + jc;
    if (tz < box.qlo[2] || tz >= box.qhi[2]) continue;
    const int lz = SGN * tz + box.add[2];
#pragma unroll
    for (int jb = 0; jb < NT; ++jb) {
      const int ty = f[1] - HL + jb;
      if (ty < box.qlo[1] || ty >= box.qhi[1]) continue;
      const int ly = SGN * ty + box.add[1];
      const float wyz = wy[jb] * wz[jc];
      const float ur = wyz * c.x, ui = wyz * c.y, uw = wyz * wv;
      const int rowb = lz * TSZ + ly * TSY + lx0;
#pragma unroll
      for (int ja = 0; ja < NT; ++ja) {
        const int li = rowb + SGN * ja;
        atomicAdd(&tile[li], pack_fixed(fixed_round(wx[ja], ur), fixed_round(wx[ja], ui)));
        if constexpr (WEIGHTS) atomicAdd(&wtile[li], (unsigned int)fixed_round(wx[ja], uw));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Largest |Re|, |Im| (and |Wimg|) of every image per band of pixel radius
// |k| in [bw * i, bw * (i + 1)).  A brick's window scale is then taken over
// the bands that can reach the brick only, so large low-frequency values do
// not coarsen the fixed-point grid of the outer bricks.
// ---------------------------------------------------------------------------
template <bool WEIGHTS>
__global__ void __launch_bounds__(256) k_band_max(const float2* __restrict__ Y, const float* __restrict__ Wimg,
                                                  float* __restrict__ ymax, float* __restrict__ wmax, KGeom g,
                                                  ScatterGrid sg) {
  __shared__ unsigned int bm[MAX_BANDS], bw[MAX_BANDS];
  for (int bn = blockIdx.x; bn < g.B * g.P; bn += gridDim.x) {
    for (int i = threadIdx.x; i < sg.nbands; i += blockDim.x) { bm[i] = 0u; bw[i] = 0u; }
    __syncthreads();
    const float2* Yb = Y + (int64_t)bn * g.npix;
    for (int pix = threadIdx.x; pix < g.npix; pix += blockDim.x) {
      int ikx, iky;
      pixel_freq(g, pix, ikx, iky);
      const float kx = (float)ikx, ky = (float)iky;
      if (!in_mask(g, kx, ky)) continue;
      const int band = min((int)(sqrtf(fmaf(kx, kx, ky * ky)) * sg.inv_band_w), sg.nbands - 1);
      const float2 v = Yb[pix];
      atomicMax(&bm[band], __float_as_uint(fmaxf(fabsf(v.x), fabsf(v.y))));
      if constexpr (WEIGHTS) atomicMax(&bw[band], __float_as_uint(fabsf(Wimg[(int64_t)bn * g.npix + pix])));
    }
    __syncthreads();
    for (int i = threadIdx.x; i < sg.nbands; i += blockDim.x) {
      ymax[(int64_t)bn * sg.nbands + i] = __uint_as_float(bm[i]);
      if constexpr (WEIGHTS) wmax[(int64_t)bn * sg.nbands + i] = __uint_as_float(bw[i]);
    }
    __syncthreads();
  }
}

// Largest value a pose can put into a box: the bands of the pixel radii that
// map into the box [bl, bh) (|k| between |p| / sigma_max and |p| / sigma_min).
__device__ __forceinline__ float box_band_max(const KGeom& g, const ScatterGrid& sg, const float* R,
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
  const float kmin = sqrtf(dn) / smax - 1.0f, kmax = sqrtf(df) / smin + 1.0f;
  int b0 = (int)fmaxf(0.f, kmin * sg.inv_band_w);
  int b1 = (kmax * sg.inv_band_w < (float)sg.nbands) ? (int)(kmax * sg.inv_band_w) : sg.nbands - 1;   // NaN -> last
  if (!(kmin == kmin)) b0 = 0;
  float m = 0.f;
  for (int i = b0; i <= b1; ++i) m = fmaxf(m, table[pose * sg.nbands + i]);
  return m;
}

// ---------------------------------------------------------------------------
// the scatter kernel
// ---------------------------------------------------------------------------
template <int NT, bool WEIGHTS>
__global__ void __launch_bounds__(256) k_scatter_brick(const float2* __restrict__ Y, const float* __restrict__ Wimg,
                                                       const float* __restrict__ rot, const float* __restrict__ shifts,
                                                       float2* __restrict__ vol, float* __restrict__ wvol,
                                                       float2* __restrict__ ws_c, float* __restrict__ ws_w, KGeom g,
                                                       ScatterGrid sg, const int* __restrict__ prefix,
                                                       const int* __restrict__ slot, const float* __restrict__ ymax,
                                                       const float* __restrict__ wmax) {
  constexpr int HL = NT == 4 ? 1 : 0;      // taps below floor(p)
  constexpr int HH = NT - 1 - HL;          // taps above floor(p)
  // Taps outside the box along x are added with weight 0 (no branch); their
  // row-relative index lies in [-3, 18], which the guard entries below index 0
  // and the row padding keep inside the arrays.
  __shared__ unsigned long long tile_mem[TSIZE + TGUARD];
  __shared__ unsigned int wtile_mem[WEIGHTS ? TSIZE + TGUARD : 1];
  unsigned long long* tile = tile_mem + TGUARD;
  unsigned int* wtile = wtile_mem + (WEIGHTS ? TGUARD : 0);
  __shared__ int hits[256];
  __shared__ float hit_m[256], hit_w[256], hit_c[256];
  __shared__ int wave_n[4];

  const int w = blockIdx.x, vsel = blockIdx.y;
  if (w >= sg.nwork) return;
  const int b = find_sbrick(prefix, sg.nb3, w);
  const int chunk = w - prefix[b], nchunk = prefix[b + 1] - prefix[b];
  int bi, bj, bk;
  sbrick_coords(sg, b, bi, bj, bk);
  const int blo[3] = {bi * SB, bj * SB, bk * SB};
  const int bhi[3] = {min(blo[0] + SB, sg.W), min(blo[1] + SB, sg.D), min(blo[2] + SB, sg.D)};
  const int64_t e0 = (int64_t)sg.list_len * chunk / nchunk, e1 = (int64_t)sg.list_len * (chunk + 1) / nchunk;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  float2 acc[PER_LANE];
  float accw[PER_LANE];
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) {
    acc[i] = make_float2(0.f, 0.f);
    accw[i] = 0.f;
    const int idx = tid + 256 * i;
    if (idx < TSIZE) {
      tile[idx] = 0ull;
      if constexpr (WEIGHTS) wtile[idx] = 0u;
    }
  }
  if (tid < TGUARD) {
    tile_mem[tid] = 0ull;
    if constexpr (WEIGHTS) wtile_mem[tid] = 0u;
  }
  __syncthreads();

  // preimage boxes: direct copies of x, y, z, then mirrored copies (per-axis
  // copy lists in LDS, built by one lane)
  __shared__ AxisCopies cd[3], cm[3];
  if (tid == 0) {
    for (int a = 0; a < 3; ++a) axis_copies(blo[a], bhi[a], blo[a], sg.D, sg.tmin, sg.tmax, false, cd[a]);
    axis_copies(max(blo[0], 1), min(bhi[0], sg.half), blo[0], sg.D, sg.tmin, sg.tmax, true, cm[0]);
    for (int a = 1; a < 3; ++a) axis_copies(blo[a], bhi[a], blo[a], sg.D, sg.tmin, sg.tmax, true, cm[a]);
  }
  __syncthreads();
  const int nd = cd[0].n * cd[1].n * cd[2].n, nm = cm[0].n * cm[1].n * cm[2].n;

  for (int q = 0; q < nd + nm; ++q) {
    TBox box;
    {
      const bool mir = q >= nd;
      const AxisCopies* c = mir ? cm : cd;
      int r = mir ? q - nd : q;
      const int i0 = r % c[0].n; r /= c[0].n;
      const int i1 = r % c[1].n; r /= c[1].n;
      const int i2 = r;
      const int ii[3] = {i0, i1, i2};
      for (int a = 0; a < 3; ++a) { box.qlo[a] = c[a].qlo[ii[a]]; box.qhi[a] = c[a].qhi[ii[a]]; box.add[a] = c[a].add[ii[a]]; }
      box.sgn = mir ? -1 : 1;
    }
    // floor(p) values whose taps reach the box, within the served range
    int flo[3], fhi[3];
    bool empty = false;
    for (int a = 0; a < 3; ++a) {
      flo[a] = max(box.qlo[a] - HH, sg.fmin);
      fhi[a] = min(box.qhi[a] + HL, sg.fmax + 1);
      empty = empty || flo[a] >= fhi[a];
    }
    if (empty) continue;
    float bl[3], bh[3];
    for (int a = 0; a < 3; ++a) { bl[a] = (float)flo[a]; bh[a] = (float)fhi[a]; }

    for (int64_t eb = e0; eb < e1; eb += 256) {
      // ---- hit detection: one pose per lane, with its window bounds ----
      bool hit = false;
      float hm = 0.f, hw = 0.f, hc = 0.f;
      const int64_t e = eb + tid;
      if (e < e1) {
        int bimg, n;
        list_entry(g, vsel, (int)e, bimg, n);
        const float* R = rot + 9 * ((int64_t)(g.Br == 1 ? 0 : bimg) * g.P + n);
        hc = contrib_bound<NT>(g, R);
        hit = scatter_pose_ok(hc) && slice_meets_box(g, R, bl, bh);
        if (hit) {
          const int64_t pose = (int64_t)bimg * g.P + n;
          hm = box_band_max(g, sg, R, ymax, pose, bl, bh);
          if constexpr (WEIGHTS) hw = box_band_max(g, sg, R, wmax, pose, bl, bh);
        }
      }
      const unsigned long long m = __ballot(hit);
      if (lane == 0) wave_n[wave] = __popcll(m);
      __syncthreads();
      int before = 0, nh = 0;
      for (int v = 0; v < 4; ++v) { if (v < wave) before += wave_n[v]; nh += wave_n[v]; }
      if (hit) {
        const int slot_i = before + __popcll(m & ((1ull << lane) - 1ull));
        hits[slot_i] = (int)e;
        hit_m[slot_i] = hm;
        hit_w[slot_i] = hw;
        hit_c[slot_i] = hc;
      }
      __syncthreads();

      for (int hb = 0; hb < nh; hb += WINDOW) {
        const int nw = min(WINDOW, nh - hb);
        // window scale: largest value and per-voxel contribution bound
        float M = 0.f, MW = 0.f, C = 0.f;
        for (int h = 0; h < nw; ++h) {
          M = fmaxf(M, hit_m[hb + h]);
          MW = fmaxf(MW, hit_w[hb + h]);
          C += hit_c[hb + h];
        }
        // |re|, |im| <= sqrt(2) M per unit weight (the phase rotates); every
        // contribution also stays below 2^22 for the magic rounding
        const float scale = M > 0.f ? fminf(FIX_RANGE - C, 0.99f * 4194304.0f * C) / (1.41421356f * M * C) : 0.f;
        const float wscale = (WEIGHTS && MW > 0.f) ? fminf(FIX_RANGE - C, 0.99f * 4194304.0f * C) / (MW * C) : 0.f;

        // ---- pass 2: accumulate the in-box taps ----
        for (int h = wave; h < nw; h += 4) {
          int bimg, n;
          list_entry(g, vsel, hits[hb + h], bimg, n);
          const float* R = rot + 9 * ((int64_t)(g.Br == 1 ? 0 : bimg) * g.P + n);
          const float* s = shifts ? shifts + 2 * ((int64_t)(g.Bs == 1 ? 0 : bimg) * g.P + n) : nullptr;
          SliceRows rows;
          if (!slice_rows_box(g, R, bl, bh, rows)) continue;
          const int64_t ib = ((int64_t)bimg * g.P + n) * g.npix;
          for (int r0 = rows.ky_lo; r0 <= rows.ky_hi; r0 += 64) {
            RowBatch rb;
            row_batch(g, rows, r0, lane, rb);
            for (int base = 0; base < rb.total; base += 64) {
              const int i = base + lane;
              int kx, ky;
              candidate(rb, r0, i, kx, ky);
              if (i >= rb.total) continue;
              const float fkx = (float)kx, fky = (float)ky;
              float p[3];
              slice_coord(g, R, fkx, fky, p);
              int f[3];
              if (!floor_in(p, flo, fhi, f) || !in_mask(g, fkx, fky)) continue;
              const int64_t k = ib + pixel_index(g, kx, ky);
              float2 c = Y[k];
              if (s) c = cmulc(shift_phase(fkx, fky, s[0], s[1], g.inv_h), c);   // conj(phi) * Y
              if (box.sgn < 0) c.y = -c.y;                                        // Friedel mate
              c.x *= scale;
              c.y *= scale;
              const float wv = WEIGHTS ? Wimg[k] * wscale : 0.f;
              float wx[NT], wy[NT], wz[NT];
              axis_weights<NT>(p[0] - floorf(p[0]), wx);
              axis_weights<NT>(p[1] - floorf(p[1]), wy);
              axis_weights<NT>(p[2] - floorf(p[2]), wz);
#pragma unroll
              for (int ja = 0; ja < NT; ++ja) {
                const int tx = f[0] - HL + ja;
                if (tx < box.qlo[0] || tx >= box.qhi[0]) wx[ja] = 0.f;
              }
              if (box.sgn > 0) scatter_taps<NT, WEIGHTS, 1>(tile, wtile, box, f, wx, wy, wz, c, wv);
              else scatter_taps<NT, WEIGHTS, -1>(tile, wtile, box, f, wx, wy, wz, c, wv);
            }
          }
        }
        __syncthreads();
        // ---- flush the window into the float accumulators ----
        const float inv = scale > 0.f ? 1.0f / scale : 0.f;
        const float winv = wscale > 0.f ? 1.0f / wscale : 0.f;
#pragma unroll
        for (int i = 0; i < PER_LANE; ++i) {
          const int idx = tid + 256 * i;
          if (idx < TSIZE) {
            const unsigned long long v = tile[idx];
            if (v != 0ull) {
              float re, im;
              unpack_fixed(v, re, im);
              acc[i].x = fmaf(re, inv, acc[i].x);
              acc[i].y = fmaf(im, inv, acc[i].y);
              tile[idx] = 0ull;
            }
            if constexpr (WEIGHTS) {
              const unsigned int u = wtile[idx];
              if (u != 0u) {
                accw[i] = fmaf((float)(int)u, winv, accw[i]);
                wtile[idx] = 0u;
              }
            }
          }
        }
        __syncthreads();
      }
    }
  }

  // ---- write the brick (or this chunk's partial tile) ----
  const int64_t nvol = (int64_t)g.D * g.D * g.W;
  const bool direct = nchunk == 1;
  const int64_t sl = direct ? 0 : ((int64_t)vsel * sg.nslots + slot[b] + chunk) * TSIZE;
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) {
    const int idx = tid + 256 * i;
    if (idx >= TSIZE) continue;
    if (direct) {
      const int lz = idx / TSZ, rem = idx - lz * TSZ, ly = rem / TSY, lx = rem - ly * TSY;
      if (lx >= SB || ly >= SB) continue;
      const int x = blo[0] + lx, y = blo[1] + ly, z = blo[2] + lz;
      if (x >= bhi[0] || y >= bhi[1] || z >= bhi[2]) continue;
      const int64_t o = nvol * vsel + ((int64_t)z * g.D + y) * g.W + x;
      vol[o] = acc[i];
      if (WEIGHTS) wvol[o] = accw[i];
    } else {
      ws_c[sl + idx] = acc[i];
      if (WEIGHTS) ws_w[sl + idx] = accw[i];
    }
  }
}

// Sum the partial tiles of bricks that were split into several chunks.
template <bool WEIGHTS>
__global__ void __launch_bounds__(256) k_scatter_reduce(float2* __restrict__ vol, float* __restrict__ wvol,
                                                        const float2* __restrict__ ws_c, const float* __restrict__ ws_w,
                                                        KGeom g, ScatterGrid sg, const int* __restrict__ prefix,
                                                        const int* __restrict__ slot) {
  const int64_t nvol = (int64_t)g.D * g.D * g.W;   // < 2^31 for D <= 1024
  const int vsel = blockIdx.y;
  for (int v = blockIdx.x * blockDim.x + threadIdx.x; v < (int)nvol; v += gridDim.x * blockDim.x) {
    const int xy = v % (g.W * g.D), z = v / (g.W * g.D);
    const int x = xy % g.W, y = xy / g.W;
    const int bi = x / SB, bj = y / SB, bk = z / SB;
    const int b = (bk * sg.nby + bj) * sg.nbx + bi;
    const int k = prefix[b + 1] - prefix[b];
    if (k <= 1) continue;
    const int idx = (z - bk * SB) * TSZ + (y - bj * SB) * TSY + (x - bi * SB);
    const int64_t s0 = ((int64_t)vsel * sg.nslots + slot[b]) * TSIZE + idx;
    float2 a = make_float2(0.f, 0.f);
    float aw = 0.f;
    for (int c = 0; c < k; ++c) {
      const float2 t = ws_c[s0 + (int64_t)c * TSIZE];
      a.x += t.x;
      a.y += t.y;
      if (WEIGHTS) aw += ws_w[s0 + (int64_t)c * TSIZE];
    }
    vol[nvol * vsel + v] = a;
    if (WEIGHTS) wvol[nvol * vsel + v] = aw;
  }
}

// Pixels the bricks do not serve (degenerate maps, samples outside the served
// floor range): all their taps, with global atomics, after the bricks wrote.
template <int NT, bool WEIGHTS>
__global__ void __launch_bounds__(256) k_scatter_edge(const float2* __restrict__ Y, const float* __restrict__ Wimg,
                                                      const float* __restrict__ rot, const float* __restrict__ shifts,
                                                      float2* __restrict__ vol, float* __restrict__ wvol, KGeom g,
                                                      ScatterGrid sg) {
  const int pix = blockIdx.x * blockDim.x + threadIdx.x;
  if (pix >= g.npix) return;
  int ikx, iky;
  pixel_freq(g, pix, ikx, iky);
  const float kx = (float)ikx, ky = (float)iky;
  if (!in_mask(g, kx, ky)) return;
  const int64_t nvol = (int64_t)g.D * g.D * g.W;
  const int lo[3] = {sg.fmin, sg.fmin, sg.fmin}, hi[3] = {sg.fmax + 1, sg.fmax + 1, sg.fmax + 1};
  for (int bn = blockIdx.y; bn < g.B * g.P; bn += gridDim.y) {
    const int bimg = bn / g.P, n = bn - bimg * g.P;
    const float* R = rot + 9 * ((int64_t)(g.Br == 1 ? 0 : bimg) * g.P + n);
    const bool pose_ok = scatter_pose_ok(contrib_bound<NT>(g, R));
    // every sample of the pose inside the served floor range: nothing to do
    if (pose_ok && pose_pmax(g, R) <= 0.9995f * (float)(sg.fmax)) continue;
    float p[3];
    slice_coord(g, R, kx, ky, p);
    int f[3];
    if (pose_ok && floor_in(p, lo, hi, f)) continue;
    float2 c = Y[(int64_t)bn * g.npix + pix];
    if (shifts) {
      const float* s = shifts + 2 * ((int64_t)(g.Bs == 1 ? 0 : bimg) * g.P + n);
      c = cmulc(shift_phase(kx, ky, s[0], s[1], g.inv_h), c);
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
          if (WEIGHTS) unsafeAtomicAdd(VW + idx, wt * wimg);
        }
  }
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------
static size_t band_bytes(const ScatterGrid& sg) {
  return ((size_t)sg.npose * sg.nbands * sizeof(float) * (sg.weights ? 2 : 1) + 255) / 256 * 256;
}

size_t scatter_ws_bytes(const ScatterGrid& sg, int Bv) {
  const size_t tables = ((size_t)(sg.nb3 + 1) * 2 * sizeof(int) + 255) / 256 * 256;
  const size_t per_tile = (size_t)TSIZE * (sizeof(float2) + (sg.weights ? sizeof(float) : 0));
  return tables + band_bytes(sg) + (size_t)sg.nslots * Bv * per_tile;
}

hipError_t launch_scatter_brick(const KGeom& g, int interp, const ScatterGrid& sg, void* workspace, const float2* Y,
                                const float* Wimg, const float* rot, const float* shifts, float2* vol, float* wvol,
                                hipStream_t st) {
  int* prefix = (int*)workspace;
  int* slot = prefix + (sg.nb3 + 1);
  const size_t tables = ((size_t)(sg.nb3 + 1) * 2 * sizeof(int) + 255) / 256 * 256;
  float* ymax = (float*)((char*)workspace + tables);
  float* wmax = ymax + (size_t)sg.npose * sg.nbands;
  float2* ws_c = (float2*)((char*)workspace + tables + band_bytes(sg));
  float* ws_w = (float*)(ws_c + (size_t)sg.nslots * g.Bv * TSIZE);
  hipLaunchKernelGGL(k_sbrick_prefix, dim3(1), dim3(1024), 0, st, sg, prefix, slot);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    const int nb = sg.npose < 65535 ? sg.npose : 65535;
    if (Wimg) hipLaunchKernelGGL((k_band_max<true>), dim3(nb), dim3(256), 0, st, Y, Wimg, ymax, wmax, g, sg);
    else hipLaunchKernelGGL((k_band_max<false>), dim3(nb), dim3(256), 0, st, Y, Wimg, ymax, wmax, g, sg);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 grid(sg.nwork, g.Bv), blk(256);
  const bool wt = Wimg != nullptr;
#define TP_SCATTER(NT_, W_)                                                                                      \
  hipLaunchKernelGGL((k_scatter_brick<NT_, W_>), grid, blk, 0, st, Y, Wimg, rot, shifts, vol, wvol, ws_c, ws_w, g, \
                     sg, prefix, slot, ymax, wmax)
  if (interp == 1) { if (wt) TP_SCATTER(4, true); else TP_SCATTER(4, false); }
  else { if (wt) TP_SCATTER(2, true); else TP_SCATTER(2, false); }
#undef TP_SCATTER
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (sg.nslots > 0) {
    const int64_t nvol = (int64_t)g.D * g.D * g.W;
    const int blocks = (int)((nvol + 255) / 256 < 4096 ? (nvol + 255) / 256 : 4096);
    if (wt) hipLaunchKernelGGL((k_scatter_reduce<true>), dim3(blocks, g.Bv), blk, 0, st, vol, wvol, ws_c, ws_w, g, sg,
                               prefix, slot);
    else hipLaunchKernelGGL((k_scatter_reduce<false>), dim3(blocks, g.Bv), blk, 0, st, vol, wvol, ws_c, ws_w, g, sg,
                            prefix, slot);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int gy = g.B * g.P < 2048 ? g.B * g.P : 2048;
  const dim3 eg((g.npix + 255) / 256, gy);
  if (interp == 1) {
    if (wt) hipLaunchKernelGGL((k_scatter_edge<4, true>), eg, blk, 0, st, Y, Wimg, rot, shifts, vol, wvol, g, sg);
    else hipLaunchKernelGGL((k_scatter_edge<4, false>), eg, blk, 0, st, Y, Wimg, rot, shifts, vol, wvol, g, sg);
  } else {
    if (wt) hipLaunchKernelGGL((k_scatter_edge<2, true>), eg, blk, 0, st, Y, Wimg, rot, shifts, vol, wvol, g, sg);
    else hipLaunchKernelGGL((k_scatter_edge<2, false>), eg, blk, 0, st, Y, Wimg, rot, shifts, vol, wvol, g, sg);
  }
  return hipGetLastError();
}

}  // namespace tproj
