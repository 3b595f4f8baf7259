// Brick-binned gather kernels of libtproj for gfx950.
//
// k_brick_prefix   work list: prefix sums of the pose chunks of every brick
//                  and the bricks' active ranks
// k_hit_lists      per work item, the poses of its chunk whose slice reaches
//                  the brick (in order)
// k_fwd_brick      3D->2D forward (complex volume, with the shift phase) or
//                  its real counterpart (weight channel): a workgroup stages
//                  one tap-space brick of the Hermitian-extended periodic
//                  volume plus the interpolation halo in LDS, enumerates the
//                  pixels of its hit poses whose floor(p) falls in the brick
//                  (enum_block.h) and interpolates them from LDS (cubic: a
//                  bank-split tile read in a per-lane rotated tap order;
//                  linear: a padded tile, each pixel in the lane a
//                  bank-spreading order gives it).
// k_grad_brick     rotation / shift gradients on the same decomposition: the
//                  value and the three partial derivatives of the
//                  interpolant come from the LDS tile; per-pose wavefront
//                  sums by a butterfly reduce-scatter, per-window sums in
//                  LDS, then one global atomic per pose and term.
// *_edge           masked pixels and the rare samples outside every active
//                  brick (maps that are not rotations), from global memory.
//
// The operations are the rotated central slice with linear or Catmull-Rom
// interpolation, per-tap Friedel symmetry, Fourier-phase shifts and the
// gradients w.r.t. rotations and shifts (torch-projectors pages: Spanish
// "Resumen tecnico" 2, Dutch Methodologie, French "Resume technique" 2).
#include "brick_grid.h"
#include "brick_kernels.h"
#include "device_common.h"
#include "enum_block.h"
#include "gather_common.h"

namespace tproj {

// ---------------------------------------------------------------------------
// work list
// ---------------------------------------------------------------------------
// prefix[0..nb3]: running sums of the bricks' chunk counts; prefix[nb3 + 1 +
// b]: the active rank of brick b (bricks with chunks before it).  One
// workgroup; both sums in one 64-bit scan (chunks low, bricks high).  The
// chunk counts (64-bit divisions) are computed first, with no barrier
// between bricks, into prefix[b + 1]; the scan then reads them back (the
// thread that wrote an entry is the one that reads and overwrites it).
__global__ void __launch_bounds__(1024) k_brick_prefix(BrickGrid bg, int* __restrict__ prefix) {
  __shared__ long long warp_tot[16];
  __shared__ long long carry;
  for (int b = threadIdx.x; b < bg.nb3; b += 1024) {
    int bi, bj, bk;
    brick_coords(bg, b, bi, bj, bk);
    prefix[b + 1] = brick_chunks(bg, bi, bj, bk);
  }
  if (threadIdx.x == 0) { carry = 0; prefix[0] = 0; }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int base = 0; base < bg.nb3; base += 1024) {
    const int b = base + threadIdx.x;
    const int k = b < bg.nb3 ? prefix[b + 1] : 0;
    const long long own = (long long)k + (k > 0 ? (1ll << 32) : 0ll);
    long long v = own;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const long long u = __shfl_up(v, off, 64);
      if (lane >= off) v += u;
    }
    if (lane == 63) warp_tot[wave] = v;
    __syncthreads();
    long long before = carry;
    for (int w = 0; w < wave; ++w) before += warp_tot[w];
    if (b < bg.nb3) {
      prefix[b + 1] = (int)((before + v) & 0xffffffffll);
      prefix[bg.nb3 + 1 + b] = (int)((before + v - own) >> 32);
    }
    __syncthreads();
    if (threadIdx.x == 1023) carry = before + v;
    __syncthreads();
  }
}

// Hit lists of the forward and gradient bricks: does the slice of pose e
// reach the box?
__global__ void __launch_bounds__(256) k_hit_lists(const float* __restrict__ rot, KGeom g, BrickGrid bg,
                                                   const int* __restrict__ prefix, unsigned short* __restrict__ hits,
                                                   int* __restrict__ counts) {
  build_hit_list(bg, prefix, hits, counts, [&](int vsel, int e, const float* bl, const float* bh) {
    int bimg, n;
    list_entry(g, vsel, e, bimg, n);
    return slice_meets_box(g, rot + 9 * ((int64_t)(g.Br == 1 ? 0 : bimg) * g.P + n), bl, bh);
  });
}

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
// hits per window: 64 with the cubic tile (about 3% faster than 32 at D=128);
// 32 with the larger padded linear tile, so that four workgroups fit a CU's LDS
template <int NT>
constexpr int FWD_WIN = NT == 4 ? 64 : 32;
constexpr int FWD_NW = 4;   // wavefronts per workgroup

template <int NT, typename T>
__global__ void __launch_bounds__(256) k_fwd_brick(const T* __restrict__ vol, const float* __restrict__ rot,
                                                   const float* __restrict__ shifts, T* __restrict__ out, KGeom g,
                                                   BrickGrid bg, const int* __restrict__ prefix,
                                                   const unsigned short* __restrict__ hits,
                                                   const int* __restrict__ counts) {
  using Tl = Tile<NT>;
  constexpr bool CPLX = sizeof(T) == 8;
  __shared__ T tile[Tl::SIZE];
  __shared__ EnumShared<FWD_WIN<NT>, FWD_NW> es;
  __shared__ std::conditional_t<Tl::SPLIT, SplitLut, char> lut;   // tap tables of the bank-split tile
  const int w = blockIdx.x, vsel = blockIdx.y;
  if (w >= bg.nwork) return;
  const int nh = counts[(int64_t)vsel * bg.nwork + w];
  if (nh == 0) return;   // block-uniform, before any barrier
  const int b = find_brick(prefix, bg.nb3, w);
  int e0, e1;
  item_chunk(bg, prefix, b, w, e0, e1);
  const unsigned short* hl = hits + hit_slot(bg, prefix, vsel, b, e0);
  int bi, bj, bk;
  brick_coords(bg, b, bi, bj, bk);
  const int lo[3] = {bg.origin + bi * bg.S, bg.origin + bj * bg.S, bg.origin + bk * bg.S};
  const float bl[3] = {(float)lo[0], (float)lo[1], (float)lo[2]};
  const float bh[3] = {(float)(lo[0] + bg.S), (float)(lo[1] + bg.S), (float)(lo[2] + bg.S)};
  if constexpr (Tl::SPLIT) split_lut_fill(lut);
  stage_tile_t<NT, FWD_NW * 64>(tile, vol + (int64_t)vsel * g.D * g.D * g.W, g, lo);
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  {
    for (int hw = 0; hw < nh; hw += FWD_WIN<NT>) {
      const int nw = min(FWD_WIN<NT>, nh - hw);
      window_setup(es, g, rot, CPLX ? shifts : nullptr, vsel, e0, hl + hw, nw, bl, bh);
      const int nrows = es.hrow[nw];
      for (int qb = 0; qb < nrows;) {
        int nr;
        const int ncand = row_stage(es, g, qb, nrows, nw, bl, bh, nr);
        for (int c0 = wave * 64; c0 < ncand; c0 += FWD_NW * 64) {   // wave-uniform (lane permutes)
          Cand cu;
          cand_prep(es, g, c0 + lane, ncand, lo, bg.S, cu);
          if constexpr (Tl::SPLIT) {
            // each lane interpolates its own pixel, in its slot's tap order
            if (cu.act) {
              float wx[4], wy[4], wz[4];
              axis_weights<4>(frac_of(cu.p[0]), wx);
              axis_weights<4>(frac_of(cu.p[1]), wy);
              axis_weights<4>(frac_of(cu.p[2]), wz);
              T I;
              interp_split<false>(tile, lut, cu.l, wx, wy, wz, wx, wy, wz, I, (T*)nullptr);
              if constexpr (CPLX) {
                if (shifts) I = cmul(shift_phase(cu.kx, cu.ky, cu.sx, cu.sy, g.inv_h), I);
              }
              out[cu.k] = I;
            }
          } else {
            // the interpolation runs in the lane the bank-spreading order gives
            // the pixel; the value comes back to the pixel's own lane
            float f[3] = {0.f, 0.f, 0.f};
            int pk = 0, key = -1;
            if (cu.act) {
#pragma unroll
              for (int a = 0; a < 3; ++a) f[a] = frac_of(cu.p[a]);
              pk = 1 | (cu.l[0] << 1) | (cu.l[1] << 5) | (cu.l[2] << 9);
              key = (cu.l[0] + cu.l[1] * Tl::SY + cu.l[2] * Tl::SZ) & 15;
            }
            const int dest = spread_dest(key);
            const int mpk = lane_send(pk, dest);
            float mf[3];
#pragma unroll
            for (int a = 0; a < 3; ++a) mf[a] = lane_send(f[a], dest);
            T I = zero_of(T{});
            if (mpk & 1) {
              const int ml[3] = {(mpk >> 1) & 15, (mpk >> 5) & 15, (mpk >> 9) & 15};
              float wx[NT], wy[NT], wz[NT];
              axis_weights<NT>(mf[0], wx);
              axis_weights<NT>(mf[1], wy);
              axis_weights<NT>(mf[2], wz);
              interp_tile_w<NT, false>(tile, ml, wx, wy, wz, wx, wy, wz, I, (T*)nullptr);
            }
            I = lane_fetch(I, dest);
            if (cu.act) {
              if constexpr (CPLX) {
                if (shifts) I = cmul(shift_phase(cu.kx, cu.ky, cu.sx, cu.sy, g.inv_h), I);
              }
              out[cu.k] = I;
            }
          }
        }
        __syncthreads();   // the next row stage rewrites the rows
        qb += nr;
      }
      __syncthreads();     // the next window rewrites the hit table
    }
  }
}

// Masked pixels -> 0; pixels outside every active brick -> direct gather.
// One workgroup per pose: a pose whose largest sample radius is below the
// brick grid's bound is served entirely by the bricks, and only its masked
// pixels are written here.
template <int NT, typename T>
__global__ void __launch_bounds__(256) k_fwd_edge(const T* __restrict__ vol, const float* __restrict__ rot,
                                                  const float* __restrict__ shifts, T* __restrict__ out, KGeom g,
                                                  BrickGrid bg) {
  constexpr bool CPLX = sizeof(T) == 8;
  const int64_t nvol = (int64_t)g.D * g.D * g.W;
  for (int bn = blockIdx.x; bn < g.B * g.P; bn += gridDim.x) {
    const int bimg = bn / g.P, n = bn - bimg * g.P;
    const float* R = rot + 9 * ((int64_t)(g.Br == 1 ? 0 : bimg) * g.P + n);
    const bool inside = pose_pmax(g, R) <= 0.9995f * (float)bg.pmax_i;
    T* O = out + (int64_t)bn * g.npix;
    for (PixelWalk pw(g, threadIdx.x, blockDim.x); pw.pix < g.npix; pw.step(g, blockDim.x)) {
      const int pix = pw.pix;
      const float kx = (float)pw.kx(), ky = (float)pw.ky(g);
      if (!in_mask(g, kx, ky)) { O[pix] = zero_of(T{}); continue; }
      if (inside) continue;
      float p[3];
      slice_coord(g, R, kx, ky, p);
      if (served_by_bricks(bg, p)) continue;
      if constexpr (CPLX) {
        float2 I = interp_global<NT>(vol + nvol * (g.Bv == 1 ? 0 : bimg), g, p);
        if (shifts) {
          const float* s = shifts + 2 * ((int64_t)(g.Bs == 1 ? 0 : bimg) * g.P + n);
          I = cmul(shift_phase(kx, ky, s[0], s[1], g.inv_h), I);
        }
        O[pix] = I;
      } else {
        float I;
        interp_r<NT, false>(vol + nvol * (g.Bv == 1 ? 0 : bimg), g, p[0], p[1], p[2], I, nullptr);
        O[pix] = I;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// rotation / shift gradients
//   gR[i][j] += o * sum_k M (Re(conj(U) phi dI_i(Vc)) + Ur dI_i(Vr)) k3_j
//   gs       += (2 pi / H) sum_k M (kx, ky) Im(conj(U) phi I(Vc))
// Each candidate lane computes its 8 terms; a butterfly reduce-scatter over
// the lanes of each hit (candidates are ordered by hit, grad_collect) leaves
// the hit's 8 totals in lanes 0-7, which add them to the hit's sum in LDS.  At
// the end of a window the sums go to the pose's gradient with global atomics.
// ---------------------------------------------------------------------------
// hits per window: 32 with the cubic tile, 16 with the larger padded linear
// one (four workgroups per CU fit the LDS either way)
template <int NT>
constexpr int GRAD_WIN = NT == 4 ? 32 : 16;
constexpr int GRAD_NW = 4;

template <int NT, bool CPLX, bool REAL>
__global__ void __launch_bounds__(256, (CPLX && REAL) ? 2 : 4) k_grad_brick(const float2* __restrict__ volc, const float* __restrict__ volr,
                                                    const float2* __restrict__ U, const float* __restrict__ Ur,
                                                    const float* __restrict__ rot, const float* __restrict__ shifts,
                                                    float* __restrict__ grad_rot, float* __restrict__ grad_s, KGeom g,
                                                    BrickGrid bg, const int* __restrict__ prefix,
                                                    const unsigned short* __restrict__ hits,
                                                    const int* __restrict__ counts) {
  using Tl = Tile<NT>;
  __shared__ float2 tc[CPLX ? Tl::SIZE : 1];
  __shared__ float tr[REAL ? Tl::SIZE : 1];
  constexpr int WIN = GRAD_WIN<NT>;
  __shared__ EnumShared<WIN, GRAD_NW> es;
  __shared__ float gw[WIN][8];
  __shared__ std::conditional_t<Tl::SPLIT, SplitLut, char> lut;   // tap tables of the bank-split tile
  const int w = blockIdx.x, vsel = blockIdx.y;
  if (w >= bg.nwork) return;
  const int nh = counts[(int64_t)vsel * bg.nwork + w];
  if (nh == 0) return;   // block-uniform, before any barrier
  const int b = find_brick(prefix, bg.nb3, w);
  int e0, e1;
  item_chunk(bg, prefix, b, w, e0, e1);
  const unsigned short* hl = hits + hit_slot(bg, prefix, vsel, b, e0);
  int bi, bj, bk;
  brick_coords(bg, b, bi, bj, bk);
  const int lo[3] = {bg.origin + bi * bg.S, bg.origin + bj * bg.S, bg.origin + bk * bg.S};
  const float bl[3] = {(float)lo[0], (float)lo[1], (float)lo[2]};
  const float bh[3] = {(float)(lo[0] + bg.S), (float)(lo[1] + bg.S), (float)(lo[2] + bg.S)};
  const int64_t nvol = (int64_t)g.D * g.D * g.W;
  if constexpr (CPLX) stage_tile_t<NT, GRAD_NW * 64>(tc, volc + (int64_t)vsel * nvol, g, lo);
  if constexpr (REAL) stage_tile_t<NT, GRAD_NW * 64>(tr, volr + (int64_t)vsel * nvol, g, lo);
  for (int i = threadIdx.x; i < WIN * 8; i += GRAD_NW * 64) (&gw[0][0])[i] = 0.f;
  if constexpr (Tl::SPLIT) split_lut_fill(lut);
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  {
    for (int hw = 0; hw < nh; hw += WIN) {
      const int nw = min(WIN, nh - hw);
      window_setup(es, g, rot, CPLX ? shifts : nullptr, vsel, e0, hl + hw, nw, bl, bh);
      const int nrows = es.hrow[nw];
      for (int qb = 0; qb < nrows;) {
        int nr;
        const int ncand = row_stage(es, g, qb, nrows, nw, bl, bh, nr);
        for (int c0 = wave * 64; c0 < ncand; c0 += GRAD_NW * 64) {   // wave-uniform: permutes, sums
          Cand cu;
          cand_prep(es, g, c0 + lane, ncand, lo, bg.S, cu);
          float2 uc = make_float2(0.f, 0.f);
          float ur = 0.f;
          float2 Ic = make_float2(0.f, 0.f), dIc[3] = {Ic, Ic, Ic};
          float Ir = 0.f, dIr[3] = {0.f, 0.f, 0.f};
          if constexpr (Tl::SPLIT) {
            // each lane interpolates its own pixel, in its slot's tap order
            if (cu.act) {
              if constexpr (CPLX) uc = U[cu.k];
              if constexpr (REAL) ur = Ur[cu.k];
              float wx[4], wy[4], wz[4], dx[4], dy[4], dz[4];
              const float fx = frac_of(cu.p[0]), fy = frac_of(cu.p[1]), fz = frac_of(cu.p[2]);
              axis_weights<4>(fx, wx);
              axis_weights<4>(fy, wy);
              axis_weights<4>(fz, wz);
              axis_dweights<4>(fx, dx);
              axis_dweights<4>(fy, dy);
              axis_dweights<4>(fz, dz);
              if constexpr (CPLX) interp_split<true>(tc, lut, cu.l, wx, wy, wz, dx, dy, dz, Ic, dIc);
              if constexpr (REAL) interp_split<true>(tr, lut, cu.l, wx, wy, wz, dx, dy, dz, Ir, dIr);
            }
          } else {
            float f[3] = {0.f, 0.f, 0.f};
            int pk = 0, key = -1;
            if (cu.act) {
              if constexpr (CPLX) uc = U[cu.k];
              if constexpr (REAL) ur = Ur[cu.k];
#pragma unroll
              for (int a = 0; a < 3; ++a) f[a] = frac_of(cu.p[a]);
              pk = 1 | (cu.l[0] << 1) | (cu.l[1] << 5) | (cu.l[2] << 9);
              key = (cu.l[0] + cu.l[1] * Tl::SY + cu.l[2] * Tl::SZ) & 15;
            }
            // the interpolation runs in the lane the bank-spreading order gives
            // the pixel; value and derivatives come back to the pixel's lane
            const int dest = spread_dest(key);
            const int mpk = lane_send(pk, dest);
            float mf[3];
#pragma unroll
            for (int a = 0; a < 3; ++a) mf[a] = lane_send(f[a], dest);
            if (mpk & 1) {
              const int ml[3] = {(mpk >> 1) & 15, (mpk >> 5) & 15, (mpk >> 9) & 15};
              float wx[NT], wy[NT], wz[NT], dx[NT], dy[NT], dz[NT];
              axis_weights<NT>(mf[0], wx);
              axis_weights<NT>(mf[1], wy);
              axis_weights<NT>(mf[2], wz);
              axis_dweights<NT>(mf[0], dx);
              axis_dweights<NT>(mf[1], dy);
              axis_dweights<NT>(mf[2], dz);
              if constexpr (CPLX) interp_tile_w<NT, true>(tc, ml, wx, wy, wz, dx, dy, dz, Ic, dIc);
              if constexpr (REAL) interp_tile_w<NT, true>(tr, ml, wx, wy, wz, dx, dy, dz, Ir, dIr);
            }
            if constexpr (CPLX) {
              Ic = lane_fetch(Ic, dest);
#pragma unroll
              for (int a = 0; a < 3; ++a) dIc[a] = lane_fetch(dIc[a], dest);
            }
            if constexpr (REAL) {
#pragma unroll
              for (int a = 0; a < 3; ++a) dIr[a] = lane_fetch(dIr[a], dest);
            }
          }
          float acc[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) acc[q] = 0.f;
          float e3[3] = {0.f, 0.f, 0.f};
          const float fkx = cu.act ? cu.kx : 0.f, fky = cu.act ? cu.ky : 0.f;
          if constexpr (CPLX) {
            float2 phi = make_float2(1.f, 0.f);
            if (shifts && cu.act) phi = shift_phase(fkx, fky, cu.sx, cu.sy, g.inv_h);
            const float2 cc = cmulc(uc, phi);   // conj(U) * phi
#pragma unroll
            for (int a = 0; a < 3; ++a) e3[a] = cc.x * dIc[a].x - cc.y * dIc[a].y;
            const float im = cc.x * Ic.y + cc.y * Ic.x;
            acc[6] = fkx * im;
            acc[7] = fky * im;
          }
          if constexpr (REAL) {
#pragma unroll
            for (int a = 0; a < 3; ++a) e3[a] = fmaf(ur, dIr[a], e3[a]);
          }
#pragma unroll
          for (int a = 0; a < 3; ++a) {
            acc[2 * a] = e3[a] * fkx;
            acc[2 * a + 1] = e3[a] * fky;
          }
          grad_collect(acc, cu.key, gw);
        }
        __syncthreads();
        qb += nr;
      }
      grad_flush<WIN>(g, es, gw, nw, grad_rot, CPLX ? grad_s : nullptr);
      __syncthreads();
    }
  }
}

// Pixels outside every active brick: their gradient terms from global memory
// (one workgroup per pose; poses inside the brick grid are skipped whole).
template <int NT, bool CPLX, bool REAL>
__global__ void __launch_bounds__(256) k_grad_edge(const float2* __restrict__ volc, const float* __restrict__ volr,
                                                   const float2* __restrict__ U, const float* __restrict__ Ur,
                                                   const float* __restrict__ rot, const float* __restrict__ shifts,
                                                   float* __restrict__ grad_rot, float* __restrict__ grad_s, KGeom g,
                                                   BrickGrid bg) {
  const int64_t nvol = (int64_t)g.D * g.D * g.W;
  for (int bn = blockIdx.x; bn < g.B * g.P; bn += gridDim.x) {
    const int bimg = bn / g.P, n = bn - bimg * g.P;
    const float* R = rot + 9 * ((int64_t)(g.Br == 1 ? 0 : bimg) * g.P + n);
    if (pose_pmax(g, R) <= 0.9995f * (float)bg.pmax_i) continue;
    for (PixelWalk pw(g, threadIdx.x, blockDim.x); pw.pix < g.npix; pw.step(g, blockDim.x)) {
      const int pix = pw.pix;
      const float kx = (float)pw.kx(), ky = (float)pw.ky(g);
      if (!in_mask(g, kx, ky)) continue;
      float p[3];
      slice_coord(g, R, kx, ky, p);
      if (served_by_bricks(bg, p)) continue;
      const int64_t k = (int64_t)bn * g.npix + pix;
      float e[3] = {0.f, 0.f, 0.f}, im = 0.f;
      if constexpr (CPLX) {
        float2 I, dI[3];
        interp_c<NT, true>(volc + nvol * (g.Bv == 1 ? 0 : bimg), g, p[0], p[1], p[2], I, dI);
        float2 phi = make_float2(1.f, 0.f);
        if (shifts) {
          const float* s = shifts + 2 * ((int64_t)(g.Bs == 1 ? 0 : bimg) * g.P + n);
          phi = shift_phase(kx, ky, s[0], s[1], g.inv_h);
        }
        const float2 cu = cmulc(U[k], phi);
        for (int a = 0; a < 3; ++a) e[a] = cu.x * dI[a].x - cu.y * dI[a].y;
        im = cu.x * I.y + cu.y * I.x;
      }
      if constexpr (REAL) {
        float I, dI[3];
        interp_r<NT, true>(volr + nvol * (g.Bv == 1 ? 0 : bimg), g, p[0], p[1], p[2], I, dI);
        for (int a = 0; a < 3; ++a) e[a] = fmaf(Ur[k], dI[a], e[a]);
      }
      if (grad_rot) {
        float* gr = grad_rot + 9 * ((int64_t)(g.Br == 1 ? 0 : bimg) * g.P + n);
        for (int a = 0; a < 3; ++a) {
          atomicAdd(gr + 3 * a, g.o * e[a] * kx);
          atomicAdd(gr + 3 * a + 1, g.o * e[a] * ky);
        }
      }
      if (CPLX && grad_s) {
        float* gs = grad_s + 2 * ((int64_t)(g.Bs == 1 ? 0 : bimg) * g.P + n);
        atomicAdd(gs, 6.283185307179586f * g.inv_h * kx * im);
        atomicAdd(gs + 1, 6.283185307179586f * g.inv_h * ky * im);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_brick_prefix(const BrickGrid& bg, int* prefix, hipStream_t st) {
  hipLaunchKernelGGL(k_brick_prefix, dim3(1), dim3(1024), 0, st, bg, prefix);
  return hipGetLastError();
}

// One workgroup per pose (grid-stride beyond 16384 poses).
static dim3 edge_grid(const KGeom& g) { return dim3(g.B * g.P < 16384 ? g.B * g.P : 16384); }

// The edge kernel goes to st_edge (it writes other pixels than the brick
// kernel, so the two may run at once), the brick kernel to st.
template <typename T>
static hipError_t fwd_t(const KGeom& g, int interp, const BrickGrid& bg, const BrickWork& wk, const T* vol,
                        const float* rot, const float* shifts, T* out, hipStream_t st, const EvPair* ev,
                        hipStream_t st_edge) {
  const dim3 blk(256);
  if (interp == 1) hipLaunchKernelGGL((k_fwd_edge<4, T>), edge_grid(g), blk, 0, st_edge, vol, rot, shifts, out, g, bg);
  else hipLaunchKernelGGL((k_fwd_edge<2, T>), edge_grid(g), blk, 0, st_edge, vol, rot, shifts, out, g, bg);
  hipError_t e = hipGetLastError();
  const dim3 grid(bg.nwork, g.Bv);
  if (e == hipSuccess && bg.nwork > 0) {
    hipLaunchKernelGGL(k_hit_lists, grid, blk, 0, st, rot, g, bg, wk.prefix, wk.hits, wk.counts);
    e = hipGetLastError();
  }
  ev_begin(ev, st);   // recorded even when no brick kernel runs
  if (e != hipSuccess || bg.nwork == 0) {
    ev_end(ev, st);
    return e;
  }
  if (interp == 1)
    hipLaunchKernelGGL((k_fwd_brick<4, T>), grid, blk, 0, st, vol, rot, shifts, out, g, bg, wk.prefix, wk.hits,
                       wk.counts);
  else
    hipLaunchKernelGGL((k_fwd_brick<2, T>), grid, blk, 0, st, vol, rot, shifts, out, g, bg, wk.prefix, wk.hits,
                       wk.counts);
  ev_end(ev, st);
  return hipGetLastError();
}

hipError_t launch_fwd_brick(const KGeom& g, int interp, const BrickGrid& bg, const BrickWork& wk, const float2* vol,
                            const float* rot, const float* shifts, float2* out, hipStream_t st, const EvPair* ev,
                            hipStream_t st_edge) {
  return fwd_t<float2>(g, interp, bg, wk, vol, rot, shifts, out, st, ev, st_edge);
}

hipError_t launch_fwd_brick_real(const KGeom& g, int interp, const BrickGrid& bg, const BrickWork& wk,
                                 const float* vol, const float* rot, float* out, hipStream_t st, const EvPair* ev) {
  return fwd_t<float>(g, interp, bg, wk, vol, rot, nullptr, out, st, ev, st);
}

template <int NT, bool C, bool R>
static void grad_launch(const KGeom& g, const BrickGrid& bg, const BrickWork& wk, const float2* volc,
                        const float* volr, const float2* U, const float* Ur, const float* rot, const float* shifts,
                        float* grad_rot, float* grad_s, hipStream_t st, const EvPair* ev) {
  const dim3 blk(256), grid(bg.nwork, g.Bv);
  if (bg.nwork > 0) hipLaunchKernelGGL(k_hit_lists, grid, blk, 0, st, rot, g, bg, wk.prefix, wk.hits, wk.counts);
  ev_begin(ev, st);   // recorded even when no brick kernel runs
  if (bg.nwork > 0)
    hipLaunchKernelGGL((k_grad_brick<NT, C, R>), grid, blk, 0, st, volc, volr, U, Ur, rot, shifts, grad_rot, grad_s,
                       g, bg, wk.prefix, wk.hits, wk.counts);
  ev_end(ev, st);
  // the few pixels outside every active brick (both kernels add into the
  // zeroed outputs, so the order is free)
  hipLaunchKernelGGL((k_grad_edge<NT, C, R>), edge_grid(g), blk, 0, st, volc, volr, U, Ur, rot, shifts, grad_rot,
                     grad_s, g, bg);
}

hipError_t launch_grad_brick(const KGeom& g, int interp, const BrickGrid& bg, const BrickWork& wk, const float2* volc,
                             const float* volr, const float2* U, const float* Ur, const float* rot,
                             const float* shifts, float* grad_rot, float* grad_s, hipStream_t st, const EvPair* ev) {
  const bool c = volc != nullptr, r = volr != nullptr;
#define TP_GRAD(NT_)                                                                                             \
  do {                                                                                                           \
    if (c && r) grad_launch<NT_, true, true>(g, bg, wk, volc, volr, U, Ur, rot, shifts, grad_rot, grad_s, st, ev);  \
    else if (c) grad_launch<NT_, true, false>(g, bg, wk, volc, volr, U, Ur, rot, shifts, grad_rot, grad_s, st, ev); \
    else if (r) grad_launch<NT_, false, true>(g, bg, wk, volc, volr, U, Ur, rot, shifts, grad_rot, grad_s, st, ev); \
  } while (0)
  if (interp == 1) TP_GRAD(4); else TP_GRAD(2);
#undef TP_GRAD
  return hipGetLastError();
}

}  // namespace tproj
