// Brick-binned gather kernels of libtproj for gfx950.
//
// k_brick_prefix   work list: prefix sums of the pose chunks of every brick
// k_fwd_brick      3D->2D forward: a workgroup stages one tap-space brick of
//                  the (Hermitian-extended, periodic) volume plus the
//                  interpolation halo in LDS, then every wavefront walks the
//                  poses of its chunk, enumerates the pixels whose floor(p)
//                  falls in the brick (row by row, from the slab
//                  inequalities of the rotated central slice) and
//                  interpolates them from LDS.
// k_fwd_edge       writes the masked pixels (zeros) and serves the rare
//                  pixels whose floor(p) lies in no active brick.
//
// The operation is the rotated central slice with linear or Catmull-Rom
// interpolation, per-tap Friedel symmetry and Fourier-phase shifts
// (torch-projectors pages: Spanish "Resumen tecnico" 2, Dutch Methodologie,
// French "Resume technique" 2).
#include "brick_grid.h"
#include "brick_kernels.h"
#include "device_common.h"
#include "gather_common.h"

namespace tproj {

// ---------------------------------------------------------------------------
// work list
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(1024) k_brick_prefix(BrickGrid bg, int* __restrict__ prefix) {
  __shared__ int warp_tot[16];
  __shared__ int carry;
  if (threadIdx.x == 0) { carry = 0; prefix[0] = 0; }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int base = 0; base < bg.nb3; base += 1024) {
    const int b = base + threadIdx.x;
    int k = 0;
    if (b < bg.nb3) {
      int bi, bj, bk;
      brick_coords(bg, b, bi, bj, bk);
      k = brick_chunks(bg, bi, bj, bk);
    }
    // inclusive scan within the wave
    int v = k;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int u = __shfl_up(v, off, 64);
      if (lane >= off) v += u;
    }
    if (lane == 63) warp_tot[wave] = v;
    __syncthreads();
    int before = carry;
    for (int w = 0; w < wave; ++w) before += warp_tot[w];
    if (b < bg.nb3) prefix[b + 1] = before + v;
    __syncthreads();
    if (threadIdx.x == 1023) carry = before + v;
    __syncthreads();
  }
}

// Locate work item w: brick b with prefix[b] <= w < prefix[b + 1].
__device__ __forceinline__ int find_brick(const int* __restrict__ prefix, int nb3, int w) {
  int lo = 0, hi = nb3;          // invariant: prefix[lo] <= w < prefix[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (prefix[mid] <= w) lo = mid; else hi = mid;
  }
  return lo;
}

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
template <int NT>
__global__ void __launch_bounds__(256) k_fwd_brick(const float2* __restrict__ vol, const float* __restrict__ rot,
                                                   const float* __restrict__ shifts, float2* __restrict__ out,
                                                   KGeom g, BrickGrid bg, const int* __restrict__ prefix) {
  using Tl = Tile<NT>;
  __shared__ float2 tile[Tl::SIZE];
  const int w = blockIdx.x, vsel = blockIdx.y;
  if (w >= bg.nwork) return;
  const int b = find_brick(prefix, bg.nb3, w);
  const int chunk = w - prefix[b], nchunk = prefix[b + 1] - prefix[b];
  int bi, bj, bk;
  brick_coords(bg, b, bi, bj, bk);
  const int lo[3] = {bg.origin + bi * bg.S, bg.origin + bj * bg.S, bg.origin + bk * bg.S};
  const float2* V = vol + (int64_t)vsel * g.D * g.D * g.W;

  stage_tile<NT>(tile, V, g, lo);
  __syncthreads();

  const int64_t e0 = (int64_t)bg.list_len * chunk / nchunk, e1 = (int64_t)bg.list_len * (chunk + 1) / nchunk;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int64_t e = e0 + wave; e < e1; e += 4) {
    int bimg, n;
    list_entry(g, vsel, (int)e, bimg, n);
    const float* R = rot + 9 * ((int64_t)(g.Br == 1 ? 0 : bimg) * g.P + n);
    const float* s = shifts ? shifts + 2 * ((int64_t)(g.Bs == 1 ? 0 : bimg) * g.P + n) : nullptr;
    SliceRows rows;
    if (!slice_rows_setup(g, R, lo, bg.S, rows)) continue;
    float2* O = out + ((int64_t)bimg * g.P + n) * g.npix;
    for (int r0 = rows.ky_lo; r0 <= rows.ky_hi; r0 += 64) {
      RowBatch rb;
      row_batch(g, rows, r0, lane, rb);
      for (int base = 0; base < rb.total; base += 64) {   // wave-uniform loop
        const int i = base + lane;
        int kx, ky;
        candidate(rb, r0, i, kx, ky);
        if (i >= rb.total) continue;
        const float fkx = (float)kx, fky = (float)ky;
        float p[3];
        slice_coord(g, R, fkx, fky, p);
        int l[3];
        if (!owned(p, lo, bg.S, l) || !in_mask(g, fkx, fky)) continue;
        float2 I = interp_tile<NT>(tile, p, l);
        if (s) I = cmul(shift_phase(fkx, fky, s[0], s[1], g.inv_h), I);
        O[pixel_index(g, kx, ky)] = I;
      }
    }
  }
}

// Masked pixels -> 0; pixels outside every active brick -> direct gather.
template <int NT>
__global__ void __launch_bounds__(256) k_fwd_edge(const float2* __restrict__ vol, const float* __restrict__ rot,
                                                  const float* __restrict__ shifts, float2* __restrict__ out, KGeom g,
                                                  BrickGrid bg) {
  const int pix = blockIdx.x * blockDim.x + threadIdx.x;
  if (pix >= g.npix) return;
  int ikx, iky;
  pixel_freq(g, pix, ikx, iky);
  const float kx = (float)ikx, ky = (float)iky;
  const bool m = in_mask(g, kx, ky);
  const int64_t nvol = (int64_t)g.D * g.D * g.W;
  for (int bn = blockIdx.y; bn < g.B * g.P; bn += gridDim.y) {
    const int bimg = bn / g.P, n = bn - bimg * g.P;
    float2* o = out + (int64_t)bn * g.npix + pix;
    if (!m) { *o = make_float2(0.f, 0.f); continue; }
    const float* R = rot + 9 * ((int64_t)(g.Br == 1 ? 0 : bimg) * g.P + n);
    float p[3];
    slice_coord(g, R, kx, ky, p);
    if (in_active_brick(bg, p)) continue;
    float2 I = interp_global<NT>(vol + nvol * (g.Bv == 1 ? 0 : bimg), g, p);
    if (shifts) {
      const float* s = shifts + 2 * ((int64_t)(g.Bs == 1 ? 0 : bimg) * g.P + n);
      I = cmul(shift_phase(kx, ky, s[0], s[1], g.inv_h), I);
    }
    *o = I;
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_brick_prefix(const BrickGrid& bg, int* prefix, hipStream_t st) {
  hipLaunchKernelGGL(k_brick_prefix, dim3(1), dim3(1024), 0, st, bg, prefix);
  return hipGetLastError();
}

hipError_t launch_fwd_brick(const KGeom& g, int interp, const BrickGrid& bg, const int* prefix, const float2* vol,
                            const float* rot, const float* shifts, float2* out, hipStream_t st) {
  const int gy = g.B * g.P < 65535 ? g.B * g.P : 65535;
  const dim3 eg((g.npix + 255) / 256, gy), blk(256);
  if (interp == 1) hipLaunchKernelGGL((k_fwd_edge<4>), eg, blk, 0, st, vol, rot, shifts, out, g, bg);
  else hipLaunchKernelGGL((k_fwd_edge<2>), eg, blk, 0, st, vol, rot, shifts, out, g, bg);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || bg.nwork == 0) return e;
  const dim3 grid(bg.nwork, g.Bv);
  if (interp == 1) hipLaunchKernelGGL((k_fwd_brick<4>), grid, blk, 0, st, vol, rot, shifts, out, g, bg, prefix);
  else hipLaunchKernelGGL((k_fwd_brick<2>), grid, blk, 0, st, vol, rot, shifts, out, g, bg, prefix);
  return hipGetLastError();
}

}  // namespace tproj
