// Direct (one pixel per lane) kernels of libtproj for gfx950:
//   k_project        3D->2D forward gather (rotated central slice)
//   k_project_real   the same gather on a real volume (weight channel)
//   k_rot_shift_grad rotation / shift gradients, one workgroup per pose
//   k_spread_atomic  adjoint scatter with global float atomics
//   k_zero           fill
// Operation definitions follow the torch-projectors summary pages (Spanish
// page "Resumen tecnico" 2, Dutch page Methodologie, French page "Resume
// technique" 2).
#include "device_common.h"
#include "gather_common.h"
#include "kernels.h"

namespace tproj {

// ---------------------------------------------------------------------------
// Forward: out[b,n,k] = M * phi * I(V[bv], o R (kx,ky,0)).
// grid.x over pixel tiles, grid.y strides over (b, n).
// ---------------------------------------------------------------------------
template <int NT>
__global__ void __launch_bounds__(256) k_project(const float2* __restrict__ vol, const float* __restrict__ rot,
                                                 const float* __restrict__ shifts, float2* __restrict__ out,
                                                 KGeom g) {
  const int pix = blockIdx.x * blockDim.x + threadIdx.x;
  if (pix >= g.npix) return;
  int ikx, iky;
  pixel_freq(g, pix, ikx, iky);
  const float kx = (float)ikx, ky = (float)iky;
  const bool m = in_mask(g, kx, ky);
  const int64_t nvol = (int64_t)g.D * g.D * g.W;
  for (int bn = blockIdx.y; bn < g.B * g.P; bn += gridDim.y) {
    const int b = bn / g.P, n = bn - b * g.P;
    float2 y = make_float2(0.f, 0.f);
    if (m) {
      const float* R = rot + 9 * ((int64_t)(g.Br == 1 ? 0 : b) * g.P + n);
      const float px = g.o * fmaf(R[1], ky, R[0] * kx);
      const float py = g.o * fmaf(R[4], ky, R[3] * kx);
      const float pz = g.o * fmaf(R[7], ky, R[6] * kx);
      float2 I;
      interp_c<NT, false>(vol + nvol * (g.Bv == 1 ? 0 : b), g, px, py, pz, I, nullptr);
      if (shifts) {
        const float* s = shifts + 2 * ((int64_t)(g.Bs == 1 ? 0 : b) * g.P + n);
        I = cmul(shift_phase(kx, ky, s[0], s[1], g.inv_h), I);
      }
      y = I;
    }
    out[(int64_t)bn * g.npix + pix] = y;
  }
}

// Real-volume gather (no phase): out[b,n,k] = M * I(V[bv], p).
template <int NT>
__global__ void __launch_bounds__(256) k_project_real(const float* __restrict__ vol, const float* __restrict__ rot,
                                                      float* __restrict__ out, KGeom g) {
  const int pix = blockIdx.x * blockDim.x + threadIdx.x;
  if (pix >= g.npix) return;
  int ikx, iky;
  pixel_freq(g, pix, ikx, iky);
  const float kx = (float)ikx, ky = (float)iky;
  const bool m = in_mask(g, kx, ky);
  const int64_t nvol = (int64_t)g.D * g.D * g.W;
  for (int bn = blockIdx.y; bn < g.B * g.P; bn += gridDim.y) {
    const int b = bn / g.P, n = bn - b * g.P;
    float y = 0.f;
    if (m) {
      const float* R = rot + 9 * ((int64_t)(g.Br == 1 ? 0 : b) * g.P + n);
      const float px = g.o * fmaf(R[1], ky, R[0] * kx);
      const float py = g.o * fmaf(R[4], ky, R[3] * kx);
      const float pz = g.o * fmaf(R[7], ky, R[6] * kx);
      interp_r<NT, false>(vol + nvol * (g.Bv == 1 ? 0 : b), g, px, py, pz, y, nullptr);
    }
    out[(int64_t)bn * g.npix + pix] = y;
  }
}

// ---------------------------------------------------------------------------
// Rotation / shift gradients, one workgroup of 256 lanes per (b, n):
//   gR[i][j] = o sum_k M (Re(conj(U) phi dI_i(Vc)) + Ur dI_i(Vr)) k3_j,  j < 2
//   gs      = (2 pi / H) sum_k M (kx, ky) Im(conj(U) phi I(Vc))
// Partials are reduced with wavefront shuffles, then across the 4 waves in
// LDS.  Broadcast outputs (Br or Bs == 1 < B) are accumulated atomically.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

template <int NT, bool CPLX, bool REAL>
__global__ void __launch_bounds__(256) k_rot_shift_grad(const float2* __restrict__ volc, const float* __restrict__ volr,
                                                        const float2* __restrict__ U, const float* __restrict__ Ur,
                                                        const float* __restrict__ rot,
                                                        const float* __restrict__ shifts, float* __restrict__ grad_rot,
                                                        float* __restrict__ grad_s, KGeom g) {
  __shared__ float red[4][8];
  const int bn = blockIdx.x;
  const int b = bn / g.P, n = bn - b * g.P;
  const int64_t nvol = (int64_t)g.D * g.D * g.W;
  const float* R = rot + 9 * ((int64_t)(g.Br == 1 ? 0 : b) * g.P + n);
  const float* s = shifts ? shifts + 2 * ((int64_t)(g.Bs == 1 ? 0 : b) * g.P + n) : nullptr;
  const float2* Vc = CPLX ? volc + nvol * (g.Bv == 1 ? 0 : b) : nullptr;
  const float* Vr = REAL ? volr + nvol * (g.Bv == 1 ? 0 : b) : nullptr;
  const float2* Ub = CPLX ? U + (int64_t)bn * g.npix : nullptr;
  const float* Urb = REAL ? Ur + (int64_t)bn * g.npix : nullptr;
  float acc[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) acc[q] = 0.f;
  for (PixelWalk pw(g, threadIdx.x, blockDim.x); pw.pix < g.npix; pw.step(g, blockDim.x)) {
    const int pix = pw.pix;
    const float kx = (float)pw.kx(), ky = (float)pw.ky(g);
    if (!in_mask(g, kx, ky)) continue;
    const float px = g.o * fmaf(R[1], ky, R[0] * kx);
    const float py = g.o * fmaf(R[4], ky, R[3] * kx);
    const float pz = g.o * fmaf(R[7], ky, R[6] * kx);
    float e[3] = {0.f, 0.f, 0.f};
    if constexpr (CPLX) {
      float2 I, dI[3];
      interp_c<NT, true>(Vc, g, px, py, pz, I, dI);
      const float2 u = Ub[pix];
      float2 phi = make_float2(1.f, 0.f);
      if (s) phi = shift_phase(kx, ky, s[0], s[1], g.inv_h);
      // conj(U) * phi, then Re(. * dI_i) and Im(. * I)
      const float2 cu = cmulc(u, phi);
#pragma unroll
      for (int i = 0; i < 3; ++i) e[i] = cu.x * dI[i].x - cu.y * dI[i].y;
      const float im = cu.x * I.y + cu.y * I.x;
      acc[6] = fmaf(kx, im, acc[6]);
      acc[7] = fmaf(ky, im, acc[7]);
    }
    if constexpr (REAL) {
      float I, dI[3];
      interp_r<NT, true>(Vr, g, px, py, pz, I, dI);
      const float w = Urb[pix];
#pragma unroll
      for (int i = 0; i < 3; ++i) e[i] = fmaf(w, dI[i], e[i]);
    }
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      acc[2 * i] = fmaf(e[i], kx, acc[2 * i]);
      acc[2 * i + 1] = fmaf(e[i], ky, acc[2 * i + 1]);
    }
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const float v = wave_sum(acc[q]);
    if (lane == 0) red[wave][q] = v;
  }
  __syncthreads();
  if (threadIdx.x < 8) {
    const int q = threadIdx.x;
    const float v = red[0][q] + red[1][q] + red[2][q] + red[3][q];
    if (q < 6) {
      if (grad_rot) {
        const int i = q >> 1, j = q & 1;
        float* gr = grad_rot + 9 * ((int64_t)(g.Br == 1 ? 0 : b) * g.P + n) + 3 * i + j;
        if (g.Br == 1 && g.B > 1) atomicAdd(gr, g.o * v); else *gr = g.o * v;
      }
    } else if (grad_s && CPLX) {
      float* gs = grad_s + 2 * ((int64_t)(g.Bs == 1 ? 0 : b) * g.P + n) + (q - 6);
      const float val = 6.283185307179586f * g.inv_h * v;
      if (g.Bs == 1 && g.B > 1) atomicAdd(gs, val); else *gs = val;
    }
  }
}

// ---------------------------------------------------------------------------
// Adjoint scatter with global float atomics (the simple reference variant):
// each in-mask pixel adds w * c, c = conj(phi) * Y (conj at mirrored taps),
// and w * Wimg to the weight volume.
// ---------------------------------------------------------------------------
template <int NT, bool WEIGHTS>
__global__ void __launch_bounds__(256) k_spread_atomic(const float2* __restrict__ Y, const float* __restrict__ Wimg,
                                                       const float* __restrict__ rot, const float* __restrict__ shifts,
                                                       float2* __restrict__ Vd, float* __restrict__ Vw, KGeom g) {
  const int pix = blockIdx.x * blockDim.x + threadIdx.x;
  if (pix >= g.npix) return;
  int ikx, iky;
  pixel_freq(g, pix, ikx, iky);
  const float kx = (float)ikx, ky = (float)iky;
  if (!in_mask(g, kx, ky)) return;
  const int64_t nvol = (int64_t)g.D * g.D * g.W;
  for (int bn = blockIdx.y; bn < g.B * g.P; bn += gridDim.y) {
    const int b = bn / g.P, n = bn - b * g.P;
    const float* R = rot + 9 * ((int64_t)(g.Br == 1 ? 0 : b) * g.P + n);
    const float px = g.o * fmaf(R[1], ky, R[0] * kx);
    const float py = g.o * fmaf(R[4], ky, R[3] * kx);
    const float pz = g.o * fmaf(R[7], ky, R[6] * kx);
    float2 c = Y[(int64_t)bn * g.npix + pix];
    if (shifts) {
      const float* s = shifts + 2 * ((int64_t)(g.Bs == 1 ? 0 : b) * g.P + n);
      c = cmulc(shift_phase(kx, ky, s[0], s[1], g.inv_h), c);
    }
    const float wimg = WEIGHTS ? Wimg[(int64_t)bn * g.npix + pix] : 0.f;
    float2* V = Vd + nvol * (g.Bv == 1 ? 0 : b);
    float* VW = WEIGHTS ? Vw + nvol * (g.Bv == 1 ? 0 : b) : nullptr;
    const float flx = safe_floor(px), fly = safe_floor(py), flz = safe_floor(pz);
    float wx[NT], wy[NT], wz[NT];
    axis_weights<NT>(px - flx, wx);
    axis_weights<NT>(py - fly, wy);
    axis_weights<NT>(pz - flz, wz);
    const int x0 = (int)flx + first_tap<NT>(), y0 = (int)fly + first_tap<NT>(), z0 = (int)flz + first_tap<NT>();
#pragma unroll
    for (int cc = 0; cc < NT; ++cc)
#pragma unroll
      for (int bb = 0; bb < NT; ++bb) {
        const float wyz = wy[bb] * wz[cc];
#pragma unroll
        for (int aa = 0; aa < NT; ++aa) {
          bool cj;
          const int64_t idx = tap_index<true>(g, x0 + aa, y0 + bb, z0 + cc, cj);
          const float w = wx[aa] * wyz;
          float* dst = reinterpret_cast<float*>(V + idx);
          unsafeAtomicAdd(dst, w * c.x);
          unsafeAtomicAdd(dst + 1, cj ? -w * c.y : w * c.y);
          if constexpr (WEIGHTS) unsafeAtomicAdd(VW + idx, w * wimg);
        }
      }
  }
}

__global__ void k_zero(float* __restrict__ p, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.f;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
static dim3 pixel_grid(const KGeom& g) {
  const int gy = g.B * g.P < 65535 ? g.B * g.P : 65535;
  return dim3((g.npix + 255) / 256, gy);
}

hipError_t launch_zero(float* p, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_zero, dim3((unsigned)blocks), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

hipError_t launch_project(const KGeom& g, int interp, const float2* vol, const float* rot, const float* shifts,
                          float2* out, hipStream_t st) {
  const dim3 grid = pixel_grid(g), block(256);
  if (interp == 1) hipLaunchKernelGGL((k_project<4>), grid, block, 0, st, vol, rot, shifts, out, g);
  else hipLaunchKernelGGL((k_project<2>), grid, block, 0, st, vol, rot, shifts, out, g);
  return hipGetLastError();
}

hipError_t launch_project_real(const KGeom& g, int interp, const float* vol, const float* rot, float* out,
                               hipStream_t st) {
  const dim3 grid = pixel_grid(g), block(256);
  if (interp == 1) hipLaunchKernelGGL((k_project_real<4>), grid, block, 0, st, vol, rot, out, g);
  else hipLaunchKernelGGL((k_project_real<2>), grid, block, 0, st, vol, rot, out, g);
  return hipGetLastError();
}

template <int NT>
static void launch_grad_nt(const KGeom& g, const float2* volc, const float* volr, const float2* U, const float* Ur,
                           const float* rot, const float* shifts, float* grad_rot, float* grad_s, hipStream_t st) {
  const dim3 grid(g.B * g.P), block(256);
  const bool cp = volc != nullptr, re = volr != nullptr;
  if (cp && re)
    hipLaunchKernelGGL((k_rot_shift_grad<NT, true, true>), grid, block, 0, st, volc, volr, U, Ur, rot, shifts, grad_rot,
                       grad_s, g);
  else if (cp)
    hipLaunchKernelGGL((k_rot_shift_grad<NT, true, false>), grid, block, 0, st, volc, volr, U, Ur, rot, shifts,
                       grad_rot, grad_s, g);
  else if (re)
    hipLaunchKernelGGL((k_rot_shift_grad<NT, false, true>), grid, block, 0, st, volc, volr, U, Ur, rot, shifts,
                       grad_rot, grad_s, g);
}

hipError_t launch_rot_shift_grad(const KGeom& g, int interp, const float2* volc, const float* volr, const float2* U,
                                 const float* Ur, const float* rot, const float* shifts, float* grad_rot,
                                 float* grad_s, hipStream_t st) {
  if (interp == 1) launch_grad_nt<4>(g, volc, volr, U, Ur, rot, shifts, grad_rot, grad_s, st);
  else launch_grad_nt<2>(g, volc, volr, U, Ur, rot, shifts, grad_rot, grad_s, st);
  return hipGetLastError();
}

hipError_t launch_spread_atomic(const KGeom& g, int interp, const float2* Y, const float* Wimg, const float* rot,
                                const float* shifts, float2* Vd, float* Vw, hipStream_t st) {
  const dim3 grid = pixel_grid(g), block(256);
  if (interp == 1) {
    if (Wimg) hipLaunchKernelGGL((k_spread_atomic<4, true>), grid, block, 0, st, Y, Wimg, rot, shifts, Vd, Vw, g);
    else hipLaunchKernelGGL((k_spread_atomic<4, false>), grid, block, 0, st, Y, Wimg, rot, shifts, Vd, Vw, g);
  } else {
    if (Wimg) hipLaunchKernelGGL((k_spread_atomic<2, true>), grid, block, 0, st, Y, Wimg, rot, shifts, Vd, Vw, g);
    else hipLaunchKernelGGL((k_spread_atomic<2, false>), grid, block, 0, st, Y, Wimg, rot, shifts, Vd, Vw, g);
  }
  return hipGetLastError();
}

}  // namespace tproj
