// Device helpers shared by the gfx950 kernels of libtproj: complex arithmetic,
// interpolation weights, slice geometry and the Friedel/periodic tap lookup.
//
// Citations name a torch-projectors summary page ("torch-projectors: A
// High-Performance Differentiable Projection Library for PyTorch") by language
// and section.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tproj {

// Geometry as the kernels see it (validated on the host).
struct KGeom {
  int B, P, Bv, Br, Bs;     // Bs = 0 without shifts
  int D, H;                 // volume box, image box
  int half;                 // D / 2
  int W;                    // D / 2 + 1 (stored x extent)
  int Wi;                   // H / 2 + 1 (image row length)
  int npix;                 // H * Wi
  float o;                  // oversampling
  float r2;                 // radius^2, < 0: no cutoff
  float inv_h;              // 1 / H
  float kmax;               // largest |k| of an in-mask pixel
};

// floor() clamped to +-2^24 (NaN -> -2^24) so that the int conversion and the
// tap arithmetic never overflow, whatever the rotation holds.
__device__ __forceinline__ float safe_floor(float p) {
  return fminf(fmaxf(floorf(p), -16777216.0f), 16777216.0f);
}

// p - floor(p) in one instruction (v_fract_f32), for the finite sample
// coordinates of owned pixels; where p - floor(p) rounds up to 1 (p a tiny
// negative number) it returns the largest float below 1, a weight change of
// one ulp.
__device__ __forceinline__ float frac_of(float p) { return __builtin_amdgcn_fractf(p); }

__device__ __forceinline__ float2 cmul(float2 a, float2 b) {
  return make_float2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}
// conj(a) * b
__device__ __forceinline__ float2 cmulc(float2 a, float2 b) {
  return make_float2(a.x * b.x + a.y * b.y, a.x * b.y - a.y * b.x);
}

// Keys cubic convolution weights (Catmull-Rom, a = -1/2; Spanish page 2,
// Dutch page Methodologie, French page 2) for taps floor(p) + {-1, 0, 1, 2}
// at fractional offset f = p - floor(p), expanded in powers of f.
__device__ __forceinline__ void cubic_weights(float f, float w[4]) {
  const float f2 = f * f;
  w[0] = fmaf(fmaf(-0.5f, f, 1.0f), f2, -0.5f * f);   // -f^3/2 + f^2 - f/2
  w[1] = fmaf(fmaf(1.5f, f, -2.5f), f2, 1.0f);        // 3f^3/2 - 5f^2/2 + 1
  w[2] = fmaf(fmaf(-1.5f, f, 2.0f), f2, 0.5f * f);    // -3f^3/2 + 2f^2 + f/2
  w[3] = fmaf(0.5f, f, -0.5f) * f2;                   // f^3/2 - f^2/2
}
// d w / d p of the same four weights.
__device__ __forceinline__ void cubic_dweights(float f, float d[4]) {
  d[0] = fmaf(fmaf(-1.5f, f, 2.0f), f, -0.5f);
  d[1] = fmaf(4.5f, f, -5.0f) * f;
  d[2] = fmaf(fmaf(-4.5f, f, 4.0f), f, 0.5f);
  d[3] = fmaf(1.5f, f, -1.0f) * f;
}
// Linear weights for taps floor(p) + {0, 1}; the derivative is that of the
// cell [floor(p), floor(p) + 1).
__device__ __forceinline__ void linear_weights(float f, float w[2]) { w[0] = 1.0f - f; w[1] = f; }
__device__ __forceinline__ void linear_dweights(float, float d[2]) { d[0] = -1.0f; d[1] = 1.0f; }

template <int NT>
__device__ __forceinline__ void axis_weights(float f, float w[NT]) {
  if constexpr (NT == 4) cubic_weights(f, w); else linear_weights(f, w);
}
template <int NT>
__device__ __forceinline__ void axis_dweights(float f, float d[NT]) {
  if constexpr (NT == 4) cubic_dweights(f, d); else linear_dweights(f, d);
}
// Offset of the first tap from floor(p).
template <int NT>
constexpr int first_tap() { return NT == 4 ? -1 : 0; }

// Image pixel -> frequency: kx = ix (rfftfreq), ky = fftfreq(H)[iy].
__device__ __forceinline__ void pixel_freq(const KGeom& g, int pix, int& kx, int& ky) {
  int iy = pix / g.Wi;
  kx = pix - iy * g.Wi;
  ky = iy < (g.H >> 1) ? iy : iy - g.H;
}

// The pixels start, start + stride, ... of one image with their frequency
// indices, stepped without a division per pixel (pix = iy * Wi + ix; a step
// adds stride / Wi rows and stride mod Wi columns, then carries one row).
struct PixelWalk {
  int pix, iy, ix, drow, dcol;
  __device__ __forceinline__ PixelWalk(const KGeom& g, int start, int stride) : pix(start) {
    iy = start / g.Wi;
    ix = start - iy * g.Wi;
    drow = stride / g.Wi;
    dcol = stride - drow * g.Wi;
  }
  __device__ __forceinline__ void step(const KGeom& g, int stride) {
    pix += stride;
    ix += dcol;
    iy += drow;
    if (ix >= g.Wi) {
      ix -= g.Wi;
      ++iy;
    }
  }
  __device__ __forceinline__ int kx() const { return ix; }
  __device__ __forceinline__ int ky(const KGeom& g) const { return iy < (g.H >> 1) ? iy : iy - g.H; }
};

__device__ __forceinline__ bool in_mask(const KGeom& g, float kx, float ky) {
  return g.r2 < 0.0f || fmaf(kx, kx, ky * ky) <= g.r2;
}

// Fourier shift phase phi = exp(-2 pi i (kx sx + ky sy) / H) (Dutch page,
// Methodologie; French page 2).  The argument, in turns, is reduced to
// [-1/2, 1/2]; the hardware sine and cosine take turns directly and are
// within about one ulp there (measured: 1.3e-7 absolute).
__device__ __forceinline__ float2 shift_phase(float kx, float ky, float sx, float sy, float inv_h) {
  float t = fmaf(kx, sx, ky * sy) * inv_h;   // turns
  t -= rintf(t);
  return make_float2(__builtin_amdgcn_cosf(t), -__builtin_amdgcn_sinf(t));
}

// Wrap an integer tap into [0, D).
__device__ __forceinline__ int wrap_fast(int t, int D) {  // valid for t in [-D, 2D)
  return t < 0 ? t + D : (t >= D ? t - D : t);
}
__device__ __forceinline__ int wrap_any(int t, int D) {
  int r = t % D;
  return r < 0 ? r + D : r;
}

// Stored index of an integer tap (tx, ty, tz) under the per-tap Friedel rule
// (F(-k) = conj F(k); Dutch page Methodologie, French page 2) combined with
// DFT periodicity: m = tx mod D; m <= D/2 -> (tz, ty, m) direct, otherwise the
// Friedel mate (-tz, -ty, D - m), conjugated.
template <bool GENERAL>
__device__ __forceinline__ int64_t tap_index(const KGeom& g, int tx, int ty, int tz, bool& conj) {
  int m = GENERAL ? wrap_any(tx, g.D) : wrap_fast(tx, g.D);
  int x, y, z;
  if (m <= g.half) {
    conj = false; x = m;
    y = GENERAL ? wrap_any(ty, g.D) : wrap_fast(ty, g.D);
    z = GENERAL ? wrap_any(tz, g.D) : wrap_fast(tz, g.D);
  } else {
    conj = true; x = g.D - m;
    y = GENERAL ? wrap_any(-ty, g.D) : wrap_fast(-ty, g.D);
    z = GENERAL ? wrap_any(-tz, g.D) : wrap_fast(-tz, g.D);
  }
  return ((int64_t)z * g.D + y) * g.W + x;
}

}  // namespace tproj
