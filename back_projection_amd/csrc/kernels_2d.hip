// 2D -> 2D kernels of libtproj for gfx950: rotation of 2D Fourier data (the
// forward), the accumulation into a 2D reconstruction (its adjoint), and the
// rotation / shift gradients (torch-projectors pages: Dutch Methodologie,
// operations 1 and 2; Spanish "Resumen tecnico" 2; French "Resume technique" 2).
//
// The 2D source is small (a D x (D/2+1) rfft image), so every kernel works on
// its periodic Hermitian extension E[y][x]: a pre-pass writes E once for x, y
// in [-2, D + 2) (the entry of (x mod D, y mod D): as stored for x mod D <=
// D/2, else the conjugated Friedel mate).  A sample's floor is reduced to
// [0, D) once per axis; its taps then lie in the margin-extended box, at fixed
// offsets from the first one -- no per-tap wrap or branch, rows of contiguous
// taps.  The row stride is D + 5 entries, so the bank pair of an 8-byte entry
// changes with both coordinates.
//
// k2_expand     source -> E (complex, or real for the weight channel)
// k2_gather     forward: M * phi * I(E, p); E staged in LDS when it fits
//               (D <= 128), else read from global memory
// k2_grad       rotation / shift gradients: value and derivatives of the
//               interpolant, per-pose block sums, one atomic per term
// k2_img_max    largest |Re|, |Im| (or |w|) of every image: the fixed-point
//               scale of the accumulation
// k2_bp         accumulation of a window of poses at a time into a
//               fixed-point copy of E in LDS (one 64- or 32-bit integer
//               atomic per tap), flushed into per-thread float sums; each
//               workgroup writes its partial E
// k2_bp_direct  degenerate maps, and boxes too large for LDS: float atomics
//               into a partial E in global memory
// k2_fold       partial Es -> stored half-spectrum (direct entry plus, for
//               1 <= x <= D/2 - 1, the conjugated mate), in a fixed order
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "fixed_point_bound.h"
#include "gather_common.h"
#include "kernels_2d.h"

namespace tproj {

namespace {

constexpr int T2 = 1024;        // threads per workgroup (one workgroup per CU when E is in LDS)
constexpr int WIN2 = 16;        // poses per fixed-point window of the accumulation
constexpr float FIX2_RANGE = 0.9f * 2147483648.0f;

__device__ __forceinline__ int pmod_int(int t, int D) {
  t %= D;
  return t < 0 ? t + D : t;
}

__device__ __forceinline__ float2 conj_of(float2 v) { return make_float2(v.x, -v.y); }
__device__ __forceinline__ float conj_of(float v) { return v; }

// ---------------------------------------------------------------------------
// E from the stored half-spectrum: one thread per entry of E.
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256) k2_expand(const T* __restrict__ X, T* __restrict__ E, KGeom g) {
  const int D = g.D, EW = e2_rows(D), ES = e2_stride(D);
  const int64_t n = (int64_t)g.Bv * EW * EW;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int xp = (int)(i % EW);
    const int yp = (int)((i / EW) % EW);
    const int v = (int)(i / ((int64_t)EW * EW));
    const int x = pmod_int(xp - 2, D), y = pmod_int(yp - 2, D);
    const T* Xv = X + (int64_t)v * D * g.W;
    T val;
    if (x <= g.half) val = Xv[(int64_t)y * g.W + x];
    else val = conj_of(Xv[(int64_t)((D - y) % D) * g.W + (D - x)]);
    E[(int64_t)v * e2_size(D) + (int64_t)yp * ES + xp] = val;
  }
}

// 2D sample of image pixel (kx, ky): p = o * R * (kx, ky)^T, R row-major 2x2.
__device__ __forceinline__ void slice_coord2(const KGeom& g, const float* R, float kx, float ky, float& px,
                                             float& py) {
  px = g.o * fmaf(R[1], ky, R[0] * kx);
  py = g.o * fmaf(R[3], ky, R[2] * kx);
}

// floor(p) reduced to [0, D): floor - D floor(floor / D), exact for the
// integer-valued floats that safe_floor returns (one correction step covers
// the rounding of the quotient).
__device__ __forceinline__ int reduce_mod(float fl, const KGeom& g) {
  const float D = (float)g.D;
  float m = fl - D * floorf(fl * (1.0f / D));
  m = m >= D ? m - D : m;
  m = m < 0.f ? m + D : m;
  return (int)m;
}

// Index in E of the first tap of the sample p (NT per axis; the others at
// + b * stride + a), and the fractional parts.
template <int NT>
__device__ __forceinline__ int taps2(const KGeom& g, float px, float py, float& fx, float& fy) {
  const float flx = safe_floor(px), fly = safe_floor(py);
  fx = px - flx;
  fy = py - fly;
  const int x0 = reduce_mod(flx, g), y0 = reduce_mod(fly, g);
  return (y0 + 2 + first_tap<NT>()) * e2_stride(g.D) + (x0 + 2 + first_tap<NT>());
}

__device__ __forceinline__ float2 zero2(float2) { return make_float2(0.f, 0.f); }
__device__ __forceinline__ float zero2(float) { return 0.f; }
__device__ __forceinline__ void fma2(float w, float2 v, float2& a) { a.x = fmaf(w, v.x, a.x); a.y = fmaf(w, v.y, a.y); }
__device__ __forceinline__ void fma2(float w, float v, float& a) { a = fmaf(w, v, a); }

// Value (and with DERIV the derivatives along x and y) of the interpolant.
template <int NT, bool DERIV, typename T>
__device__ __forceinline__ void interp2(const T* E, int base, int ES, const float wx[NT], const float wy[NT],
                                        const float dx[NT], const float dy[NT], T& I, T* dI) {
  I = zero2(T{});
  if constexpr (DERIV) { dI[0] = zero2(T{}); dI[1] = zero2(T{}); }
#pragma unroll
  for (int b = 0; b < NT; ++b) {
    T r = zero2(T{}), rx = zero2(T{});
    const T* row = E + base + b * ES;
#pragma unroll
    for (int a = 0; a < NT; ++a) {
      const T v = row[a];
      fma2(wx[a], v, r);
      if constexpr (DERIV) fma2(dx[a], v, rx);
    }
    fma2(wy[b], r, I);
    if constexpr (DERIV) {
      fma2(wy[b], rx, dI[0]);
      fma2(dy[b], r, dI[1]);
    }
  }
}

// E of volume v into LDS (rows padded as in global memory).
template <typename T>
__device__ __forceinline__ void stage_e(T* lds, const T* __restrict__ E, const KGeom& g, int v) {
  const int n = (int)e2_size(g.D);
  const T* src = E + (int64_t)v * n;
  for (int i = threadIdx.x; i < n; i += blockDim.x) lds[i] = src[i];
}

// ---------------------------------------------------------------------------
// forward gather; grid (NB, Bv): workgroup (w, v) takes the poses w, w + NB,
// ... of volume v's pose list.
// ---------------------------------------------------------------------------
template <int NT, typename T, bool LDS>
__global__ void __launch_bounds__(T2) k2_gather(const T* __restrict__ E, const float* __restrict__ rot,
                                                const float* __restrict__ shifts, T* __restrict__ out, KGeom g,
                                                int list_len) {
  extern __shared__ __align__(16) unsigned char smem2[];
  const int vsel = blockIdx.y;
  const T* src = E + (int64_t)vsel * e2_size(g.D);
  const int ES = e2_stride(g.D);
  if constexpr (LDS) {
    stage_e((T*)smem2, E, g, vsel);
    __syncthreads();
    src = (const T*)smem2;
  }
  constexpr bool CPLX = sizeof(T) == 8;
  for (int e = blockIdx.x; e < list_len; e += gridDim.x) {
    int bimg, n;
    list_entry(g, vsel, e, bimg, n);
    const float* R = rot + 4 * ((int64_t)(g.Br == 1 ? 0 : bimg) * g.P + n);
    float sx = 0.f, sy = 0.f;
    if (CPLX && shifts) {
      const float* s = shifts + 2 * ((int64_t)(g.Bs == 1 ? 0 : bimg) * g.P + n);
      sx = s[0];
      sy = s[1];
    }
    T* O = out + ((int64_t)bimg * g.P + n) * g.npix;
    for (PixelWalk pw(g, threadIdx.x, blockDim.x); pw.pix < g.npix; pw.step(g, blockDim.x)) {
      const int pix = pw.pix;
      const float kx = (float)pw.kx(), ky = (float)pw.ky(g);
      if (!in_mask(g, kx, ky)) { O[pix] = zero2(T{}); continue; }
      float px, py, fx, fy, wx[NT], wy[NT];
      slice_coord2(g, R, kx, ky, px, py);
      const int base = taps2<NT>(g, px, py, fx, fy);
      axis_weights<NT>(fx, wx);
      axis_weights<NT>(fy, wy);
      T I;
      interp2<NT, false>(src, base, ES, wx, wy, wx, wy, I, (T*)nullptr);
      if constexpr (CPLX) {
        if (shifts) I = cmul(shift_phase(kx, ky, sx, sy, g.inv_h), I);
      }
      O[pix] = I;
    }
  }
}

// ---------------------------------------------------------------------------
// rotation / shift gradients:
//   gR[i][j] += o * sum_k M (Re(conj(U) phi dI_i(Ec)) + Ur dI_i(Er)) k_j
//   gs       += (2 pi / H) sum_k M (kx, ky) Im(conj(U) phi I(Ec))
// Each thread sums its pixels of the pose; the workgroup adds the six sums
// and one thread adds them to the outputs (zeroed first; atomics, since
// broadcast maps collect several batch entries).
// ---------------------------------------------------------------------------
template <int N>
__device__ __forceinline__ void block_sum(float (&v)[N], float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int q = 0; q < N; ++q)
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v[q] += __shfl_xor(v[q], off, 64);
  if (lane == 0)
#pragma unroll
    for (int q = 0; q < N; ++q) red[wave * N + q] = v[q];
  __syncthreads();
  if (threadIdx.x < N) {
    float s = 0.f;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) s += red[w * N + threadIdx.x];
    red[16 * N + threadIdx.x] = s;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < N; ++q) v[q] = red[16 * N + q];
  __syncthreads();
}

template <int NT, bool CPLX, bool REAL, bool LDS>
__global__ void __launch_bounds__(T2) k2_grad(const float2* __restrict__ Ec, const float* __restrict__ Er,
                                              const float2* __restrict__ U, const float* __restrict__ Ur,
                                              const float* __restrict__ rot, const float* __restrict__ shifts,
                                              float* __restrict__ grad_rot, float* __restrict__ grad_s, KGeom g,
                                              int list_len) {
  extern __shared__ __align__(16) unsigned char smem2[];
  __shared__ float red[17 * 6];
  const int vsel = blockIdx.y;
  const int64_t ne = e2_size(g.D);
  const int ES = e2_stride(g.D);
  const float2* srcc = CPLX ? Ec + vsel * ne : nullptr;
  const float* srcr = REAL ? Er + vsel * ne : nullptr;
  if constexpr (LDS) {
    float2* lc = (float2*)smem2;
    float* lr = (float*)(smem2 + (CPLX ? ne * sizeof(float2) : 0));
    if constexpr (CPLX) stage_e(lc, Ec, g, vsel);
    if constexpr (REAL) stage_e(lr, Er, g, vsel);
    __syncthreads();
    srcc = lc;
    srcr = lr;
  }
  for (int e = blockIdx.x; e < list_len; e += gridDim.x) {
    int bimg, n;
    list_entry(g, vsel, e, bimg, n);
    const int64_t pose_r = (int64_t)(g.Br == 1 ? 0 : bimg) * g.P + n;
    const float* R = rot + 4 * pose_r;
    float sx = 0.f, sy = 0.f;
    if (CPLX && shifts) {
      const float* s = shifts + 2 * ((int64_t)(g.Bs == 1 ? 0 : bimg) * g.P + n);
      sx = s[0];
      sy = s[1];
    }
    const int64_t img = ((int64_t)bimg * g.P + n) * g.npix;
    float acc[6] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (PixelWalk pw(g, threadIdx.x, blockDim.x); pw.pix < g.npix; pw.step(g, blockDim.x)) {
      const int pix = pw.pix;
      const float kx = (float)pw.kx(), ky = (float)pw.ky(g);
      if (!in_mask(g, kx, ky)) continue;
      float px, py, fx, fy, wx[NT], wy[NT], dx[NT], dy[NT];
      slice_coord2(g, R, kx, ky, px, py);
      const int base = taps2<NT>(g, px, py, fx, fy);
      axis_weights<NT>(fx, wx);
      axis_weights<NT>(fy, wy);
      axis_dweights<NT>(fx, dx);
      axis_dweights<NT>(fy, dy);
      float e0 = 0.f, e1 = 0.f, im = 0.f;
      if constexpr (CPLX) {
        float2 I, dI[2];
        interp2<NT, true>(srcc, base, ES, wx, wy, dx, dy, I, dI);
        float2 phi = make_float2(1.f, 0.f);
        if (shifts) phi = shift_phase(kx, ky, sx, sy, g.inv_h);
        const float2 cc = cmulc(U[img + pix], phi);   // conj(U) * phi
        e0 = cc.x * dI[0].x - cc.y * dI[0].y;
        e1 = cc.x * dI[1].x - cc.y * dI[1].y;
        im = cc.x * I.y + cc.y * I.x;
      }
      if constexpr (REAL) {
        float I, dI[2];
        interp2<NT, true>(srcr, base, ES, wx, wy, dx, dy, I, dI);
        const float ur = Ur[img + pix];
        e0 = fmaf(ur, dI[0], e0);
        e1 = fmaf(ur, dI[1], e1);
      }
      acc[0] = fmaf(e0, kx, acc[0]);
      acc[1] = fmaf(e0, ky, acc[1]);
      acc[2] = fmaf(e1, kx, acc[2]);
      acc[3] = fmaf(e1, ky, acc[3]);
      acc[4] = fmaf(im, kx, acc[4]);
      acc[5] = fmaf(im, ky, acc[5]);
    }
    block_sum(acc, red);
    if (threadIdx.x == 0) {
      if (grad_rot)
        for (int q = 0; q < 4; ++q) atomicAdd(grad_rot + 4 * pose_r + q, g.o * acc[q]);
      if (CPLX && grad_s) {
        float* gs = grad_s + 2 * ((int64_t)(g.Bs == 1 ? 0 : bimg) * g.P + n);
        atomicAdd(gs, 6.283185307179586f * g.inv_h * acc[4]);
        atomicAdd(gs + 1, 6.283185307179586f * g.inv_h * acc[5]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Largest max(|Re|, |Im|) (data) or |w| (weights) over the in-mask pixels of
// every image (one workgroup per image).
// ---------------------------------------------------------------------------
template <bool WEIGHTS>
__global__ void __launch_bounds__(256) k2_img_max(const float2* __restrict__ Y, const float* __restrict__ Wimg,
                                                  float* __restrict__ mx, KGeom g) {
  __shared__ float red[4];
  for (int bn = blockIdx.x; bn < g.B * g.P; bn += gridDim.x) {
    float m = 0.f;
    for (PixelWalk pw(g, threadIdx.x, blockDim.x); pw.pix < g.npix; pw.step(g, blockDim.x)) {
      const int pix = pw.pix;
      if (!in_mask(g, (float)pw.kx(), (float)pw.ky(g))) continue;
      if constexpr (WEIGHTS) m = fmaxf(m, fabsf(Wimg[(int64_t)bn * g.npix + pix]));
      else {
        const float2 v = Y[(int64_t)bn * g.npix + pix];
        m = fmaxf(m, fmaxf(fabsf(v.x), fabsf(v.y)));
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) mx[bn] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
  }
}

// Bound on the sum of |weights| that one entry of E receives from all pixels
// of one pose, its periodic translates included (fixed_point_bound.h).
// Degenerate maps get infinity (they take the direct kernel).
template <int NT>
__device__ __forceinline__ float weight_sum_bound2(const KGeom& g, const float* R) {
  return weight_sum_bound_2d<NT>(g.o, g.kmax, g.D, R);
}

__device__ __forceinline__ bool pose2_ok(float c) { return c <= 4096.0f; }

// 2^22 > |w u|: the magic-number rounding (bits = 0x4B400000 + k).
__device__ __forceinline__ int fix_round2(float w, float u) {
  return __float_as_int(fmaf(w, u, 12582912.0f)) - 0x4B400000;
}
__device__ __forceinline__ unsigned long long fix_pair2(float w, float ur, float ui) {
  const unsigned long long lo = __float_as_uint(fmaf(w, ur, 12582912.0f));
  const unsigned long long hi = __float_as_uint(fmaf(w, ui, 12582912.0f));
  return ((hi << 32) | lo) - 0x4B4000004B400000ull;
}
__device__ __forceinline__ void unpack2(unsigned long long v, float& re, float& im) {
  const int lo = (int)(unsigned)(v & 0xffffffffull);
  const int hi = (int)(unsigned)(v >> 32) + (lo < 0 ? 1 : 0);   // undo the borrow of a negative low word
  re = (float)lo;
  im = (float)hi;
}

// ---------------------------------------------------------------------------
// Accumulation of images (WEIGHTS: weight images) into partial Es.  Grid (NB,
// Bv): workgroup (w, v) takes the poses w, w + NB, ... of volume v's list,
// WIN2 at a time: the window's fixed-point scale keeps every sum below 2^31
// (sqrt(2) m c <= lim for the window's largest value m and summed bound c),
// then each pose's pixels add their taps with 64-bit (data) or 32-bit
// (weights) integer atomics; after the window, the tile is added to the
// thread's float sums.  Degenerate maps are left to k2_bp_direct.
// ---------------------------------------------------------------------------
template <int NT, bool WEIGHTS>
__global__ void __launch_bounds__(T2) k2_bp(const float2* __restrict__ Y, const float* __restrict__ Wimg,
                                            const float* __restrict__ rot, const float* __restrict__ shifts,
                                            const float* __restrict__ mx, void* __restrict__ parts, KGeom g,
                                            int list_len) {
  using Acc = typename std::conditional<WEIGHTS, unsigned int, unsigned long long>::type;
  extern __shared__ __align__(16) unsigned char smem2[];
  __shared__ float win_c[WIN2], win_m[WIN2];
  __shared__ float win_scale;
  Acc* acc_t = (Acc*)smem2;
  const int vsel = blockIdx.y;
  const int ne = (int)e2_size(g.D), ES = e2_stride(g.D);
  constexpr int PER = 18;   // entries per thread: ceil(132 * 133 / 1024), D <= 128
  float2 sum[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) sum[i] = make_float2(0.f, 0.f);
  for (int i = threadIdx.x; i < ne; i += blockDim.x) acc_t[i] = 0;
  __syncthreads();
  for (int e0 = blockIdx.x; e0 < list_len; e0 += WIN2 * gridDim.x) {
    // ---- the window's scale ----
    if (threadIdx.x < WIN2) {
      const int e = e0 + threadIdx.x * gridDim.x;
      float c = 0.f, m = 0.f;
      if (e < list_len) {
        int bimg, n;
        list_entry(g, vsel, e, bimg, n);
        const float cb = weight_sum_bound2<NT>(g, rot + 4 * ((int64_t)(g.Br == 1 ? 0 : bimg) * g.P + n));
        if (pose2_ok(cb)) {
          c = cb;
          m = mx[(int64_t)bimg * g.P + n];
        }
      }
      win_c[threadIdx.x] = c;
      win_m[threadIdx.x] = m;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      float c = 0.f, m = 0.f;
      for (int j = 0; j < WIN2; ++j) { c += win_c[j]; m = fmaxf(m, win_m[j]); }
      const float lim = fminf(FIX2_RANGE, 0.99f * 4194304.0f * c);
      win_scale = (m > 0.f && c > 0.f) ? lim / ((WEIGHTS ? 1.0f : 1.41421356f) * m * c) : 0.f;
    }
    __syncthreads();
    const float scale = win_scale;
    for (int j = 0; j < WIN2; ++j) {
      const int e = e0 + j * gridDim.x;
      if (e >= list_len || win_c[j] == 0.f || scale == 0.f) continue;   // block-uniform
      int bimg, n;
      list_entry(g, vsel, e, bimg, n);
      const float* R = rot + 4 * ((int64_t)(g.Br == 1 ? 0 : bimg) * g.P + n);
      float sx = 0.f, sy = 0.f;
      if (!WEIGHTS && shifts) {
        const float* s = shifts + 2 * ((int64_t)(g.Bs == 1 ? 0 : bimg) * g.P + n);
        sx = s[0];
        sy = s[1];
      }
      const int64_t img = ((int64_t)bimg * g.P + n) * g.npix;
      for (PixelWalk pw(g, threadIdx.x, blockDim.x); pw.pix < g.npix; pw.step(g, blockDim.x)) {
        const int pix = pw.pix;
        const float kx = (float)pw.kx(), ky = (float)pw.ky(g);
        if (!in_mask(g, kx, ky)) continue;
        float px, py, fx, fy, wx[NT], wy[NT];
          slice_coord2(g, R, kx, ky, px, py);
        const int base = taps2<NT>(g, px, py, fx, fy);
        axis_weights<NT>(fx, wx);
        axis_weights<NT>(fy, wy);
        float2 c;
        if constexpr (WEIGHTS) {
          c = make_float2(Wimg[img + pix] * scale, 0.f);
        } else {
          c = Y[img + pix];
          if (shifts) c = cmulc(shift_phase(kx, ky, sx, sy, g.inv_h), c);   // conj(phi) * Y
          c.x *= scale;
          c.y *= scale;
        }
#pragma unroll
        for (int b = 0; b < NT; ++b) {
          const float ur = wy[b] * c.x, ui = wy[b] * c.y;
          Acc* row = acc_t + base + b * ES;
#pragma unroll
          for (int a = 0; a < NT; ++a) {
            if constexpr (WEIGHTS) atomicAdd(&row[a], (unsigned int)fix_round2(wx[a], ur));
            else atomicAdd(&row[a], fix_pair2(wx[a], ur, ui));
          }
        }
      }
    }
    __syncthreads();
    // ---- flush the window ----
    const float inv = scale > 0.f ? 1.0f / scale : 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int k = threadIdx.x + i * T2;
      if (k >= ne) break;
      const Acc u = acc_t[k];
      if (u != 0) {
        if constexpr (WEIGHTS) {
          sum[i].x = fmaf((float)(int)u, inv, sum[i].x);
        } else {
          float re, im;
          unpack2(u, re, im);
          sum[i].x = fmaf(re, inv, sum[i].x);
          sum[i].y = fmaf(im, inv, sum[i].y);
        }
        acc_t[k] = 0;
      }
    }
    __syncthreads();
  }
  // ---- this workgroup's partial E ----
  const int64_t slot = ((int64_t)vsel * gridDim.x + blockIdx.x) * ne;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int k = threadIdx.x + i * T2;
    if (k >= ne) break;
    if constexpr (WEIGHTS) ((float*)parts)[slot + k] = sum[i].x;
    else ((float2*)parts)[slot + k] = sum[i];
  }
}

// Direct accumulation with float atomics into partial slot 0 of every volume
// (ALL: every pose, for boxes whose E does not fit LDS; else only the
// degenerate maps).  One workgroup per pose.
template <int NT, bool WEIGHTS, bool ALL>
__global__ void __launch_bounds__(256) k2_bp_direct(const float2* __restrict__ Y, const float* __restrict__ Wimg,
                                                    const float* __restrict__ rot, const float* __restrict__ shifts,
                                                    void* __restrict__ parts, KGeom g, int nparts) {
  const int64_t ne = e2_size(g.D);
  const int ES = e2_stride(g.D);
  for (int bn = blockIdx.x; bn < g.B * g.P; bn += gridDim.x) {
    const int bimg = bn / g.P, n = bn - bimg * g.P;
    const float* R = rot + 4 * ((int64_t)(g.Br == 1 ? 0 : bimg) * g.P + n);
    if (!ALL && pose2_ok(weight_sum_bound2<NT>(g, R))) continue;
    const int v = g.Bv == 1 ? 0 : bimg;
    const int64_t slot = (int64_t)v * nparts * ne;
    float sx = 0.f, sy = 0.f;
    if (!WEIGHTS && shifts) {
      const float* s = shifts + 2 * ((int64_t)(g.Bs == 1 ? 0 : bimg) * g.P + n);
      sx = s[0];
      sy = s[1];
    }
    for (PixelWalk pw(g, threadIdx.x, blockDim.x); pw.pix < g.npix; pw.step(g, blockDim.x)) {
      const int pix = pw.pix;
      const float kx = (float)pw.kx(), ky = (float)pw.ky(g);
      if (!in_mask(g, kx, ky)) continue;
      float px, py, fx, fy, wx[NT], wy[NT];
      slice_coord2(g, R, kx, ky, px, py);
      const int base = taps2<NT>(g, px, py, fx, fy);
      axis_weights<NT>(fx, wx);
      axis_weights<NT>(fy, wy);
      float2 c;
      if constexpr (WEIGHTS) {
        c = make_float2(Wimg[(int64_t)bn * g.npix + pix], 0.f);
      } else {
        c = Y[(int64_t)bn * g.npix + pix];
        if (shifts) c = cmulc(shift_phase(kx, ky, sx, sy, g.inv_h), c);
      }
      for (int b = 0; b < NT; ++b)
        for (int a = 0; a < NT; ++a) {
          const float w = wx[a] * wy[b];
          const int64_t k = slot + base + b * ES + a;
          if constexpr (WEIGHTS) unsafeAtomicAdd((float*)parts + k, w * c.x);
          else {
            unsafeAtomicAdd((float*)parts + 2 * k, w * c.x);
            unsafeAtomicAdd((float*)parts + 2 * k + 1, w * c.y);
          }
        }
    }
  }
}

// Sum of the entries of E at (x + i D, y + j D), i, j in {-1, 0, 1}, inside
// the margin-extended box [-2, D + 2)^2 (every tap that aliases to (x, y)).
template <typename T>
__device__ __forceinline__ T periodic_sum(const T* E, int D, int x, int y) {
  T s = zero2(T{});
  const int ES = e2_stride(D);
#pragma unroll
  for (int j = -1; j <= 1; ++j) {
    const int yy = y + j * D;
    if (yy < -2 || yy >= D + 2) continue;
#pragma unroll
    for (int i = -1; i <= 1; ++i) {
      const int xx = x + i * D;
      if (xx < -2 || xx >= D + 2) continue;
      const T v = E[(int64_t)(yy + 2) * ES + (xx + 2)];
      if constexpr (sizeof(T) == 8) { s.x += v.x; s.y += v.y; }
      else s += v;
    }
  }
  return s;
}

// Stored entry (v, y, x) = sum over the partial Es of every position that
// aliases to (x, y) and, for 1 <= x <= D/2 - 1, of the conjugate of every
// position that aliases to the Friedel mate (D - x, -y mod D) (no conjugate
// for the real weight channel), in a fixed order.  A workgroup takes
// FOLD_E consecutive entries; its FOLD_S slices of threads each sum every
// FOLD_S-th partial, and the slices are then added in slice order, so the
// result does not depend on scheduling.
constexpr int FOLD_E = 16, FOLD_S = 16;

template <typename T>
__global__ void __launch_bounds__(FOLD_E * FOLD_S) k2_fold(const T* __restrict__ parts, T* __restrict__ out,
                                                           KGeom g, int nparts) {
  __shared__ T red[FOLD_S][FOLD_E];
  const int D = g.D;
  const int64_t ne = e2_size(D);
  const int64_t n = (int64_t)g.Bv * D * g.W;
  const int le = threadIdx.x % FOLD_E, sl = threadIdx.x / FOLD_E;
  for (int64_t i0 = (int64_t)blockIdx.x * FOLD_E; i0 < n; i0 += (int64_t)gridDim.x * FOLD_E) {
    const int64_t i = i0 + le;
    T s = zero2(T{});
    if (i < n) {
      const int x = (int)(i % g.W);
      const int y = (int)((i / g.W) % D);
      const int v = (int)(i / ((int64_t)g.W * D));
      const bool mate = x >= 1 && x <= g.half - 1;
      for (int p = sl; p < nparts; p += FOLD_S) {
        const T* E = parts + ((int64_t)v * nparts + p) * ne;
        const T a = periodic_sum(E, D, x, y);
        if constexpr (sizeof(T) == 8) {
          s.x += a.x;
          s.y += a.y;
          if (mate) {
            const T b = periodic_sum(E, D, D - x, (D - y) % D);
            s.x += b.x;
            s.y -= b.y;
          }
        } else {
          s += a;
          if (mate) s += periodic_sum(E, D, D - x, (D - y) % D);
        }
      }
    }
    red[sl][le] = s;
    __syncthreads();
    if (sl == 0 && i < n) {
      T t = red[0][le];
#pragma unroll
      for (int k = 1; k < FOLD_S; ++k) {
        if constexpr (sizeof(T) == 8) {
          t.x += red[k][le].x;
          t.y += red[k][le].y;
        } else t += red[k][le];
      }
      out[i] = t;
    }
    __syncthreads();
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
int twod_lds_fits(const KGeom& g, size_t bytes_per_entry) {
  return (size_t)e2_size(g.D) * bytes_per_entry <= (size_t)150 * 1024 && g.D <= 128;
}

static int list_len2(const KGeom& g) { return (g.Bv == 1 ? g.B : 1) * g.P; }

// Dynamic LDS above the default per-workgroup limit must be allowed per kernel.
template <typename K>
static void allow_lds(K kernel, size_t bytes) {
  if (bytes > 0) (void)hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}
static unsigned blocks_for(int64_t n) {
  int64_t b = (n + 255) / 256;
  return (unsigned)(b < 1 ? 1 : (b > 8192 ? 8192 : b));
}

int twod_parts(const KGeom& g) {
  const int per_vol = list_len2(g);
  int nb = 256 / (g.Bv < 256 ? g.Bv : 256);
  if (nb < 1) nb = 1;
  return per_vol < nb ? per_vol : nb;
}

hipError_t launch2_expand_c(const KGeom& g, const float2* X, float2* E, hipStream_t st) {
  hipLaunchKernelGGL((k2_expand<float2>), dim3(blocks_for((int64_t)g.Bv * e2_size(g.D))), dim3(256), 0, st, X, E, g);
  return hipGetLastError();
}
hipError_t launch2_expand_r(const KGeom& g, const float* X, float* E, hipStream_t st) {
  hipLaunchKernelGGL((k2_expand<float>), dim3(blocks_for((int64_t)g.Bv * e2_size(g.D))), dim3(256), 0, st, X, E, g);
  return hipGetLastError();
}

template <typename T>
static hipError_t gather_t(const KGeom& g, int interp, const T* E, const float* rot, const float* shifts, T* out,
                           hipStream_t st) {
  const int L = list_len2(g);
  const bool lds = twod_lds_fits(g, sizeof(T));
  const size_t sh = lds ? (size_t)e2_size(g.D) * sizeof(T) : 0;
  const dim3 grid(L < twod_parts(g) ? L : twod_parts(g), g.Bv), blk(T2);
#define TP2(NT_, L_)                                                                    \
  do {                                                                                  \
    allow_lds(k2_gather<NT_, T, L_>, sh);                                               \
    hipLaunchKernelGGL((k2_gather<NT_, T, L_>), grid, blk, sh, st, E, rot, shifts, out, g, L); \
  } while (0)
  if (interp == 1) { if (lds) TP2(4, true); else TP2(4, false); }
  else { if (lds) TP2(2, true); else TP2(2, false); }
#undef TP2
  return hipGetLastError();
}

hipError_t launch2_gather_c(const KGeom& g, int interp, const float2* E, const float* rot, const float* shifts,
                            float2* out, hipStream_t st) {
  return gather_t<float2>(g, interp, E, rot, shifts, out, st);
}
hipError_t launch2_gather_r(const KGeom& g, int interp, const float* E, const float* rot, float* out,
                            hipStream_t st) {
  return gather_t<float>(g, interp, E, rot, nullptr, out, st);
}

hipError_t launch2_grad(const KGeom& g, int interp, const float2* Ec, const float* Er, const float2* U,
                        const float* Ur, const float* rot, const float* shifts, float* grad_rot, float* grad_s,
                        hipStream_t st) {
  const int L = list_len2(g);
  const bool c = Ec != nullptr, r = Er != nullptr;
  const size_t per = (c ? sizeof(float2) : 0) + (r ? sizeof(float) : 0);
  const bool lds = twod_lds_fits(g, per);
  // Both channels together may not fit in LDS where each one does: then one
  // launch per channel (the gradient terms of the two add up through the same
  // atomics; the real channel has no phase, so no shift term).
  if (c && r && !lds && twod_lds_fits(g, sizeof(float2))) {
    const hipError_t e = launch2_grad(g, interp, Ec, nullptr, U, nullptr, rot, shifts, grad_rot, grad_s, st);
    if (e != hipSuccess) return e;
    return launch2_grad(g, interp, nullptr, Er, nullptr, Ur, rot, shifts, grad_rot, grad_s, st);
  }
  const size_t sh = lds ? (size_t)e2_size(g.D) * per : 0;
  const dim3 grid(L < twod_parts(g) ? L : twod_parts(g), g.Bv), blk(T2);
#define TP2G(NT_, C_, R_)                                                                                         \
  do {                                                                                                            \
    if (lds) {                                                                                                    \
      allow_lds(k2_grad<NT_, C_, R_, true>, sh);                                                                  \
      hipLaunchKernelGGL((k2_grad<NT_, C_, R_, true>), grid, blk, sh, st, Ec, Er, U, Ur, rot, shifts, grad_rot,    \
                         grad_s, g, L);                                                                           \
    }                                                                                                             \
    else hipLaunchKernelGGL((k2_grad<NT_, C_, R_, false>), grid, blk, 0, st, Ec, Er, U, Ur, rot, shifts, grad_rot, \
                            grad_s, g, L);                                                                        \
  } while (0)
  if (interp == 1) {
    if (c && r) TP2G(4, true, true); else if (c) TP2G(4, true, false); else if (r) TP2G(4, false, true);
  } else {
    if (c && r) TP2G(2, true, true); else if (c) TP2G(2, true, false); else if (r) TP2G(2, false, true);
  }
#undef TP2G
  return hipGetLastError();
}

size_t twod_bp_parts_bytes(const KGeom& g, bool weights) {
  const size_t ne = (size_t)e2_size(g.D);
  const size_t np = twod_lds_fits(g, sizeof(unsigned long long)) ? (size_t)twod_parts(g) : 1;
  return (size_t)g.Bv * np * ne * (sizeof(float2) + (weights ? sizeof(float) : 0));
}

hipError_t launch2_bp(const KGeom& g, int interp, const float2* Y, const float* Wimg, const float* rot,
                      const float* shifts, float* mx, void* parts, float2* out, float* wout, hipStream_t st) {
  const int L = list_len2(g);
  const bool lds = twod_lds_fits(g, sizeof(unsigned long long));
  const int np = lds ? twod_parts(g) : 1;
  const size_t ne = (size_t)e2_size(g.D);
  float2* pc = (float2*)parts;
  float* pw = (float*)(pc + (size_t)g.Bv * np * ne);
  const dim3 eg(g.B * g.P < 16384 ? g.B * g.P : 16384);
  for (int ch = 0; ch < (Wimg ? 2 : 1); ++ch) {
    const bool W = ch == 1;
    void* P = W ? (void*)pw : (void*)pc;
    if (lds) {
      if (W) hipLaunchKernelGGL((k2_img_max<true>), eg, dim3(256), 0, st, Y, Wimg, mx, g);
      else hipLaunchKernelGGL((k2_img_max<false>), eg, dim3(256), 0, st, Y, Wimg, mx, g);
      const dim3 grid(np, g.Bv), blk(T2);
      const size_t sh = ne * (W ? sizeof(unsigned int) : sizeof(unsigned long long));
#define TP2B(NT_, W_)                                                                          \
  do {                                                                                         \
    allow_lds(k2_bp<NT_, W_>, sh);                                                             \
    hipLaunchKernelGGL((k2_bp<NT_, W_>), grid, blk, sh, st, Y, Wimg, rot, shifts, mx, P, g, L); \
  } while (0)
      if (interp == 1) { if (W) TP2B(4, true); else TP2B(4, false); }
      else { if (W) TP2B(2, true); else TP2B(2, false); }
#undef TP2B
    } else {
      hipError_t e = launch_zero((float*)P, (int64_t)g.Bv * ne * (W ? 1 : 2), st);
      if (e != hipSuccess) return e;
    }
#define TP2D(NT_, W_, A_) hipLaunchKernelGGL((k2_bp_direct<NT_, W_, A_>), eg, dim3(256), 0, st, Y, Wimg, rot, shifts, P, g, np)
    if (interp == 1) {
      if (W) { if (lds) TP2D(4, true, false); else TP2D(4, true, true); }
      else { if (lds) TP2D(4, false, false); else TP2D(4, false, true); }
    } else {
      if (W) { if (lds) TP2D(2, true, false); else TP2D(2, true, true); }
      else { if (lds) TP2D(2, false, false); else TP2D(2, false, true); }
    }
#undef TP2D
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t ng = ((int64_t)g.Bv * g.D * g.W + FOLD_E - 1) / FOLD_E;
    const dim3 fb((unsigned)(ng < 16384 ? ng : 16384)), ft(FOLD_E * FOLD_S);
    if (W) hipLaunchKernelGGL((k2_fold<float>), fb, ft, 0, st, pw, wout, g, np);
    else hipLaunchKernelGGL((k2_fold<float2>), fb, ft, 0, st, pc, out, g, np);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace tproj
