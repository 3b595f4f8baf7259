/*
 * Fourier-slice projection oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 CPU implementation of the differentiable central-slice
 * projector described on the torch-projectors pages ("torch-projectors: A
 * High-Performance Differentiable Projection Library for PyTorch", summaries in
 * Spanish, Dutch, French and Hindi).  Only the test suite, the smoke check and
 * the benchmark's CPU-baseline leg may load it.  It shares no code, header or
 * table with the GPU library, and the GPU library never calls it.
 *
 * Citation tags used below name a summary page by language and its section:
 *   [es TS2]  Spanish page, "Resumen tecnico" section 2 (Metodologia)
 *   [nl M]    Dutch page,   "Technische samenvatting", Methodologie
 *   [fr TS2]  French page,  "Resume technique" section 2 (Methodologie)
 *   [hi 4]    Hindi page,   lay section 4 (Friedel symmetry)
 *
 * What the pages fix, and where this file takes a reading of its own (each
 * reading is listed with its reason in the design notes of the repository):
 *   - rfft half-spectrum layout, FFTW/PyTorch conventions [es TS2, fr TS2]:
 *     volume V[z][y][x], x = 0..D/2 is the halved axis, z and y in fftfreq
 *     order; image Y[iy][ix], ix = 0..H/2 = kx, iy -> ky in fftfreq order.
 *   - 3D->2D forward is the rotated central slice [es TS2, nl M, fr TS2];
 *     reading: sample p = o * R * (kx, ky, 0)^T, R rows/cols ordered (x,y,z).
 *   - linear or cubic Catmull-Rom (Keys) interpolation with a = -0.5
 *     [es TS2, nl M, fr TS2]; the kernel is written from Keys' piecewise
 *     definition at the tap distance d = p - t.
 *   - Friedel symmetry F(-k) = conj(F(k)) [nl M, fr TS2, hi 4]; reading: it is
 *     applied to every tap separately, together with DFT periodicity.
 *   - shifts by Fourier phase modulation (shift theorem) [nl M, fr TS2];
 *     reading: phi = exp(-2 pi i (kx sx + ky sy) / H).
 *   - 2D->3D back-projection accumulates images (and real weights, for CTF
 *     correction [fr TS2]) into the volume; reading: it is the exact adjoint of
 *     the forward under <a,b> = Re sum conj(a) b over stored entries.
 *   - every op is differentiable w.r.t. its inputs, rotations and shifts
 *     [es TS2, nl M]; complex gradients follow dL/dRe + i dL/dIm.
 *   - radius cutoff (reading): pixel kept iff r < 0 or kx^2 + ky^2 <= r^2.
 *   - 2D -> 2D forward and backward [nl M, es TS2, fr TS2]: the same
 *     definitions one dimension down (2x2 map, 2D rfft source); see the
 *     section of that name below.
 *
 * All entry points return 0 on success and a negative value on a bad argument.
 * Complex arrays are interleaved (re, im) doubles.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ */
/* Interpolation kernels                                               */
/* ------------------------------------------------------------------ */

/* Keys cubic convolution kernel W(d) with a = -1/2 (Catmull-Rom), written
 * from its piecewise definition [es TS2, fr TS2]:
 *   |d| <= 1 : (a+2)|d|^3 - (a+3)|d|^2 + 1
 *   1<|d|<2  : a|d|^3 - 5a|d|^2 + 8a|d| - 4a
 *   else     : 0                                                        */
static double keys_w(double d) {
  const double a = -0.5;
  double x = fabs(d);
  if (x <= 1.0) return (a + 2.0) * x * x * x - (a + 3.0) * x * x + 1.0;
  if (x < 2.0) return a * x * x * x - 5.0 * a * x * x + 8.0 * a * x - 4.0 * a;
  return 0.0;
}

/* dW/dd of the Keys kernel (continuous: the kernel is C1). */
static double keys_dw(double d) {
  const double a = -0.5;
  double x = fabs(d), s = d < 0.0 ? -1.0 : 1.0;
  if (x <= 1.0) return s * (3.0 * (a + 2.0) * x * x - 2.0 * (a + 3.0) * x);
  if (x < 2.0) return s * (3.0 * a * x * x - 10.0 * a * x + 8.0 * a);
  return 0.0;
}

/* Linear ("tent") kernel W(d) = 1 - |d| on |d| < 1 [fr TS2]. */
static double tent_w(double d) {
  double x = fabs(d);
  return x < 1.0 ? 1.0 - x : 0.0;
}

/* dW/dd of the tent kernel, taken on the half-open cell [floor(p), floor(p)+1)
 * (reading: right derivative in p).  The two taps of that cell sit at
 * d = p - t in [0, 1) (tap floor(p), slope -1) and d in [-1, 0) (tap
 * floor(p)+1, slope +1); both ends of the cell are closed on the side of p,
 * so at an integer p the tap one step above still carries slope +1. */
static double tent_dw(double d) {
  if (d >= 1.0 || d < -1.0) return 0.0;
  return d >= 0.0 ? -1.0 : 1.0;
}

/* Exported for the kernel self-tests (closed-form checks of the weights). */
double oracle_kernel_weight(int interp, double d) { return interp == 1 ? keys_w(d) : tent_w(d); }
double oracle_kernel_dweight(int interp, double d) { return interp == 1 ? keys_dw(d) : tent_dw(d); }

/* Taps along one axis for sample coordinate c: first tap index and count.
 * Linear uses floor(c) + {0,1}; cubic uses floor(c) + {-1,0,1,2}. */
static void taps_of(int interp, double c, long* first, int* count) {
  long f = (long)floor(c);
  if (interp == 1) { *first = f - 1; *count = 4; }
  else { *first = f; *count = 2; }
}

static double kw(int interp, double d) { return interp == 1 ? keys_w(d) : tent_w(d); }
static double kdw(int interp, double d) { return interp == 1 ? keys_dw(d) : tent_dw(d); }

/* ------------------------------------------------------------------ */
/* Hermitian-extended tap lookup (per tap)                             */
/* ------------------------------------------------------------------ */

static long pmod(long a, long n) { long r = a % n; return r < 0 ? r + n : r; }

/* Map an unbounded integer tap t = (tx,ty,tz) onto a stored rfft entry.
 * With m = tx mod D: if m <= D/2 the entry (z,y,x) = (tz mod D, ty mod D, m)
 * is used as is; otherwise the Friedel mate (-tz mod D, -ty mod D, D - m) is
 * used and conjugated [nl M, fr TS2, hi 4].  Returns the linear voxel index
 * and sets *conj. */
static long tap_index(int D, long tx, long ty, long tz, int* conj) {
  long half = D / 2, m = pmod(tx, D), x, y, z;
  if (m <= half) { x = m; y = pmod(ty, D); z = pmod(tz, D); *conj = 0; }
  else { x = D - m; y = pmod(-ty, D); z = pmod(-tz, D); *conj = 1; }
  return (z * D + y) * (half + 1) + x;
}

/* ------------------------------------------------------------------ */
/* Geometry shared by all ops                                          */
/* ------------------------------------------------------------------ */

typedef struct {
  int B, P, Bv, Br, Bs, D, H, interp;
  double o, r;
} geom_t;

static int check_geom(const geom_t* g) {
  if (g->B <= 0 || g->P <= 0 || g->D <= 0 || g->H <= 0) return -1;
  if ((g->D & 1) || (g->H & 1)) return -2;
  if (!(g->Bv == 1 || g->Bv == g->B) || !(g->Br == 1 || g->Br == g->B)) return -3;
  if (!(g->Bs == 0 || g->Bs == 1 || g->Bs == g->B)) return -3;
  if (g->interp != 0 && g->interp != 1) return -4;
  if (!(g->o > 0.0)) return -5;
  if (g->r != g->r) return -6;
  return 0;
}

/* Frequency of image pixel (iy, ix): kx from rfftfreq, ky from fftfreq. */
static void pixel_freq(int H, int iy, int ix, double* kx, double* ky) {
  *kx = (double)ix;
  *ky = (double)(iy < H / 2 ? iy : iy - H);
}

static int in_mask(double r, double kx, double ky) { return r < 0.0 || kx * kx + ky * ky <= r * r; }

/* Rotated central-slice coordinate p = o * R * (kx, ky, 0)^T. */
static void slice_coord(const double* R, double o, double kx, double ky, double p[3]) {
  for (int i = 0; i < 3; ++i) p[i] = o * (R[3 * i + 0] * kx + R[3 * i + 1] * ky);
}

/* Shift phase phi = exp(-2 pi i (kx sx + ky sy) / H) [nl M, fr TS2]. */
static void shift_phase(const double* s, int H, double kx, double ky, double* pr, double* pi) {
  if (!s) { *pr = 1.0; *pi = 0.0; return; }
  double ang = -2.0 * M_PI * (kx * s[0] + ky * s[1]) / (double)H;
  *pr = cos(ang); *pi = sin(ang);
}

/* Interpolate the complex volume at p: value I(p) and, if dI != NULL, the
 * three partial derivatives dI/dp_a (each complex, interleaved). */
static void interp_complex(const double* V, int D, int interp, const double p[3], double I[2], double* dI) {
  long f[3]; int n[3];
  for (int a = 0; a < 3; ++a) taps_of(interp, p[a], &f[a], &n[a]);
  I[0] = I[1] = 0.0;
  if (dI) for (int q = 0; q < 6; ++q) dI[q] = 0.0;
  for (int c = 0; c < n[2]; ++c) {
    long tz = f[2] + c; double dz = p[2] - (double)tz;
    for (int b = 0; b < n[1]; ++b) {
      long ty = f[1] + b; double dy = p[1] - (double)ty;
      for (int a = 0; a < n[0]; ++a) {
        long tx = f[0] + a; double dx = p[0] - (double)tx;
        int cj; long idx = tap_index(D, tx, ty, tz, &cj);
        double vr = V[2 * idx], vi = cj ? -V[2 * idx + 1] : V[2 * idx + 1];
        double wx = kw(interp, dx), wy = kw(interp, dy), wz = kw(interp, dz);
        double w = wx * wy * wz;
        I[0] += w * vr; I[1] += w * vi;
        if (dI) {
          double gx = kdw(interp, dx) * wy * wz, gy = wx * kdw(interp, dy) * wz, gz = wx * wy * kdw(interp, dz);
          dI[0] += gx * vr; dI[1] += gx * vi;
          dI[2] += gy * vr; dI[3] += gy * vi;
          dI[4] += gz * vr; dI[5] += gz * vi;
        }
      }
    }
  }
}

/* Same for a real volume (weight channel): mirrored taps take no conjugate. */
static void interp_real(const double* W, int D, int interp, const double p[3], double* I, double* dI) {
  long f[3]; int n[3];
  for (int a = 0; a < 3; ++a) taps_of(interp, p[a], &f[a], &n[a]);
  *I = 0.0;
  if (dI) dI[0] = dI[1] = dI[2] = 0.0;
  for (int c = 0; c < n[2]; ++c) {
    long tz = f[2] + c; double dz = p[2] - (double)tz;
    for (int b = 0; b < n[1]; ++b) {
      long ty = f[1] + b; double dy = p[1] - (double)ty;
      for (int a = 0; a < n[0]; ++a) {
        long tx = f[0] + a; double dx = p[0] - (double)tx;
        int cj; long idx = tap_index(D, tx, ty, tz, &cj);
        double v = W[idx];
        double wx = kw(interp, dx), wy = kw(interp, dy), wz = kw(interp, dz);
        *I += wx * wy * wz * v;
        if (dI) {
          dI[0] += kdw(interp, dx) * wy * wz * v;
          dI[1] += wx * kdw(interp, dy) * wz * v;
          dI[2] += wx * wy * kdw(interp, dz) * v;
        }
      }
    }
  }
}

/* Adjoint of interp_complex at p: add the complex value c to every tap with
 * its weight; a mirrored tap receives conj(c) [reading: exact adjoint]. */
static void spread_complex(double* V, int D, int interp, const double p[3], double cr, double ci) {
  long f[3]; int n[3];
  for (int a = 0; a < 3; ++a) taps_of(interp, p[a], &f[a], &n[a]);
  for (int c = 0; c < n[2]; ++c) {
    long tz = f[2] + c; double wz = kw(interp, p[2] - (double)tz);
    for (int b = 0; b < n[1]; ++b) {
      long ty = f[1] + b; double wy = kw(interp, p[1] - (double)ty);
      for (int a = 0; a < n[0]; ++a) {
        long tx = f[0] + a; double wx = kw(interp, p[0] - (double)tx);
        int cj; long idx = tap_index(D, tx, ty, tz, &cj);
        double w = wx * wy * wz;
        V[2 * idx] += w * cr;
        V[2 * idx + 1] += w * (cj ? -ci : ci);
      }
    }
  }
}

/* Adjoint of interp_real: real value, no conjugate on mirrored taps. */
static void spread_real(double* W, int D, int interp, const double p[3], double v) {
  long f[3]; int n[3];
  for (int a = 0; a < 3; ++a) taps_of(interp, p[a], &f[a], &n[a]);
  for (int c = 0; c < n[2]; ++c) {
    long tz = f[2] + c; double wz = kw(interp, p[2] - (double)tz);
    for (int b = 0; b < n[1]; ++b) {
      long ty = f[1] + b; double wy = kw(interp, p[1] - (double)ty);
      for (int a = 0; a < n[0]; ++a) {
        long tx = f[0] + a; double wx = kw(interp, p[0] - (double)tx);
        int cj; long idx = tap_index(D, tx, ty, tz, &cj);
        W[idx] += wx * wy * wz * v;
      }
    }
  }
}

/* ------------------------------------------------------------------ */
/* Sizes and batch indexing                                            */
/* ------------------------------------------------------------------ */

static size_t vol_elems(const geom_t* g) { return (size_t)g->D * g->D * (g->D / 2 + 1); }
static size_t img_elems(const geom_t* g) { return (size_t)g->H * (g->H / 2 + 1); }
static int bsel(int Bx, int b) { return Bx == 1 ? 0 : b; }

/* ------------------------------------------------------------------ */
/* 3D -> 2D forward                                                    */
/* ------------------------------------------------------------------ */

/* out[b][n][iy][ix] = M * phi * I(V[bv], p) [es TS2, nl M, fr TS2]. */
static void project_one(const geom_t* g, const double* V, const double* R, const double* s, double* out) {
  int W2 = g->H / 2 + 1;
  for (int iy = 0; iy < g->H; ++iy)
    for (int ix = 0; ix < W2; ++ix) {
      double kx, ky; pixel_freq(g->H, iy, ix, &kx, &ky);
      double* o = out + 2 * ((size_t)iy * W2 + ix);
      if (!in_mask(g->r, kx, ky)) { o[0] = o[1] = 0.0; continue; }
      double p[3], I[2], pr, pi;
      slice_coord(R, g->o, kx, ky, p);
      interp_complex(V, g->D, g->interp, p, I, NULL);
      shift_phase(s, g->H, kx, ky, &pr, &pi);
      o[0] = pr * I[0] - pi * I[1];
      o[1] = pr * I[1] + pi * I[0];
    }
}

int oracle_project(int B, int P, int Bv, int Br, int Bs, int D, int H, int interp, double o, double r,
                   const double* vol, const double* rot, const double* shifts, double* out) {
  geom_t g = {B, P, Bv, Br, shifts ? Bs : 0, D, H, interp, o, r};
  int e = check_geom(&g); if (e) return e;
  if (!vol || !rot || !out) return -7;
  size_t nv = vol_elems(&g), ni = img_elems(&g);
  long total = (long)B * P;
#pragma omp parallel for schedule(dynamic, 1)
  for (long bn = 0; bn < total; ++bn) {
    int b = (int)(bn / P), n = (int)(bn % P);
    const double* V = vol + 2 * nv * bsel(Bv, b);
    const double* R = rot + 9 * ((size_t)bsel(Br, b) * P + n);
    const double* s = shifts ? shifts + 2 * ((size_t)bsel(Bs, b) * P + n) : NULL;
    project_one(&g, V, R, s, out + 2 * ni * (size_t)bn);
  }
  return 0;
}

/* ------------------------------------------------------------------ */
/* 2D -> 3D back-projection (adjoint)                                  */
/* ------------------------------------------------------------------ */

/* Accumulate image (b, n) into the data volume (and its weight image into the
 * weight volume) [es TS2, nl M, fr TS2]: c = conj(phi) * Y, spread with the
 * interpolation weights; the weight channel is real, unshifted. */
static void backproject_one(const geom_t* g, const double* Y, const double* Wimg, const double* R,
                            const double* s, double* Vd, double* Vw) {
  int W2 = g->H / 2 + 1;
  for (int iy = 0; iy < g->H; ++iy)
    for (int ix = 0; ix < W2; ++ix) {
      double kx, ky; pixel_freq(g->H, iy, ix, &kx, &ky);
      if (!in_mask(g->r, kx, ky)) continue;
      size_t k = (size_t)iy * W2 + ix;
      double p[3], pr, pi;
      slice_coord(R, g->o, kx, ky, p);
      shift_phase(s, g->H, kx, ky, &pr, &pi);
      double yr = Y[2 * k], yi = Y[2 * k + 1];
      /* conj(phi) * Y */
      double cr = pr * yr + pi * yi, ci = pr * yi - pi * yr;
      spread_complex(Vd, g->D, g->interp, p, cr, ci);
      if (Wimg && Vw) spread_real(Vw, g->D, g->interp, p, Wimg[k]);
    }
}

/* Sum over all (b, n) into Bv volumes.  Threads accumulate into private
 * volumes that are added together at the end. */
static int backproject_all(const geom_t* g, const double* images, const double* weights, const double* rot,
                           const double* shifts, double* data_vol, double* weight_vol) {
  size_t nv = vol_elems(g), ni = img_elems(g);
  memset(data_vol, 0, sizeof(double) * 2 * nv * g->Bv);
  if (weight_vol) memset(weight_vol, 0, sizeof(double) * nv * g->Bv);
  long total = (long)g->B * g->P;
  int nthreads = 1;
#ifdef _OPENMP
  nthreads = omp_get_max_threads();
#endif
  size_t per_d = 2 * nv * g->Bv, per_w = weight_vol ? nv * g->Bv : 0;
  double* priv = (double*)calloc((size_t)nthreads * (per_d + per_w), sizeof(double));
  if (!priv) return -8;
#pragma omp parallel num_threads(nthreads)
  {
    int tid = 0;
#ifdef _OPENMP
    tid = omp_get_thread_num();
#endif
    double* myd = priv + (size_t)tid * (per_d + per_w);
    double* myw = weight_vol ? myd + per_d : NULL;
#pragma omp for schedule(dynamic, 1)
    for (long bn = 0; bn < total; ++bn) {
      int b = (int)(bn / g->P), n = (int)(bn % g->P), bv = bsel(g->Bv, b);
      const double* R = rot + 9 * ((size_t)bsel(g->Br, b) * g->P + n);
      const double* s = shifts ? shifts + 2 * ((size_t)bsel(g->Bs, b) * g->P + n) : NULL;
      backproject_one(g, images + 2 * ni * (size_t)bn, weights ? weights + ni * (size_t)bn : NULL, R, s,
                      myd + 2 * nv * bv, myw ? myw + nv * bv : NULL);
    }
  }
  for (int t = 0; t < nthreads; ++t) {
    const double* src = priv + (size_t)t * (per_d + per_w);
#pragma omp parallel for
    for (long i = 0; i < (long)per_d; ++i) data_vol[i] += src[i];
    if (weight_vol) {
#pragma omp parallel for
      for (long i = 0; i < (long)per_w; ++i) weight_vol[i] += src[per_d + i];
    }
  }
  free(priv);
  return 0;
}

int oracle_backproject(int B, int P, int Bv, int Br, int Bs, int D, int H, int interp, double o, double r,
                       const double* images, const double* weights, const double* rot, const double* shifts,
                       double* data_vol, double* weight_vol) {
  geom_t g = {B, P, Bv, Br, shifts ? Bs : 0, D, H, interp, o, r};
  int e = check_geom(&g); if (e) return e;
  if (!images || !rot || !data_vol) return -7;
  if ((weights == NULL) != (weight_vol == NULL)) return -7;
  return backproject_all(&g, images, weights, rot, shifts, data_vol, weight_vol);
}

/* ------------------------------------------------------------------ */
/* Gradients of the rotation and the shift for one projection          */
/* ------------------------------------------------------------------ */

/* For one (b, n): given the volume Vc (complex, may be NULL), the real volume
 * Vr (may be NULL), the complex upstream U (pairs with Vc) and the real
 * upstream Ur (pairs with Vr), accumulate
 *   gR[i][j] += o * sum_k M * ( Re(conj(U) phi dI_i(Vc)) + Ur dI_i(Vr) ) * k3_j
 *   gs[0..1] += (2 pi / H) * sum_k M * (kx, ky) * Im(conj(U) phi I(Vc))
 * with k3 = (kx, ky, 0).  This is the derivative of L = Re<U, phi I(Vc)> +
 * <Ur, I(Vr)> w.r.t. R and s [es TS2, nl M]. */
static void rot_shift_grad_one(const geom_t* g, const double* Vc, const double* Vr, const double* U,
                               const double* Ur, const double* R, const double* s, double gR[9],
                               double gs[2]) {
  int W2 = g->H / 2 + 1;
  for (int q = 0; q < 9; ++q) gR[q] = 0.0;
  gs[0] = gs[1] = 0.0;
  for (int iy = 0; iy < g->H; ++iy)
    for (int ix = 0; ix < W2; ++ix) {
      double kx, ky; pixel_freq(g->H, iy, ix, &kx, &ky);
      if (!in_mask(g->r, kx, ky)) continue;
      size_t k = (size_t)iy * W2 + ix;
      double p[3], k3[3] = {kx, ky, 0.0}, e[3] = {0.0, 0.0, 0.0};
      slice_coord(R, g->o, kx, ky, p);
      if (Vc) {
        double I[2], dI[6], pr, pi;
        interp_complex(Vc, g->D, g->interp, p, I, dI);
        shift_phase(s, g->H, kx, ky, &pr, &pi);
        double ur = U[2 * k], ui = U[2 * k + 1];
        for (int i = 0; i < 3; ++i) {
          /* phi * dI_i */
          double ar = pr * dI[2 * i] - pi * dI[2 * i + 1], ai = pr * dI[2 * i + 1] + pi * dI[2 * i];
          e[i] += ur * ar + ui * ai; /* Re(conj(U) * a) */
        }
        double yr = pr * I[0] - pi * I[1], yi = pr * I[1] + pi * I[0];
        double im = ur * yi - ui * yr; /* Im(conj(U) * Y) */
        gs[0] += 2.0 * M_PI / g->H * kx * im;
        gs[1] += 2.0 * M_PI / g->H * ky * im;
      }
      if (Vr) {
        double I, dI[3];
        interp_real(Vr, g->D, g->interp, p, &I, dI);
        for (int i = 0; i < 3; ++i) e[i] += Ur[k] * dI[i];
      }
      for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j) gR[3 * i + j] += g->o * e[i] * k3[j];
    }
}

/* ------------------------------------------------------------------ */
/* Backward of the 3D -> 2D forward                                    */
/* ------------------------------------------------------------------ */

/* grad_vol = BP(grad_out) (the adjoint), grad_rot and grad_shifts from the
 * formulas above with (volume, upstream) = (vol, grad_out).  Gradients of
 * broadcast inputs are summed over the batch.  Any output may be NULL. */
int oracle_project_backward(int B, int P, int Bv, int Br, int Bs, int D, int H, int interp, double o, double r,
                            const double* grad_out, const double* vol, const double* rot, const double* shifts,
                            double* grad_vol, double* grad_rot, double* grad_shifts) {
  geom_t g = {B, P, Bv, Br, shifts ? Bs : 0, D, H, interp, o, r};
  int e = check_geom(&g); if (e) return e;
  if (!grad_out || !rot) return -7;
  if ((grad_rot || grad_shifts) && !vol) return -7;
  if (grad_shifts && !shifts) return -7;
  if (grad_vol) {
    e = backproject_all(&g, grad_out, NULL, rot, shifts, grad_vol, NULL);
    if (e) return e;
  }
  if (grad_rot || grad_shifts) {
    size_t nv = vol_elems(&g), ni = img_elems(&g);
    long total = (long)B * P;
    double* gr = (double*)calloc((size_t)total * 11, sizeof(double));
    if (!gr) return -8;
#pragma omp parallel for schedule(dynamic, 1)
    for (long bn = 0; bn < total; ++bn) {
      int b = (int)(bn / P), n = (int)(bn % P);
      const double* R = rot + 9 * ((size_t)bsel(Br, b) * P + n);
      const double* s = shifts ? shifts + 2 * ((size_t)bsel(g.Bs, b) * P + n) : NULL;
      rot_shift_grad_one(&g, vol + 2 * nv * bsel(Bv, b), NULL, grad_out + 2 * ni * (size_t)bn, NULL, R, s,
                         gr + 11 * bn, gr + 11 * bn + 9);
    }
    if (grad_rot) memset(grad_rot, 0, sizeof(double) * 9 * (size_t)Br * P);
    if (grad_shifts) memset(grad_shifts, 0, sizeof(double) * 2 * (size_t)g.Bs * P);
    for (long bn = 0; bn < total; ++bn) {
      int b = (int)(bn / P), n = (int)(bn % P);
      if (grad_rot)
        for (int q = 0; q < 9; ++q) grad_rot[9 * ((size_t)bsel(Br, b) * P + n) + q] += gr[11 * bn + q];
      if (grad_shifts)
        for (int q = 0; q < 2; ++q) grad_shifts[2 * ((size_t)bsel(g.Bs, b) * P + n) + q] += gr[11 * bn + 9 + q];
    }
    free(gr);
  }
  return 0;
}

/* ------------------------------------------------------------------ */
/* Backward of the 2D -> 3D back-projection                            */
/* ------------------------------------------------------------------ */

/* grad_images = M phi I(grad_data_vol, p)   (the forward of the upstream),
 * grad_weights = M I_real(grad_weight_vol, p),
 * grad_rot / grad_shifts from the formulas above with (volume, upstream) =
 * (grad_data_vol, images) plus the real channel (grad_weight_vol, weights).
 * Any output may be NULL. */
int oracle_backproject_backward(int B, int P, int Bv, int Br, int Bs, int D, int H, int interp, double o,
                                double r, const double* grad_data_vol, const double* grad_weight_vol,
                                const double* images, const double* weights, const double* rot,
                                const double* shifts, double* grad_images, double* grad_weights,
                                double* grad_rot, double* grad_shifts) {
  geom_t g = {B, P, Bv, Br, shifts ? Bs : 0, D, H, interp, o, r};
  int e = check_geom(&g); if (e) return e;
  if (!grad_data_vol || !rot) return -7;
  if (grad_weights && !grad_weight_vol) return -7;
  if ((grad_rot || grad_shifts) && !images) return -7;
  if (grad_rot && grad_weight_vol && !weights) return -7;
  if (grad_shifts && !shifts) return -7;
  size_t nv = vol_elems(&g), ni = img_elems(&g);
  long total = (long)B * P;
  if (grad_images) {
    e = oracle_project(B, P, Bv, Br, Bs, D, H, interp, o, r, grad_data_vol, rot, shifts, grad_images);
    if (e) return e;
  }
  if (grad_weights) {
    int W2 = H / 2 + 1;
#pragma omp parallel for schedule(dynamic, 1)
    for (long bn = 0; bn < total; ++bn) {
      int b = (int)(bn / P), n = (int)(bn % P);
      const double* R = rot + 9 * ((size_t)bsel(Br, b) * P + n);
      const double* Vw = grad_weight_vol + nv * bsel(Bv, b);
      double* out = grad_weights + ni * (size_t)bn;
      for (int iy = 0; iy < H; ++iy)
        for (int ix = 0; ix < W2; ++ix) {
          double kx, ky; pixel_freq(H, iy, ix, &kx, &ky);
          size_t k = (size_t)iy * W2 + ix;
          if (!in_mask(r, kx, ky)) { out[k] = 0.0; continue; }
          double p[3], I;
          slice_coord(R, o, kx, ky, p);
          interp_real(Vw, D, interp, p, &I, NULL);
          out[k] = I;
        }
    }
  }
  if (grad_rot || grad_shifts) {
    double* gr = (double*)calloc((size_t)total * 11, sizeof(double));
    if (!gr) return -8;
    int use_w = grad_weight_vol != NULL && weights != NULL;
#pragma omp parallel for schedule(dynamic, 1)
    for (long bn = 0; bn < total; ++bn) {
      int b = (int)(bn / P), n = (int)(bn % P);
      const double* R = rot + 9 * ((size_t)bsel(Br, b) * P + n);
      const double* s = shifts ? shifts + 2 * ((size_t)bsel(g.Bs, b) * P + n) : NULL;
      rot_shift_grad_one(&g, grad_data_vol + 2 * nv * bsel(Bv, b), use_w ? grad_weight_vol + nv * bsel(Bv, b) : NULL,
                         images + 2 * ni * (size_t)bn, use_w ? weights + ni * (size_t)bn : NULL, R, s,
                         gr + 11 * bn, gr + 11 * bn + 9);
    }
    if (grad_rot) memset(grad_rot, 0, sizeof(double) * 9 * (size_t)Br * P);
    if (grad_shifts) memset(grad_shifts, 0, sizeof(double) * 2 * (size_t)g.Bs * P);
    for (long bn = 0; bn < total; ++bn) {
      int b = (int)(bn / P), n = (int)(bn % P);
      if (grad_rot)
        for (int q = 0; q < 9; ++q) grad_rot[9 * ((size_t)bsel(Br, b) * P + n) + q] += gr[11 * bn + q];
      if (grad_shifts)
        for (int q = 0; q < 2; ++q) grad_shifts[2 * ((size_t)bsel(g.Bs, b) * P + n) + q] += gr[11 * bn + 9 + q];
    }
    free(gr);
  }
  return 0;
}

/* ================================================================== */
/* 2D -> 2D: rotation of 2D Fourier data and its adjoint              */
/* ================================================================== */
/* The pages list 2D -> 2D forward (rotation of 2D Fourier data) and 2D -> 2D
 * backward (accumulation into a 2D reconstruction) next to the 3D ops
 * [nl M ops 1-2, es TS2, fr TS2].  Readings, mirroring the 3D ops: the source
 * is an rfft image X[y][x] of box D (x halved); the sample of output pixel
 * (kx, ky) is p = o * R * (kx, ky)^T with a 2x2 map R (rows/cols (x, y));
 * taps are looked up with the same per-tap Friedel rule in 2D; shifts,
 * cutoff, weights and gradients are defined exactly as for the 3D ops. */

/* Stored entry of the 2D tap (tx, ty): m = tx mod D; m <= D/2 -> (ty mod D,
 * m); otherwise the conjugated mate (-ty mod D, D - m). */
static long tap_index2(int D, long tx, long ty, int* conj) {
  long half = D / 2, m = pmod(tx, D);
  if (m <= half) { *conj = 0; return pmod(ty, D) * (half + 1) + m; }
  *conj = 1;
  return pmod(-ty, D) * (half + 1) + (D - m);
}

static void slice_coord2(const double* R, double o, double kx, double ky, double p[2]) {
  for (int i = 0; i < 2; ++i) p[i] = o * (R[2 * i + 0] * kx + R[2 * i + 1] * ky);
}

/* I(p) of the complex source and, if dI != NULL, dI/dp_0, dI/dp_1. */
static void interp2_complex(const double* X, int D, int interp, const double p[2], double I[2], double* dI) {
  long f[2]; int n[2];
  for (int a = 0; a < 2; ++a) taps_of(interp, p[a], &f[a], &n[a]);
  I[0] = I[1] = 0.0;
  if (dI) for (int q = 0; q < 4; ++q) dI[q] = 0.0;
  for (int b = 0; b < n[1]; ++b) {
    long ty = f[1] + b; double dy = p[1] - (double)ty;
    for (int a = 0; a < n[0]; ++a) {
      long tx = f[0] + a; double dx = p[0] - (double)tx;
      int cj; long idx = tap_index2(D, tx, ty, &cj);
      double vr = X[2 * idx], vi = cj ? -X[2 * idx + 1] : X[2 * idx + 1];
      double wx = kw(interp, dx), wy = kw(interp, dy), w = wx * wy;
      I[0] += w * vr; I[1] += w * vi;
      if (dI) {
        double gx = kdw(interp, dx) * wy, gy = wx * kdw(interp, dy);
        dI[0] += gx * vr; dI[1] += gx * vi;
        dI[2] += gy * vr; dI[3] += gy * vi;
      }
    }
  }
}

static void interp2_real(const double* W, int D, int interp, const double p[2], double* I, double* dI) {
  long f[2]; int n[2];
  for (int a = 0; a < 2; ++a) taps_of(interp, p[a], &f[a], &n[a]);
  *I = 0.0;
  if (dI) dI[0] = dI[1] = 0.0;
  for (int b = 0; b < n[1]; ++b) {
    long ty = f[1] + b; double dy = p[1] - (double)ty;
    for (int a = 0; a < n[0]; ++a) {
      long tx = f[0] + a; double dx = p[0] - (double)tx;
      int cj; long idx = tap_index2(D, tx, ty, &cj);
      double v = W[idx], wx = kw(interp, dx), wy = kw(interp, dy);
      *I += wx * wy * v;
      if (dI) { dI[0] += kdw(interp, dx) * wy * v; dI[1] += wx * kdw(interp, dy) * v; }
    }
  }
}

/* Adjoints of the two interpolations. */
static void spread2_complex(double* X, int D, int interp, const double p[2], double cr, double ci) {
  long f[2]; int n[2];
  for (int a = 0; a < 2; ++a) taps_of(interp, p[a], &f[a], &n[a]);
  for (int b = 0; b < n[1]; ++b) {
    long ty = f[1] + b; double wy = kw(interp, p[1] - (double)ty);
    for (int a = 0; a < n[0]; ++a) {
      long tx = f[0] + a; double w = kw(interp, p[0] - (double)tx) * wy;
      int cj; long idx = tap_index2(D, tx, ty, &cj);
      X[2 * idx] += w * cr;
      X[2 * idx + 1] += w * (cj ? -ci : ci);
    }
  }
}

static void spread2_real(double* W, int D, int interp, const double p[2], double v) {
  long f[2]; int n[2];
  for (int a = 0; a < 2; ++a) taps_of(interp, p[a], &f[a], &n[a]);
  for (int b = 0; b < n[1]; ++b) {
    long ty = f[1] + b; double wy = kw(interp, p[1] - (double)ty);
    for (int a = 0; a < n[0]; ++a) {
      long tx = f[0] + a;
      int cj; long idx = tap_index2(D, tx, ty, &cj);
      W[idx] += kw(interp, p[0] - (double)tx) * wy * v;
    }
  }
}

static size_t src2_elems(const geom_t* g) { return (size_t)g->D * (g->D / 2 + 1); }

/* out[b][n] = M * phi * I(X[bx], o R k). */
int oracle_project2d(int B, int P, int Bv, int Br, int Bs, int D, int H, int interp, double o, double r,
                     const double* src, const double* rot, const double* shifts, double* out) {
  geom_t g = {B, P, Bv, Br, shifts ? Bs : 0, D, H, interp, o, r};
  int e = check_geom(&g); if (e) return e;
  if (!src || !rot || !out) return -7;
  size_t nx = src2_elems(&g), ni = img_elems(&g);
  int W2 = H / 2 + 1;
  long total = (long)B * P;
#pragma omp parallel for schedule(dynamic, 1)
  for (long bn = 0; bn < total; ++bn) {
    int b = (int)(bn / P), n = (int)(bn % P);
    const double* X = src + 2 * nx * bsel(Bv, b);
    const double* R = rot + 4 * ((size_t)bsel(Br, b) * P + n);
    const double* s = shifts ? shifts + 2 * ((size_t)bsel(g.Bs, b) * P + n) : NULL;
    double* O = out + 2 * ni * (size_t)bn;
    for (int iy = 0; iy < H; ++iy)
      for (int ix = 0; ix < W2; ++ix) {
        double kx, ky; pixel_freq(H, iy, ix, &kx, &ky);
        double* q = O + 2 * ((size_t)iy * W2 + ix);
        if (!in_mask(r, kx, ky)) { q[0] = q[1] = 0.0; continue; }
        double p[2], I[2], pr, pi;
        slice_coord2(R, o, kx, ky, p);
        interp2_complex(X, D, interp, p, I, NULL);
        shift_phase(s, H, kx, ky, &pr, &pi);
        q[0] = pr * I[0] - pi * I[1];
        q[1] = pr * I[1] + pi * I[0];
      }
  }
  return 0;
}

/* Accumulation of images (and real weights) into Bv 2D reconstructions: the
 * adjoint of oracle_project2d (weights: real, unshifted). */
int oracle_backproject2d(int B, int P, int Bv, int Br, int Bs, int D, int H, int interp, double o, double r,
                         const double* images, const double* weights, const double* rot, const double* shifts,
                         double* data_img, double* weight_img) {
  geom_t g = {B, P, Bv, Br, shifts ? Bs : 0, D, H, interp, o, r};
  int e = check_geom(&g); if (e) return e;
  if (!images || !rot || !data_img) return -7;
  if ((weights == NULL) != (weight_img == NULL)) return -7;
  size_t nx = src2_elems(&g), ni = img_elems(&g);
  int W2 = H / 2 + 1;
  memset(data_img, 0, sizeof(double) * 2 * nx * Bv);
  if (weight_img) memset(weight_img, 0, sizeof(double) * nx * Bv);
  /* one pass in (b, n) order: the result does not depend on thread count */
  for (long bn = 0; bn < (long)B * P; ++bn) {
    int b = (int)(bn / P), n = (int)(bn % P), bv = bsel(Bv, b);
    const double* R = rot + 4 * ((size_t)bsel(Br, b) * P + n);
    const double* s = shifts ? shifts + 2 * ((size_t)bsel(g.Bs, b) * P + n) : NULL;
    const double* Y = images + 2 * ni * (size_t)bn;
    for (int iy = 0; iy < H; ++iy)
      for (int ix = 0; ix < W2; ++ix) {
        double kx, ky; pixel_freq(H, iy, ix, &kx, &ky);
        if (!in_mask(r, kx, ky)) continue;
        size_t k = (size_t)iy * W2 + ix;
        double p[2], pr, pi;
        slice_coord2(R, o, kx, ky, p);
        shift_phase(s, H, kx, ky, &pr, &pi);
        double yr = Y[2 * k], yi = Y[2 * k + 1];
        spread2_complex(data_img + 2 * nx * bv, D, interp, p, pr * yr + pi * yi, pr * yi - pi * yr);
        if (weights) spread2_real(weight_img + nx * bv, D, interp, p, weights[ni * (size_t)bn + k]);
      }
  }
  return 0;
}

/* gR (2x2) and gs of one projection: derivative of Re<U, phi I(Xc)> +
 * <Ur, I(Xr)> w.r.t. R and s; same formulas as the 3D ops with k2 = (kx, ky). */
static void rot_shift_grad2_one(const geom_t* g, const double* Xc, const double* Xr, const double* U,
                                const double* Ur, const double* R, const double* s, double gR[4], double gs[2]) {
  int W2 = g->H / 2 + 1;
  for (int q = 0; q < 4; ++q) gR[q] = 0.0;
  gs[0] = gs[1] = 0.0;
  for (int iy = 0; iy < g->H; ++iy)
    for (int ix = 0; ix < W2; ++ix) {
      double kx, ky; pixel_freq(g->H, iy, ix, &kx, &ky);
      if (!in_mask(g->r, kx, ky)) continue;
      size_t k = (size_t)iy * W2 + ix;
      double p[2], k2[2] = {kx, ky}, e[2] = {0.0, 0.0};
      slice_coord2(R, g->o, kx, ky, p);
      if (Xc) {
        double I[2], dI[4], pr, pi;
        interp2_complex(Xc, g->D, g->interp, p, I, dI);
        shift_phase(s, g->H, kx, ky, &pr, &pi);
        double ur = U[2 * k], ui = U[2 * k + 1];
        for (int i = 0; i < 2; ++i) {
          double ar = pr * dI[2 * i] - pi * dI[2 * i + 1], ai = pr * dI[2 * i + 1] + pi * dI[2 * i];
          e[i] += ur * ar + ui * ai;
        }
        double yr = pr * I[0] - pi * I[1], yi = pr * I[1] + pi * I[0];
        double im = ur * yi - ui * yr;
        gs[0] += 2.0 * M_PI / g->H * kx * im;
        gs[1] += 2.0 * M_PI / g->H * ky * im;
      }
      if (Xr) {
        double I, dI[2];
        interp2_real(Xr, g->D, g->interp, p, &I, dI);
        for (int i = 0; i < 2; ++i) e[i] += Ur[k] * dI[i];
      }
      for (int i = 0; i < 2; ++i)
        for (int j = 0; j < 2; ++j) gR[2 * i + j] += g->o * e[i] * k2[j];
    }
}

/* Sum the per-projection gR/gs of every (b, n) into the (broadcast) outputs. */
static int rot_shift_grads2(const geom_t* g, const double* Xc, const double* Xr, const double* U, const double* Ur,
                            const double* rot, const double* shifts, double* grad_rot, double* grad_shifts) {
  size_t nx = src2_elems(g), ni = img_elems(g);
  long total = (long)g->B * g->P;
  double* gr = (double*)calloc((size_t)total * 6, sizeof(double));
  if (!gr) return -8;
#pragma omp parallel for schedule(dynamic, 1)
  for (long bn = 0; bn < total; ++bn) {
    int b = (int)(bn / g->P), n = (int)(bn % g->P);
    const double* R = rot + 4 * ((size_t)bsel(g->Br, b) * g->P + n);
    const double* s = shifts ? shifts + 2 * ((size_t)bsel(g->Bs, b) * g->P + n) : NULL;
    rot_shift_grad2_one(g, Xc ? Xc + 2 * nx * bsel(g->Bv, b) : NULL, Xr ? Xr + nx * bsel(g->Bv, b) : NULL,
                        U + 2 * ni * (size_t)bn, Ur ? Ur + ni * (size_t)bn : NULL, R, s, gr + 6 * bn,
                        gr + 6 * bn + 4);
  }
  if (grad_rot) memset(grad_rot, 0, sizeof(double) * 4 * (size_t)g->Br * g->P);
  if (grad_shifts) memset(grad_shifts, 0, sizeof(double) * 2 * (size_t)g->Bs * g->P);
  for (long bn = 0; bn < total; ++bn) {
    int b = (int)(bn / g->P), n = (int)(bn % g->P);
    if (grad_rot)
      for (int q = 0; q < 4; ++q) grad_rot[4 * ((size_t)bsel(g->Br, b) * g->P + n) + q] += gr[6 * bn + q];
    if (grad_shifts)
      for (int q = 0; q < 2; ++q) grad_shifts[2 * ((size_t)bsel(g->Bs, b) * g->P + n) + q] += gr[6 * bn + 4 + q];
  }
  free(gr);
  return 0;
}

/* Backward of oracle_project2d: grad_src = adjoint(grad_out), grad_rot,
 * grad_shifts.  Any output may be NULL. */
int oracle_project2d_backward(int B, int P, int Bv, int Br, int Bs, int D, int H, int interp, double o, double r,
                              const double* grad_out, const double* src, const double* rot, const double* shifts,
                              double* grad_src, double* grad_rot, double* grad_shifts) {
  geom_t g = {B, P, Bv, Br, shifts ? Bs : 0, D, H, interp, o, r};
  int e = check_geom(&g); if (e) return e;
  if (!grad_out || !rot) return -7;
  if ((grad_rot || grad_shifts) && !src) return -7;
  if (grad_shifts && !shifts) return -7;
  if (grad_src) {
    e = oracle_backproject2d(B, P, Bv, Br, Bs, D, H, interp, o, r, grad_out, NULL, rot, shifts, grad_src, NULL);
    if (e) return e;
  }
  if (grad_rot || grad_shifts) return rot_shift_grads2(&g, src, NULL, grad_out, NULL, rot, shifts, grad_rot, grad_shifts);
  return 0;
}

/* Backward of oracle_backproject2d: grad_images = M phi I(grad_data),
 * grad_weights = M I_real(grad_weight), grad_rot / grad_shifts with (source,
 * upstream) = (grad_data, images) plus the real channel (grad_weight,
 * weights).  Any output may be NULL. */
int oracle_backproject2d_backward(int B, int P, int Bv, int Br, int Bs, int D, int H, int interp, double o,
                                  double r, const double* grad_data, const double* grad_weight,
                                  const double* images, const double* weights, const double* rot,
                                  const double* shifts, double* grad_images, double* grad_weights,
                                  double* grad_rot, double* grad_shifts) {
  geom_t g = {B, P, Bv, Br, shifts ? Bs : 0, D, H, interp, o, r};
  int e = check_geom(&g); if (e) return e;
  if (!grad_data || !rot) return -7;
  if (grad_weights && !grad_weight) return -7;
  if ((grad_rot || grad_shifts) && !images) return -7;
  if (grad_rot && grad_weight && !weights) return -7;
  if (grad_shifts && !shifts) return -7;
  if (grad_images) {
    e = oracle_project2d(B, P, Bv, Br, Bs, D, H, interp, o, r, grad_data, rot, shifts, grad_images);
    if (e) return e;
  }
  if (grad_weights) {
    size_t nx = src2_elems(&g), ni = img_elems(&g);
    int W2 = H / 2 + 1;
#pragma omp parallel for schedule(dynamic, 1)
    for (long bn = 0; bn < (long)B * P; ++bn) {
      int b = (int)(bn / P), n = (int)(bn % P);
      const double* R = rot + 4 * ((size_t)bsel(Br, b) * P + n);
      double* out = grad_weights + ni * (size_t)bn;
      for (int iy = 0; iy < H; ++iy)
        for (int ix = 0; ix < W2; ++ix) {
          double kx, ky; pixel_freq(H, iy, ix, &kx, &ky);
          size_t k = (size_t)iy * W2 + ix;
          if (!in_mask(r, kx, ky)) { out[k] = 0.0; continue; }
          double p[2], I;
          slice_coord2(R, o, kx, ky, p);
          interp2_real(grad_weight + nx * bsel(Bv, b), D, interp, p, &I, NULL);
          out[k] = I;
        }
    }
  }
  if (grad_rot || grad_shifts) {
    int use_w = grad_weight != NULL && weights != NULL;
    return rot_shift_grads2(&g, grad_data, use_w ? grad_weight : NULL, images, use_w ? weights : NULL, rot, shifts,
                            grad_rot, grad_shifts);
  }
  return 0;
}

/* Number of OpenMP threads the oracle will use (reported by the benchmark). */
int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Set the number of OpenMP threads of later calls (n >= 1; the benchmark
 * times the oracle on all host cores and on one).  Returns the new count. */
int oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
  return omp_get_max_threads();
#else
  (void)n;
  return 1;
#endif
}
