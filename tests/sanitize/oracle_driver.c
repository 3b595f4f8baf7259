/* Sanitizer driver for the CPU oracle (oracle/oracle.c): every entry point on
 * small problems whose buffers are allocated to their exact sizes, with
 * broadcast sources, several batch entries, images larger and smaller than
 * the box, a radius cutoff of none / zero / a few pixels, shifts present and
 * absent, linear and cubic interpolation, oversampling above one, and
 * non-rotation maps.  Built and run under AddressSanitizer and
 * UndefinedBehaviorSanitizer by tests/test_sanitizers.py; any out-of-bounds
 * access or undefined behaviour aborts with a report, any non-zero status is
 * a failure.  Test infrastructure only. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_project(int B, int P, int Bv, int Br, int Bs, int D, int H, int interp, double o, double r,
                   const double* vol, const double* rot, const double* shifts, double* out);
int oracle_backproject(int B, int P, int Bv, int Br, int Bs, int D, int H, int interp, double o, double r,
                       const double* images, const double* weights, const double* rot, const double* shifts,
                       double* data_vol, double* weight_vol);
int oracle_project_backward(int B, int P, int Bv, int Br, int Bs, int D, int H, int interp, double o, double r,
                            const double* grad_out, const double* vol, const double* rot, const double* shifts,
                            double* grad_vol, double* grad_rot, double* grad_shifts);
int oracle_backproject_backward(int B, int P, int Bv, int Br, int Bs, int D, int H, int interp, double o,
                                double r, const double* grad_data_vol, const double* grad_weight_vol,
                                const double* images, const double* weights, const double* rot,
                                const double* shifts, double* grad_images, double* grad_weights,
                                double* grad_rot, double* grad_shifts);
int oracle_project2d(int B, int P, int Bv, int Br, int Bs, int D, int H, int interp, double o, double r,
                     const double* src, const double* rot, const double* shifts, double* out);
int oracle_backproject2d(int B, int P, int Bv, int Br, int Bs, int D, int H, int interp, double o, double r,
                         const double* images, const double* weights, const double* rot, const double* shifts,
                         double* data_img, double* weight_img);
int oracle_project2d_backward(int B, int P, int Bv, int Br, int Bs, int D, int H, int interp, double o, double r,
                              const double* grad_out, const double* src, const double* rot, const double* shifts,
                              double* grad_src, double* grad_rot, double* grad_shifts);
int oracle_backproject2d_backward(int B, int P, int Bv, int Br, int Bs, int D, int H, int interp, double o,
                                  double r, const double* grad_data, const double* grad_weight,
                                  const double* images, const double* weights, const double* rot,
                                  const double* shifts, double* grad_images, double* grad_weights,
                                  double* grad_rot, double* grad_shifts);
double oracle_kernel_weight(int interp, double d);
double oracle_kernel_dweight(int interp, double d);

static unsigned long long rng_state = 88172645463325252ull;
static double urand(void) {   /* xorshift64, uniform in [-1, 1) */
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 7;
  rng_state ^= rng_state << 17;
  return (double)(rng_state >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}
static double* filled(size_t n) {
  double* p = (double*)malloc((n ? n : 1) * sizeof(double));
  for (size_t i = 0; i < n; ++i) p[i] = urand();
  return p;
}
/* n maps: rotations about a random axis, or (general) perturbed ones */
static double* maps(size_t n, int dim, int general) {
  double* R = (double*)malloc(n * dim * dim * sizeof(double));
  for (size_t m = 0; m < n; ++m) {
    double* A = R + m * dim * dim;
    if (dim == 2) {
      double t = 3.14159 * urand();
      A[0] = cos(t); A[1] = -sin(t); A[2] = sin(t); A[3] = cos(t);
    } else {
      double a[3] = {urand(), urand(), urand()}, nn = sqrt(a[0] * a[0] + a[1] * a[1] + a[2] * a[2]) + 1e-9;
      double t = 3.14159 * urand(), c = cos(t), s = sin(t);
      for (int i = 0; i < 3; ++i) a[i] /= nn;
      for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j) {
          double v = (1 - c) * a[i] * a[j] + (i == j ? c : 0.0);
          int k = 3 - i - j;
          if (i != j) v += (((i + 1) % 3 == j) ? -1.0 : 1.0) * s * a[k];
          A[3 * i + j] = v;
        }
    }
    if (general)
      for (int q = 0; q < dim * dim; ++q) A[q] = A[q] * 1.3 + 0.2 * urand();
  }
  return R;
}

static int failures = 0;
#define CHECK(call)                                                   \
  do {                                                                \
    int st_ = (call);                                                 \
    if (st_ != 0) {                                                   \
      fprintf(stderr, "status %d from %s (line %d)\n", st_, #call, __LINE__); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

static void case3d(int B, int P, int Bv, int Br, int Bs, int D, int H, int interp, double o, double r, int general) {
  const size_t nv = (size_t)D * D * (D / 2 + 1), ni = (size_t)H * (H / 2 + 1);
  double* vol = filled(2 * nv * Bv);
  double* wvol = filled(nv * Bv);
  double* rot = maps((size_t)Br * P, 3, general);
  double* sh = Bs ? filled(2 * (size_t)Bs * P) : NULL;
  double* img = filled(2 * ni * B * P);
  double* wimg = filled(ni * B * P);
  double* out = filled(2 * ni * B * P);
  double* gv = filled(2 * nv * Bv);
  double* gw = filled(nv * Bv);
  double* gr = filled(9 * (size_t)Br * P);
  double* gs = filled(2 * (size_t)(Bs ? Bs : 1) * P);
  double* gi = filled(2 * ni * B * P);
  double* gwi = filled(ni * B * P);
  CHECK(oracle_project(B, P, Bv, Br, Bs, D, H, interp, o, r, vol, rot, sh, out));
  CHECK(oracle_backproject(B, P, Bv, Br, Bs, D, H, interp, o, r, img, wimg, rot, sh, gv, gw));
  CHECK(oracle_backproject(B, P, Bv, Br, Bs, D, H, interp, o, r, img, NULL, rot, sh, gv, NULL));
  CHECK(oracle_project_backward(B, P, Bv, Br, Bs, D, H, interp, o, r, img, vol, rot, sh, gv, gr, Bs ? gs : NULL));
  CHECK(oracle_backproject_backward(B, P, Bv, Br, Bs, D, H, interp, o, r, vol, wvol, img, wimg, rot, sh, gi, gwi,
                                    gr, Bs ? gs : NULL));
  free(vol); free(wvol); free(rot); free(sh); free(img); free(wimg); free(out);
  free(gv); free(gw); free(gr); free(gs); free(gi); free(gwi);
}

static void case2d(int B, int P, int Bv, int Br, int Bs, int D, int H, int interp, double o, double r, int general) {
  const size_t nx = (size_t)D * (D / 2 + 1), ni = (size_t)H * (H / 2 + 1);
  double* src = filled(2 * nx * Bv);
  double* wsrc = filled(nx * Bv);
  double* rot = maps((size_t)Br * P, 2, general);
  double* sh = Bs ? filled(2 * (size_t)Bs * P) : NULL;
  double* img = filled(2 * ni * B * P);
  double* wimg = filled(ni * B * P);
  double* out = filled(2 * ni * B * P);
  double* gx = filled(2 * nx * Bv);
  double* gw = filled(nx * Bv);
  double* gr = filled(4 * (size_t)Br * P);
  double* gs = filled(2 * (size_t)(Bs ? Bs : 1) * P);
  double* gi = filled(2 * ni * B * P);
  double* gwi = filled(ni * B * P);
  CHECK(oracle_project2d(B, P, Bv, Br, Bs, D, H, interp, o, r, src, rot, sh, out));
  CHECK(oracle_backproject2d(B, P, Bv, Br, Bs, D, H, interp, o, r, img, wimg, rot, sh, gx, gw));
  CHECK(oracle_project2d_backward(B, P, Bv, Br, Bs, D, H, interp, o, r, img, src, rot, sh, gx, gr, Bs ? gs : NULL));
  CHECK(oracle_backproject2d_backward(B, P, Bv, Br, Bs, D, H, interp, o, r, src, wsrc, img, wimg, rot, sh, gi, gwi,
                                      gr, Bs ? gs : NULL));
  free(src); free(wsrc); free(rot); free(sh); free(img); free(wimg); free(out);
  free(gx); free(gw); free(gr); free(gs); free(gi); free(gwi);
}

int main(void) {
  for (int interp = 0; interp <= 1; ++interp) {
    /* B, P, Bv, Br, Bs, D, H, interp, o, r, general */
    case3d(1, 3, 1, 1, 1, 8, 8, interp, 1.0, -1.0, 0);
    case3d(2, 2, 1, 2, 2, 8, 12, interp, 1.0, 5.0, 0);
    case3d(2, 3, 2, 1, 0, 6, 4, interp, 2.0, -1.0, 0);
    case3d(1, 2, 1, 1, 1, 10, 10, interp, 1.0, 0.0, 0);
    case3d(2, 2, 2, 2, 1, 8, 8, interp, 0.7, 3.5, 1);
    case2d(1, 3, 1, 1, 1, 8, 8, interp, 1.0, -1.0, 0);
    case2d(2, 2, 1, 2, 2, 8, 12, interp, 1.0, 5.0, 0);
    case2d(2, 3, 2, 1, 0, 6, 4, interp, 2.0, -1.0, 1);
    case2d(1, 2, 1, 1, 1, 10, 10, interp, 1.0, 0.0, 0);
  }
  double s = 0.0;
  for (int i = -300; i <= 300; ++i)
    for (int interp = 0; interp <= 1; ++interp)
      s += oracle_kernel_weight(interp, i / 100.0) + oracle_kernel_dweight(interp, i / 100.0);
  /* invalid geometries are refused with a status, without touching buffers */
  if (oracle_project(1, 1, 1, 1, 0, 7, 8, 1, 1.0, -1.0, NULL, NULL, NULL, NULL) == 0) ++failures;
  if (oracle_project(2, 1, 3, 1, 0, 8, 8, 1, 1.0, -1.0, NULL, NULL, NULL, NULL) == 0) ++failures;
  if (oracle_project(1, 1, 1, 1, 0, 8, 8, 1, 0.0, -1.0, NULL, NULL, NULL, NULL) == 0) ++failures;
  if (oracle_project(1, 1, 1, 1, 0, 8, 8, 1, 1.0, NAN, NULL, NULL, NULL, NULL) == 0) ++failures;
  if (oracle_project(1, 1, 1, 1, 0, 8, 8, 1, 1.0, -1.0, NULL, NULL, NULL, NULL) == 0) ++failures;
  printf("oracle driver: %d failures (checksum %.6f)\n", failures, s);
  return failures ? 1 : 0;
}
