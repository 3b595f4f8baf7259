/* Sanitizer driver for the host layer of libtproj (argument and geometry
 * checks, workspace planning, status strings, the timing switches, the
 * spectral entry points' checks and the fixed-point bounds): every call here
 * is decided on the host, before any device work, so the driver needs no GPU
 * and never launches anything.  Built with AddressSanitizer and
 * UndefinedBehaviorSanitizer against a host-only build of the library by
 * tests/test_sanitizers.py; any out-of-bounds access or undefined behaviour
 * aborts with a report, any unexpected status is a failure. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "tproj.h"
#include "tproj_bounds.h"
#include "tproj_spectral.h"

static int failures = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "line %d: expected %s\n", __LINE__, #cond);      \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

/* an aligned stand-in for a device pointer that is never dereferenced */
#define FAKE ((void*)(uintptr_t)0x100000)
#define ODD ((void*)(uintptr_t)0x100002)

static tp_geom geom(int B, int P, int Bv, int Br, int Bs, int D, int H, int interp, float o, float r) {
  tp_geom g;
  memset(&g, 0, sizeof g);
  g.B = B; g.P = P; g.Bv = Bv; g.Br = Br; g.Bs = Bs; g.D = D; g.H = H; g.interp = interp;
  g.oversampling = o; g.radius_cutoff = r;
  return g;
}

int main(void) {
  /* geometry sweep: validation and the workspace plans of every operation */
  const int Ds[] = {2, 4, 8, 16, 32, 64, 128, 192, 256, 512, 1024};
  const int Ps[] = {1, 7, 64, 1024, 16384};
  const float rs[] = {-1.0f, 0.0f, 0.5f, 16.0f, 64.0f, 1e6f};
  size_t acc = 0;
  for (size_t a = 0; a < sizeof Ds / sizeof *Ds; ++a)
    for (size_t b = 0; b < sizeof Ps / sizeof *Ps; ++b)
      for (size_t c = 0; c < sizeof rs / sizeof *rs; ++c)
        for (int interp = 0; interp <= 1; ++interp)
          for (int hm = 0; hm < 3; ++hm) {
            const int D = Ds[a], H = hm == 0 ? D : (hm == 1 ? (D > 2 ? D / 2 : 2) : 2 * D);
            const float o = hm == 2 ? 2.0f : 1.0f;
            tp_geom g = geom(2, Ps[b], 1, 2, 2, D, H > 4096 ? 4096 : H, interp, o, rs[c]);
            EXPECT(tp_validate(&g) == TP_OK);
            for (int op = 0; op <= 7; ++op) acc += tp_workspace_size(&g, op) & 1;
          }
  /* invalid geometries: each rejected with its status, and no workspace size */
  tp_geom bad[] = {
      geom(1, 1, 1, 1, 0, 7, 8, 1, 1.0f, -1.0f),          /* odd D */
      geom(1, 1, 1, 1, 0, 8, 9, 1, 1.0f, -1.0f),          /* odd H */
      geom(1, 1, 1, 1, 0, 2048, 8, 1, 1.0f, -1.0f),       /* D too large */
      geom(0, 1, 1, 1, 0, 8, 8, 1, 1.0f, -1.0f),          /* B = 0 */
      geom(2, 1, 3, 1, 0, 8, 8, 1, 1.0f, -1.0f),          /* Bv neither 1 nor B */
      geom(2, 1, 1, 2, 3, 8, 8, 1, 1.0f, -1.0f),          /* Bs */
      geom(1, 1, 1, 1, 0, 8, 8, 5, 1.0f, -1.0f),          /* interp */
      geom(1, 1, 1, 1, 0, 8, 8, 1, 0.0f, -1.0f),          /* o = 0 */
      geom(1, 1, 1, 1, 0, 8, 8, 1, NAN, -1.0f),           /* o NaN */
      geom(1, 1, 1, 1, 0, 8, 8, 1, 1.0f, NAN),            /* r NaN */
      geom(1, -3, 1, 1, 0, 8, 8, 1, 1.0f, -1.0f),         /* P < 0 */
  };
  for (size_t i = 0; i < sizeof bad / sizeof *bad; ++i) {
    const tp_status s = tp_validate(&bad[i]);
    EXPECT(s != TP_OK && s != TP_E_DEVICE && s != TP_E_LAUNCH);
    EXPECT(strlen(tp_last_error_detail()) > 0);
    for (int op = 0; op <= 7; ++op) EXPECT(tp_workspace_size(&bad[i], op) == (size_t)-1);
  }
  EXPECT(tp_validate(NULL) == TP_E_NULL);
  EXPECT(tp_workspace_size(NULL, 0) == (size_t)-1);
  tp_geom ok = geom(1, 4, 1, 1, 1, 16, 16, 1, 1.0f, 8.0f);
  EXPECT(tp_workspace_size(&ok, 99) == (size_t)-1);

  /* entry points with bad arguments: rejected before any device work */
  tp_geom ok0 = geom(1, 4, 1, 1, 0, 16, 16, 1, 1.0f, 8.0f);   /* no shifts */
  EXPECT(project_3d_to_2d(NULL, FAKE, FAKE, NULL, FAKE, NULL, 0, NULL) == TP_E_NULL);
  EXPECT(project_3d_to_2d(&ok0, NULL, FAKE, NULL, FAKE, NULL, 0, NULL) == TP_E_NULL);
  EXPECT(project_3d_to_2d(&ok0, ODD, FAKE, NULL, FAKE, NULL, 0, NULL) == TP_E_VALUE);
  EXPECT(project_3d_to_2d(&ok0, FAKE, FAKE, FAKE, FAKE, NULL, 0, NULL) == TP_E_VALUE);   /* shifts, Bs = 0 */
  EXPECT(project_3d_to_2d(&ok, FAKE, FAKE, NULL, FAKE, NULL, 0, NULL) == TP_E_VALUE);    /* Bs = 1, no shifts */
  EXPECT(project_3d_to_2d(&bad[0], FAKE, FAKE, NULL, FAKE, NULL, 0, NULL) == TP_E_SHAPE);
  EXPECT(project_3d_to_2d_noalloc(&ok0, FAKE, FAKE, NULL, NULL, NULL) == TP_E_NULL);
  tp_geom big = geom(1, 65536, 1, 1, 0, 128, 128, 1, 1.0f, 64.0f);
  EXPECT(project_3d_to_2d_noalloc(&big, FAKE, FAKE, NULL, FAKE, NULL) == TP_E_WORKSPACE);
  EXPECT(project_3d_to_2d_backward(&ok0, NULL, FAKE, FAKE, NULL, FAKE, NULL, NULL, NULL, 0, NULL) == TP_E_NULL);
  EXPECT(project_3d_to_2d_backward(&ok0, FAKE, NULL, FAKE, NULL, NULL, FAKE, NULL, NULL, 0, NULL) == TP_E_NULL);
  EXPECT(project_3d_to_2d_backward(&ok0, FAKE, FAKE, FAKE, NULL, FAKE, NULL, NULL, FAKE, 16, NULL) ==
         TP_E_WORKSPACE);
  EXPECT(backproject_2d_to_3d(&ok0, FAKE, FAKE, FAKE, NULL, FAKE, NULL, NULL, 0, NULL) == TP_E_NULL);
  EXPECT(backproject_2d_to_3d(&ok0, FAKE, NULL, ODD, NULL, FAKE, NULL, NULL, 0, NULL) == TP_E_VALUE);
  EXPECT(backproject_2d_to_3d_backward(&ok0, NULL, NULL, FAKE, NULL, FAKE, NULL, FAKE, NULL, NULL, NULL, NULL, 0,
                                       NULL) == TP_E_NULL);
  tp_geom ok2 = geom(1, 4, 1, 1, 0, 16, 16, 1, 1.0f, 8.0f);
  EXPECT(project_2d_to_2d(&ok2, NULL, FAKE, NULL, FAKE, NULL, 0, NULL) == TP_E_NULL);
  EXPECT(project_2d_to_2d_backward(&ok2, FAKE, NULL, FAKE, NULL, NULL, FAKE, NULL, NULL, 0, NULL) == TP_E_NULL);
  EXPECT(backproject_2d_to_2d(&ok2, FAKE, FAKE, FAKE, NULL, FAKE, NULL, NULL, 0, NULL) == TP_E_NULL);
  EXPECT(backproject_2d_to_2d_backward(&ok2, NULL, NULL, FAKE, NULL, FAKE, NULL, FAKE, NULL, NULL, NULL, NULL, 0,
                                       NULL) == TP_E_NULL);

  /* status strings, ABI version, timing switches */
  for (int s = -2; s < 12; ++s) EXPECT(tp_status_string(s) != NULL);
  EXPECT(tp_abi_version() == 1);
  double ms = -1.0;
  int64_t n = -1;
  EXPECT(tp_timing_read(0, &ms, &n) == TP_OK && ms == 0.0 && n == 0);
  EXPECT(tp_timing_read(9, &ms, &n) == TP_E_VALUE);
  EXPECT(tp_timing_read(1, NULL, &n) == TP_E_NULL);
  EXPECT(tp_timing_enable(1) == TP_OK && tp_timing_enable(0) == TP_OK);

  /* spectral entry points: shapes and pointers checked on the host */
  EXPECT(tp_volume_rfft(7, 1, 1, NULL, NULL, NULL, 0, NULL) == TP_E_SHAPE);
  EXPECT(tp_volume_rfft(512, 4, 1, NULL, NULL, NULL, 0, NULL) == TP_E_SHAPE);
  EXPECT(tp_volume_rfft_workspace(63, 1, 1) == (size_t)-1);
  EXPECT(tp_images_irfft(9, 1, NULL, NULL, NULL, 0, NULL) == TP_E_SHAPE);
  EXPECT(tp_images_irfft(64, 0, NULL, NULL, NULL, 0, NULL) == TP_OK);
  EXPECT(tp_weight_images(10, 3, NULL, NULL, NULL, NULL) == TP_E_SHAPE);
  EXPECT(tp_finish_reconstruction(4, NULL, NULL, -1.0f, NULL, NULL) == TP_E_VALUE);

  /* fixed-point bounds on many maps, and the device variant's host checks */
  unsigned s = 12345u;
  for (int m = 0; m < 2000; ++m) {
    float R[9];
    for (int q = 0; q < 9; ++q) {
      s = s * 1664525u + 1013904223u;
      R[q] = (float)((int)(s >> 8) % 2001 - 1000) / 500.0f;
    }
    for (int interp = 0; interp <= 1; ++interp) {
      const float w = tp_weight_sum_bound_3d(interp, 1.0f, R), c = tp_contrib_bound_3d(interp, 1.5f, R);
      const float w2 = tp_weight_sum_bound_2d(interp, 1.0f, 40.0f, 64, R);
      EXPECT(w > 0.0f && c >= 1.0f && w2 > 0.0f);
    }
  }
  EXPECT(tp_bounds_device(5, 1, 1.0f, 0.0f, 8, NULL, 1, NULL) == TP_E_VALUE);
  EXPECT(tp_bounds_device(0, 1, 1.0f, 0.0f, 8, NULL, 1, NULL) == TP_E_NULL);

  printf("host-layer driver: %d failures (%zu)\n", failures, acc);
  return failures ? 1 : 0;
}
