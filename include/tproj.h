/*
 * tproj.h -- C ABI of the MI355X (gfx950) differentiable Fourier-slice
 * projection library (libtproj.so).
 *
 * The operations are the ones the torch-projectors pages describe ("torch-
 * projectors: A High-Performance Differentiable Projection Library for
 * PyTorch"; citations name the summary page by language and section):
 *   - 3D->2D forward: the rotated central slice of a 3D Fourier volume
 *     (Spanish page, "Resumen tecnico" 2; Dutch page, Methodologie;
 *     French page, "Resume technique" 2);
 *   - 2D->3D back-projection: accumulation of 2D Fourier images, and of real
 *     weights for CTF correction, into a 3D volume (French page, 2);
 *   - the backward pass of each, with gradients for the inputs, the rotation
 *     matrices and the shifts (Spanish page 2; Dutch page, Methodologie);
 *   - linear or cubic Catmull-Rom (a = -0.5) interpolation, Friedel-symmetric
 *     lookup F(-k) = conj(F(k)), and 2D shifts applied as a Fourier phase
 *     (Dutch page, Methodologie; French page 2).
 *
 * Layout (all row-major, contiguous, device memory, PyTorch rfft format with
 * DC at index 0; Spanish page 2 and French page 2 fix the rfft format):
 *   volume   complex64 [Bv][D][D][D/2+1]    (z, y, x); x = 0..D/2 is the halved
 *                                             axis, z and y in fftfreq order
 *   images   complex64 [B][P][H][H/2+1]     kx = ix, ky = fftfreq(H)[iy]
 *   weights  float32   [B][P][H][H/2+1]     (real weight images)
 *   weight volume float32 [Bv][D][D][D/2+1]
 *   rot      float32   [Br][P][3][3]        rows/columns ordered (x, y, z)
 *   shifts   float32   [Bs][P][2]           (sx, sy) in pixels
 * complex64 = interleaved (re, im) float pairs, 8-byte aligned.
 *
 * Definitions (one reading of the pages where they leave a step open):
 *   slice coordinate   p = o * R * (kx, ky, 0)^T
 *   mask               M = (r < 0) || (kx^2 + ky^2 <= r^2)
 *   tap lookup         for an integer tap t, m = tx mod D; m <= D/2: the stored
 *                      entry (tz mod D, ty mod D, m); otherwise the conjugate
 *                      of (-tz mod D, -ty mod D, D - m)  -- per tap
 *   interpolation      linear: taps floor(p)+{0,1}; cubic: floor(p)+{-1..2}
 *                      with Keys weights (a = -1/2), 3D tensor product
 *   phase              phi = exp(-2 pi i (kx sx + ky sy) / H)
 *   forward            Y = M * phi * sum_t w(t) Vh(t)
 *   back-projection    the exact adjoint: every in-mask pixel adds
 *                      w * conj(phi) * Y (conjugated at a mirrored tap) and,
 *                      for the weight channel, w * Wimg (never conjugated)
 * Batch broadcast: each of Bv, Br, Bs is 1 or B; gradients of a broadcast
 * input are summed over the batch; a back-projection with Bv = 1 sums all
 * batch entries into the one volume.
 *
 * Conventions common to every entry point:
 *   - All array arguments are caller-allocated device pointers on the current
 *     HIP device.  The library never allocates or frees memory.  Outputs are
 *     overwritten (accumulating outputs are cleared on the stream first).
 *   - A NULL output pointer means "not requested": that work is skipped.
 *   - Calls are asynchronous and ordered on `stream` (a hipStream_t; NULL is
 *     the default stream).  No call synchronises.
 *   - `workspace` / `ws_bytes`: caller-provided scratch device memory of at
 *     least tp_workspace_size(geom, op) bytes (may be NULL when that is 0).
 *   - Errors: argument checks run on the host before anything is enqueued and
 *     return TP_E_NULL / TP_E_SHAPE / TP_E_VALUE / TP_E_WORKSPACE; a failed
 *     launch returns TP_E_LAUNCH.  tp_last_error_detail() then describes the
 *     failure (thread-local).  Nothing throws or aborts across the ABI.
 */
#ifndef TPROJ_H
#define TPROJ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TPROJ_ABI_VERSION 1

typedef enum {
  TP_OK = 0,
  TP_E_NULL = 1,      /* a required pointer is NULL                          */
  TP_E_SHAPE = 2,     /* a size is invalid (odd D or H, batch mismatch, ...) */
  TP_E_VALUE = 3,     /* a scalar or pointer alignment is invalid            */
  TP_E_DEVICE = 4,    /* no usable HIP device                                */
  TP_E_LAUNCH = 5,    /* a kernel launch failed                              */
  TP_E_WORKSPACE = 6  /* the workspace is smaller than tp_workspace_size()   */
} tp_status;

typedef enum { TP_LINEAR = 0, TP_CUBIC = 1 } tp_interp;

/* Geometry of one call.  B >= 1 batch entries, each with P >= 1 poses. */
typedef struct {
  int32_t B, P;          /* batch, poses per batch entry                        */
  int32_t Bv, Br, Bs;    /* volume / rotation / shift batch: 1 or B; Bs = 0 iff
                            shifts == NULL                                      */
  int32_t D;             /* volume box, even, 2..1024: [Bv][D][D][D/2+1]        */
  int32_t H;             /* image box, even, 2..4096:  [B][P][H][H/2+1]         */
  int32_t interp;        /* tp_interp                                           */
  float oversampling;    /* o > 0 (1 = none): p = o * R * (kx, ky, 0)            */
  float radius_cutoff;   /* r < 0: none; else pixels with kx^2+ky^2 <= r^2      */
} tp_geom;

/* Operation ids for tp_workspace_size. */
enum {
  TP_OP_PROJECT = 0, TP_OP_PROJECT_BACKWARD = 1, TP_OP_BACKPROJECT = 2, TP_OP_BACKPROJECT_BACKWARD = 3,
  TP_OP_PROJECT_2D = 4, TP_OP_PROJECT_2D_BACKWARD = 5, TP_OP_BACKPROJECT_2D = 6, TP_OP_BACKPROJECT_2D_BACKWARD = 7
};

/* 3D -> 2D forward (rotated central slice; Spanish page 2, French page 2).
 *   vol     [Bv][D][D][D/2+1] complex64, read
 *   rot     [Br][P][3][3] float32, read
 *   shifts  [Bs][P][2] float32 or NULL, read
 *   out     [B][P][H][H/2+1] complex64, written (0 outside the mask)        */
tp_status project_3d_to_2d(const tp_geom* geom, const void* vol, const float* rot, const float* shifts, void* out,
                           void* workspace, size_t ws_bytes, void* stream);

/* Backward of project_3d_to_2d (gradients for inputs, rotations and shifts;
 * Spanish page 2, Dutch page Methodologie).  With G = grad_out
 * (= dL/dRe + i dL/dIm of the forward output):
 *   grad_vol    [Bv][D][D][D/2+1] complex64 or NULL: the back-projection of G
 *   grad_rot    [Br][P][3][3] float32 or NULL:
 *               o * sum_k M Re(conj(G) phi dI/dp_i) * (kx, ky, 0)_j
 *               (column 2 is exactly 0)
 *   grad_shifts [Bs][P][2] float32 or NULL (needs shifts):
 *               (2 pi / H) sum_k M (kx, ky) Im(conj(G) Y)
 * vol is needed when grad_rot or grad_shifts is requested.                  */
tp_status project_3d_to_2d_backward(const tp_geom* geom, const void* grad_out, const void* vol, const float* rot,
                                    const float* shifts, void* grad_vol, float* grad_rot, float* grad_shifts,
                                    void* workspace, size_t ws_bytes, void* stream);

/* 2D -> 3D back-projection (accumulation into the volume, with weights for
 * CTF correction; French page 2).  The adjoint of project_3d_to_2d.
 *   images      [B][P][H][H/2+1] complex64, read
 *   weights     [B][P][H][H/2+1] float32 or NULL, read
 *   data_vol    [Bv][D][D][D/2+1] complex64, written
 *   weight_vol  [Bv][D][D][D/2+1] float32, written; NULL iff weights NULL    */
tp_status backproject_2d_to_3d(const tp_geom* geom, const void* images, const float* weights, const float* rot,
                               const float* shifts, void* data_vol, float* weight_vol, void* workspace,
                               size_t ws_bytes, void* stream);

/* Backward of backproject_2d_to_3d.  Upstream grads: grad_data_vol (complex,
 * required) and grad_weight_vol (float, NULL = zero).  Outputs, each NULL if
 * not requested:
 *   grad_images  [B][P][H][H/2+1] complex64: M phi I(grad_data_vol, p)
 *   grad_weights [B][P][H][H/2+1] float32:   M I(grad_weight_vol, p)
 *   grad_rot     [Br][P][3][3], grad_shifts [Bs][P][2]: as for the forward
 *                backward with (volume, upstream) = (grad_data_vol, images),
 *                plus the real weight channel (grad_weight_vol, weights).
 * images is needed for grad_rot / grad_shifts; weights for the weight-channel
 * term of grad_rot when grad_weight_vol is given.                          */
tp_status backproject_2d_to_3d_backward(const tp_geom* geom, const void* grad_data_vol,
                                        const float* grad_weight_vol, const void* images, const float* weights,
                                        const float* rot, const float* shifts, void* grad_images,
                                        float* grad_weights, float* grad_rot, float* grad_shifts, void* workspace,
                                        size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * 2D -> 2D (rotation of 2D Fourier data and accumulation into a 2D
 * reconstruction; Dutch page Methodologie, operations 1 and 2; Spanish page
 * 2).  The same definitions as the 3D calls one dimension down: the source is
 * a 2D rfft image of box D, the maps are 2x2, p = o * R * (kx, ky):
 *   src      [Bv][D][D/2+1] complex64 (the 2D reconstruction / reference)
 *   rot      [Br][P][2][2] float32, row-major, rows and columns (x, y)
 *   shifts, images, weights, masks, phases, Friedel rule: as above.
 * geom is the same struct (D = the source box).  Workspace: the periodic
 * Hermitian extension of the source(s) and, for the accumulation, per
 * workgroup partial sums (tp_workspace_size with the TP_OP_*_2D ids).
 * ------------------------------------------------------------------------- */

/* out [B][P][H][H/2+1] complex64 = M * phi * I(src[bv], o R k)             */
tp_status project_2d_to_2d(const tp_geom* geom, const void* src, const float* rot, const float* shifts, void* out,
                           void* workspace, size_t ws_bytes, void* stream);

/* Backward of project_2d_to_2d: grad_src [Bv][D][D/2+1] complex64 (the
 * accumulation of grad_out), grad_rot [Br][P][2][2] (o * sum_k M Re(conj(G)
 * phi dI/dp_i) k_j), grad_shifts [Bs][P][2]; each NULL if not requested; src
 * is needed for grad_rot / grad_shifts.                                    */
tp_status project_2d_to_2d_backward(const tp_geom* geom, const void* grad_out, const void* src, const float* rot,
                                    const float* shifts, void* grad_src, float* grad_rot, float* grad_shifts,
                                    void* workspace, size_t ws_bytes, void* stream);

/* Accumulation into 2D reconstructions (the adjoint of project_2d_to_2d),
 * with real weights: data [Bv][D][D/2+1] complex64, weight_out
 * [Bv][D][D/2+1] float32 (NULL iff weights NULL), both written.             */
tp_status backproject_2d_to_2d(const tp_geom* geom, const void* images, const float* weights, const float* rot,
                               const float* shifts, void* data, float* weight_out, void* workspace,
                               size_t ws_bytes, void* stream);

/* Backward of backproject_2d_to_2d (as backproject_2d_to_3d_backward, with
 * grad_data [Bv][D][D/2+1] complex64 and grad_weight [Bv][D][D/2+1] float32
 * or NULL; grad_rot is [Br][P][2][2]).                                      */
tp_status backproject_2d_to_2d_backward(const tp_geom* geom, const void* grad_data, const float* grad_weight,
                                        const void* images, const float* weights, const float* rot,
                                        const float* shifts, void* grad_images, float* grad_weights,
                                        float* grad_rot, float* grad_shifts, void* workspace, size_t ws_bytes,
                                        void* stream);

/* Allocation-free variant of project_3d_to_2d, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, results and errors as
 * project_3d_to_2d, minus the workspace: the forward's work area (work list
 * and hit lists, tp_workspace_size(geom, TP_OP_PROJECT) bytes) lives in a
 * library-owned static device array of TP_NOALLOC_SCRATCH_BYTES, one per GPU,
 * held until the process ends.  A geometry that needs more is rejected with
 * TP_E_WORKSPACE before anything is enqueued (D = 128 with 16384 poses needs
 * about 24 MB).  The call enqueues on `stream` only (no side stream, no
 * timing events) and allocates nothing.  Every call on one GPU shares that
 * GPU's array: calls that overlap on one GPU (two streams, two threads) race
 * and must be serialised by the caller.  The array keeps the last call's
 * contents; the kernels rewrite every part of it they read, so nothing needs
 * clearing between calls.                                                   */
#define TP_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
tp_status project_3d_to_2d_noalloc(const tp_geom* geom, const void* vol, const float* rot, const float* shifts,
                                   void* out, void* stream);

/* Bytes of workspace the operation `op` (TP_OP_*) needs for this geometry
 * (0 when none).  Returns (size_t)-1 for an invalid geometry.  The brick
 * kernels keep there their work list and per work item the list of poses
 * that reach the brick (2 bytes per pose and active brick, e.g. 23 MB for
 * D = 128 with 16384 poses); the back-projection adds its band maxima and
 * one 16^3 partial tile per work item.                                      */
size_t tp_workspace_size(const tp_geom* geom, int op);

/* Event timing of the brick kernels (benchmarks, profiling).  Kernel classes: */
enum {
  TP_KT_FORWARD = 0,   /* forward gather brick kernel (complex or real volume)           */
  TP_KT_BACKWARD = 1,  /* back-projection (scatter) brick kernel                          */
  TP_KT_GRADIENT = 2,  /* rotation/shift gradient brick kernel                           */
  TP_KT_FOLD = 3,      /* fold of the back-projection partial tiles into the volume      */
  TP_KT_COUNT = 4
};
/* on != 0: from now on every call records a pair of HIP events on its stream
 * around each brick kernel it launches (the events are created by the library
 * and destroyed by tp_timing_read); on = 0 stops recording.  Process-wide host
 * state; calls that record must not run concurrently with tp_timing_read. */
tp_status tp_timing_enable(int on);
/* Waits for the recorded events of one kernel class, returns their summed
 * elapsed milliseconds and their count since the previous read of that class,
 * and forgets them.  TP_E_NULL for NULL outputs, TP_E_VALUE for an unknown
 * class, TP_E_LAUNCH if an event query fails.                              */
tp_status tp_timing_read(int kernel_class, double* total_ms, int64_t* launches);

/* Host-only argument check of a geometry (no GPU needed).                  */
tp_status tp_validate(const tp_geom* geom);

/* Text of a status code; any int (codes outside tp_status give "unknown
 * status").                                                               */
const char* tp_status_string(int s);
/* Text of the last failure on the calling thread ("" if none).             */
const char* tp_last_error_detail(void);
int tp_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TPROJ_H */
