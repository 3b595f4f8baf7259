// Host C ABI of libtproj: argument checks, kernel selection and launches.
// Declared in include/tproj.h; the operations are those of the torch-projectors
// pages (3D->2D forward, 2D->3D back-projection, and their backward passes).
#include "tproj.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <string>
#include <vector>

#include "brick_grid.h"
#include "brick_kernels.h"
#include "kernels.h"
#include "bwd_kernels.h"
#include "kernels_2d.h"

// The static work area of project_3d_to_2d_noalloc: a file-scope device
// array, so every GPU the library runs on holds its own copy for the life of
// the process.  Host code never uses the array's name as an address (on the
// host it only names the symbol); the device address of the current GPU's
// copy comes from hipGetSymbolAddress, once per device on that device's first
// call (scratch_address below), and only that address is passed on.
static __device__ __align__(256) unsigned char scratch[TP_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_detail;

tp_status fail(tp_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_detail = buf;
  return s;
}

tp_status ok() {
  g_detail.clear();
  return TP_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Pure check of the geometry (no GPU).
tp_status check_geom(const tp_geom* g) {
  if (!g) return fail(TP_E_NULL, "geometry pointer is NULL");
  if (g->B < 1 || g->P < 1) return fail(TP_E_SHAPE, "B=%d and P=%d must be >= 1", g->B, g->P);
  if (g->D < 2 || g->D > 1024 || (g->D & 1)) return fail(TP_E_SHAPE, "D=%d must be even and in [2, 1024]", g->D);
  if (g->H < 2 || g->H > 4096 || (g->H & 1)) return fail(TP_E_SHAPE, "H=%d must be even and in [2, 4096]", g->H);
  if (g->Bv != 1 && g->Bv != g->B) return fail(TP_E_SHAPE, "Bv=%d must be 1 or B=%d", g->Bv, g->B);
  if (g->Br != 1 && g->Br != g->B) return fail(TP_E_SHAPE, "Br=%d must be 1 or B=%d", g->Br, g->B);
  if (g->Bs != 0 && g->Bs != 1 && g->Bs != g->B) return fail(TP_E_SHAPE, "Bs=%d must be 0, 1 or B=%d", g->Bs, g->B);
  if (g->interp != TP_LINEAR && g->interp != TP_CUBIC) return fail(TP_E_VALUE, "interp=%d is not 0 or 1", g->interp);
  if (!std::isfinite(g->oversampling) || !(g->oversampling > 0.0f))
    return fail(TP_E_VALUE, "oversampling=%g must be finite and > 0", (double)g->oversampling);
  if (std::isnan(g->radius_cutoff)) return fail(TP_E_VALUE, "radius_cutoff is NaN");
  const int64_t npose = (int64_t)g->B * g->P;
  const int64_t nimg = npose * g->H * (g->H / 2 + 1);
  if (npose > INT32_MAX / 2 || nimg > ((int64_t)1 << 40))
    return fail(TP_E_SHAPE, "B*P=%lld poses / %lld pixels exceed the supported size", (long long)npose,
                (long long)nimg);
  return TP_OK;
}

tp_status check_shifts(const tp_geom* g, const float* shifts) {
  if (shifts == nullptr && g->Bs != 0) return fail(TP_E_VALUE, "shifts is NULL but Bs=%d (must be 0)", g->Bs);
  if (shifts != nullptr && g->Bs == 0) return fail(TP_E_VALUE, "shifts given but Bs=0");
  return TP_OK;
}

tp_status check_ptr(const void* p, const char* name, size_t align) {
  if (!p) return fail(TP_E_NULL, "%s is NULL", name);
  if (!aligned(p, align)) return fail(TP_E_VALUE, "%s is not %zu-byte aligned", name, align);
  return TP_OK;
}

tp_status check_opt(const void* p, const char* name, size_t align) {
  if (p && !aligned(p, align)) return fail(TP_E_VALUE, "%s is not %zu-byte aligned", name, align);
  return TP_OK;
}

tproj::KGeom kgeom(const tp_geom* g) {
  tproj::KGeom k;
  k.B = g->B; k.P = g->P; k.Bv = g->Bv; k.Br = g->Br; k.Bs = g->Bs;
  k.D = g->D; k.H = g->H; k.half = g->D / 2; k.W = g->D / 2 + 1; k.Wi = g->H / 2 + 1;
  k.npix = g->H * k.Wi;
  k.o = g->oversampling;
  k.r2 = g->radius_cutoff < 0.0f ? -1.0f : g->radius_cutoff * g->radius_cutoff;
  k.inv_h = 1.0f / (float)g->H;
  {
    const double h = g->H / 2;
    double km = std::sqrt(2.0) * h;
    if (g->radius_cutoff >= 0.0f) km = std::min(km, (double)g->radius_cutoff);
    k.kmax = (float)(km * (1.0 + 1e-6));
  }
  return k;
}

// Pixels of one image inside the radius cutoff.
int64_t pixels_in_mask(const tp_geom* g) {
  const int64_t half = g->H / 2;
  if (g->radius_cutoff < 0.0f) return (int64_t)g->H * (half + 1);
  const double r2 = (double)g->radius_cutoff * g->radius_cutoff;
  int64_t n = 0;
  for (int64_t ky = -half; ky < half; ++ky) {
    const double rem = r2 - (double)(ky * ky);
    if (rem < 0) continue;
    int64_t m = (int64_t)std::floor(std::sqrt(rem));
    while ((m + 1) * (m + 1) + ky * ky <= r2) ++m;
    while (m >= 0 && m * m + ky * ky > r2) --m;
    n += std::min(m, half) + 1;
  }
  return n;
}

// Brick grid of the gather kernels for this geometry; ok = false when the
// brick path does not apply (grid too large) and the direct kernels run.
struct GatherPlan {
  bool ok = false;
  tproj::BrickGrid bg{};
  size_t ws_bytes = 0;   // work area: work list, hit counts, hit lists
};

bool force_direct() {
  static const bool v = [] {
    const char* e = std::getenv("TPROJ_KERNELS");
    return e && std::string(e) == "direct";
  }();
  return v;
}

// ---- event timing of the brick kernels (tp_timing_enable / tp_timing_read) ----
struct TimedLaunch {
  int cls;
  tproj::EvPair ev;
};
std::mutex g_kt_mu;
bool g_kt_on = false;
std::vector<TimedLaunch> g_kt;

// A fresh event pair for one launch of kernel class cls (both events NULL
// when timing is off or the events cannot be created).
tproj::EvPair kt_copy(int cls) {
  std::lock_guard<std::mutex> lk(g_kt_mu);
  TimedLaunch t{cls, {}};
  if (!g_kt_on) return t.ev;
  if (hipEventCreate(&t.ev.a) != hipSuccess) return tproj::EvPair{};
  if (hipEventCreate(&t.ev.b) != hipSuccess) {
    (void)hipEventDestroy(t.ev.a);
    return tproj::EvPair{};
  }
  g_kt.push_back(t);
  return t.ev;
}

// items: work items aimed at (the pixel load split evenly); min_px: least
// pixels per item, so that small problems do not drown in per-item costs.
GatherPlan gather_plan(const tp_geom* g, int64_t items = 8192, int64_t min_px = 2048, int S = 0) {
  GatherPlan pl;
  if (force_direct()) return pl;
  // the brick enumeration packs kx <= H/2 into 11 bits and one image row's
  // candidates into its 2048-entry table
  if (g->H / 2 > 2047) return pl;
  tproj::BrickGrid& bg = pl.bg;
  const int NT = g->interp == TP_CUBIC ? 4 : 2;
  bg.S = S > 0 ? S : 17 - NT;
  double kmax = std::sqrt(2.0) * (g->H / 2);
  if (g->radius_cutoff >= 0.0f) kmax = std::min(kmax, (double)g->radius_cutoff);
  const double pmax = (double)g->oversampling * kmax;
  if (pmax > 1e5) return pl;
  bg.pmax_i = (int)std::ceil(pmax) + 1;
  bg.origin = -bg.pmax_i - 1;
  bg.nb = (2 * bg.pmax_i + 2 + bg.S - 1) / bg.S;
  const int64_t nb3 = (int64_t)bg.nb * bg.nb * bg.nb;
  if (nb3 > (1 << 20)) return pl;
  bg.nb3 = (int)nb3;
  bg.list_len = (g->Bv == 1 ? g->B : 1) * g->P;
  bg.dens_q8 = std::max(1, (int)std::lround(256.0 / ((double)g->oversampling * g->oversampling)));
  const int64_t total = (int64_t)g->B * g->P * pixels_in_mask(g);
  bg.target = std::max<int64_t>(min_px, total / items);
  int64_t nwork = 0, nactive = 0;
  for (int b = 0; b < bg.nb3; ++b) {
    int bi, bj, bk;
    tproj::brick_coords(bg, b, bi, bj, bk);
    const int k = tproj::brick_chunks(bg, bi, bj, bk);
    nwork += k;
    nactive += k > 0;
  }
  if (nwork > INT32_MAX / 2) return pl;
  bg.nwork = (int)nwork;
  bg.nactive = (int)nactive;
  // work list, hit counts and hit lists (16-bit offsets: every pose of the
  // list once per active brick and volume)
  pl.ws_bytes = tproj::brick_work_bytes(bg, g->Bv);
  pl.ok = true;
  return pl;
}

// Brick plan of the back-projection (the forward's tap-space bricks plus the
// radial band tables of the fixed-point scale); ok = false -> direct kernels.
struct BwdPlan {
  bool ok = false;
  tproj::BwdGrid bw{};
  size_t ws_bytes = 0;
};

BwdPlan bwd_plan(const tp_geom* g, bool weights) {
  BwdPlan pl;
  // each work item writes a 16^3 partial tile (the chunks of a brick are
  // summed before the fold): fewer, larger items than the gather at large
  // sizes, at least 2048 pixels each
  const GatherPlan gp = gather_plan(g, 4096, 2048, tproj::bwd_brick_edge(g->interp));
  if (!gp.ok) return pl;
  tproj::BwdGrid& bw = pl.bw;
  bw.bg = gp.bg;
  bw.npose = g->B * g->P;
  const double kimg = std::sqrt(2.0) * (g->H / 2) + 1.0;
  const double band = std::max(1.0, std::ceil(kimg / 64.0));
  bw.nbands = (int)std::ceil(kimg / band) + 1;
  bw.inv_band_w = (float)(1.0 / band);
  pl.ws_bytes = tproj::bwd_ws_bytes(bw, g->Bv, weights);
  // every active brick writes at least one partial tile: very large boxes
  // with few poses would need more scratch than they are worth; those use the
  // direct kernels
  if (pl.ws_bytes > ((size_t)4 << 30)) return BwdPlan{};
  pl.ok = true;
  return pl;
}

int64_t vol_elems(const tp_geom* g) { return (int64_t)g->D * g->D * (g->D / 2 + 1); }
int64_t img_elems(const tp_geom* g) { return (int64_t)g->B * g->P * g->H * (g->H / 2 + 1); }

tp_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(TP_E_LAUNCH, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

size_t align_up(size_t n) { return (n + 255) / 256 * 256; }

tp_status check_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return fail(TP_E_DEVICE, "no usable HIP device: %s", hipGetErrorString(e));
  }
  return TP_OK;
}

#define TRY(x)                      \
  do {                              \
    tp_status _s = (x);             \
    if (_s != TP_OK) return _s;     \
  } while (0)
#define LAUNCH(x, what)                               \
  do {                                                \
    hipError_t _e = (x);                              \
    if (_e != hipSuccess) return launched(_e, what);  \
  } while (0)

size_t workspace_need(const tp_geom* g, int op);

// The workspace is checked before anything is enqueued.
tp_status check_workspace(const tp_geom* g, int op, const void* ws, size_t ws_bytes) {
  const size_t need = workspace_need(g, op);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(TP_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu bytes needed", ws_bytes, need);
  return TP_OK;
}

// A second stream per device for the rotation / shift gradients of the
// forward's backward: they read only the upstream gradient, the volume and the
// poses, so they run beside the back-projection (the two kernels are limited
// by different units: memory latency and LDS atomics vs. VALU).  The fork and
// the join are events recorded on the caller's stream and on this one; one
// mutex keeps a call's record / wait pairs together.  Default priority.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  bool tried = false, ok = false;
};
constexpr int MAX_DEVICES = 64;
SideStream g_side[MAX_DEVICES];
std::mutex g_side_mu;

// Splitting pays only when the kernels run long enough to hide the cost of
// the cross-stream events (some tens of microseconds): measured, from about
// 2^20 image pixels for the backward's two big kernels and 2^23 for the
// forward's small edge kernel.
// A stream being captured into a graph is never split: the capture then
// holds exactly the one-stream sequence.
bool worth_splitting(const tp_geom* g, int log2_pixels, hipStream_t st) {
  if ((int64_t)g->B * g->P * g->H * (g->H / 2 + 1) < (int64_t)1 << log2_pixels) return false;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cs) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return cs == hipStreamCaptureStatusNone;
}

// Call with g_side_mu held.  NULL if the device has no side stream.
SideStream* side_stream() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) {
    (void)hipGetLastError();
    return nullptr;
  }
  SideStream& ss = g_side[dev];
  if (!ss.tried) {
    ss.tried = true;
    ss.ok = hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking) == hipSuccess &&
            hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming) == hipSuccess &&
            hipEventCreateWithFlags(&ss.join, hipEventDisableTiming) == hipSuccess;
    if (!ss.ok) (void)hipGetLastError();   // the callers then run serially
  }
  return ss.ok ? &ss : nullptr;
}

// Forward gather: brick-binned kernels when the plan applies, else direct.
// may_alloc = false: no timing events and no side stream (whose first use
// creates a stream and events): everything on st.
tp_status run_forward(const tp_geom* geom, const tproj::KGeom& k, const float2* vol, const float* rot,
                      const float* shifts, float2* out, void* workspace, size_t ws_bytes, hipStream_t st,
                      bool may_alloc = true) {
  const GatherPlan pl = gather_plan(geom);
  if (!pl.ok) {
    LAUNCH(tproj::launch_project(k, geom->interp, vol, rot, shifts, out, st), "project");
    return TP_OK;
  }
  if (!workspace || ws_bytes < pl.ws_bytes)
    return fail(TP_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu bytes needed", ws_bytes, pl.ws_bytes);
  const tproj::BrickWork wk = tproj::brick_work(pl.bg, geom->Bv, workspace);
  const tproj::EvPair ev = may_alloc ? kt_copy(TP_KT_FORWARD) : tproj::EvPair{};
  // the edge kernel on the side stream, beside the work list and the bricks
  std::lock_guard<std::mutex> lk(g_side_mu);
  SideStream* ss = may_alloc && worth_splitting(geom, 23, st) ? side_stream() : nullptr;
  hipStream_t se = st;
  if (ss) {
    hipError_t e = hipEventRecord(ss->fork, st);
    if (e == hipSuccess) e = hipStreamWaitEvent(ss->s, ss->fork, 0);
    if (e != hipSuccess) return fail(TP_E_LAUNCH, "stream fork failed: %s", hipGetErrorString(e));
    se = ss->s;
  }
  tp_status r = TP_OK;
  hipError_t e = tproj::launch_brick_prefix(pl.bg, wk.prefix, st);
  if (e == hipSuccess)
    e = tproj::launch_fwd_brick(k, geom->interp, pl.bg, wk, vol, rot, shifts, out, st, ev.a ? &ev : nullptr, se);
  if (e != hipSuccess) r = fail(TP_E_LAUNCH, "project (bricks): %s", hipGetErrorString(e));
  if (ss) {
    hipError_t ej = hipEventRecord(ss->join, ss->s);
    if (ej == hipSuccess) ej = hipStreamWaitEvent(st, ss->join, 0);
    if (ej != hipSuccess && r == TP_OK) r = fail(TP_E_LAUNCH, "stream join failed: %s", hipGetErrorString(ej));
  }
  return r;
}

// Rotation / shift gradients into zeroed outputs: bricks, else direct.
tp_status run_grads(const tp_geom* geom, const tproj::KGeom& k, const float2* volc, const float* volr,
                    const float2* U, const float* Ur, const float* rot, const float* shifts, float* grad_rot,
                    float* grad_shifts, void* workspace, size_t ws_bytes, hipStream_t st) {
  if (grad_rot) LAUNCH(tproj::launch_zero(grad_rot, 9 * (int64_t)geom->Br * geom->P, st), "zero grad_rot");
  if (grad_shifts) LAUNCH(tproj::launch_zero(grad_shifts, 2 * (int64_t)geom->Bs * geom->P, st), "zero grad_shifts");
  const GatherPlan pl = gather_plan(geom);
  if (!pl.ok) {
    LAUNCH(tproj::launch_rot_shift_grad(k, geom->interp, volc, volr, U, Ur, rot, shifts, grad_rot, grad_shifts, st),
           "rotation/shift grads");
    return TP_OK;
  }
  if (!workspace || ws_bytes < pl.ws_bytes)
    return fail(TP_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu bytes needed", ws_bytes, pl.ws_bytes);
  const tproj::BrickWork wk = tproj::brick_work(pl.bg, geom->Bv, workspace);
  LAUNCH(tproj::launch_brick_prefix(pl.bg, wk.prefix, st), "brick work list");
  const tproj::EvPair ev = kt_copy(TP_KT_GRADIENT);
  LAUNCH(tproj::launch_grad_brick(k, geom->interp, pl.bg, wk, volc, volr, U, Ur, rot, shifts, grad_rot,
                                  grad_shifts, st, ev.a ? &ev : nullptr),
         "rotation/shift grads (bricks)");
  return TP_OK;
}

tp_status run_forward_real(const tp_geom* geom, const tproj::KGeom& k, const float* vol, const float* rot,
                           float* out, void* workspace, size_t ws_bytes, hipStream_t st) {
  const GatherPlan pl = gather_plan(geom);
  if (!pl.ok) {
    LAUNCH(tproj::launch_project_real(k, geom->interp, vol, rot, out, st), "real projection");
    return TP_OK;
  }
  if (!workspace || ws_bytes < pl.ws_bytes)
    return fail(TP_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu bytes needed", ws_bytes, pl.ws_bytes);
  const tproj::BrickWork wk = tproj::brick_work(pl.bg, geom->Bv, workspace);
  LAUNCH(tproj::launch_brick_prefix(pl.bg, wk.prefix, st), "brick work list");
  const tproj::EvPair ev = kt_copy(TP_KT_FORWARD);
  LAUNCH(tproj::launch_fwd_brick_real(k, geom->interp, pl.bg, wk, vol, rot, out, st, ev.a ? &ev : nullptr),
         "real projection (bricks)");
  return TP_OK;
}

// Back-projection of Y (and of the weight images Wimg into wvol): bricks,
// else zeroed volumes and direct atomics.  may_split: the caller does not use
// the side stream in this call, so the band maxima may run on it (large calls
// only, never under graph capture).
tp_status run_bwd(const tp_geom* geom, const tproj::KGeom& k, const float2* Y, const float* Wimg, const float* rot,
                  const float* shifts, float2* vol, float* wvol, void* workspace, size_t ws_bytes, hipStream_t st,
                  bool may_split = false) {
  const BwdPlan pl = bwd_plan(geom, Wimg != nullptr);
  if (!pl.ok) {
    LAUNCH(tproj::launch_zero((float*)vol, 2 * vol_elems(geom) * geom->Bv, st), "zero volume");
    if (wvol) LAUNCH(tproj::launch_zero(wvol, vol_elems(geom) * geom->Bv, st), "zero weight volume");
    LAUNCH(tproj::launch_spread_atomic(k, geom->interp, Y, Wimg, rot, shifts, vol, wvol, st), "scatter");
    return TP_OK;
  }
  if (!workspace || ws_bytes < pl.ws_bytes)
    return fail(TP_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu bytes needed", ws_bytes, pl.ws_bytes);
  const tproj::EvPair eb = kt_copy(TP_KT_BACKWARD), ef = kt_copy(TP_KT_FOLD);
  if (may_split && worth_splitting(geom, 20, st)) {
    std::lock_guard<std::mutex> lk(g_side_mu);
    if (SideStream* ss = side_stream()) {
      const tproj::SideRef side{ss->s, ss->fork, ss->join};
      LAUNCH(tproj::launch_bwd(k, geom->interp, pl.bw, workspace, Y, Wimg, rot, shifts, vol, wvol, st,
                               eb.a ? &eb : nullptr, ef.a ? &ef : nullptr, &side),
             "back-projection (bricks)");
      return TP_OK;
    }
  }
  LAUNCH(tproj::launch_bwd(k, geom->interp, pl.bw, workspace, Y, Wimg, rot, shifts, vol, wvol, st,
                           eb.a ? &eb : nullptr, ef.a ? &ef : nullptr),
         "back-projection (bricks)");
  return TP_OK;
}

// ---- the static work area of project_3d_to_2d_noalloc (declared above) ----
struct ScratchAddr {
  void* ptr = nullptr;
  bool tried = false;
  hipError_t err = hipSuccess;
};
ScratchAddr g_scratch[MAX_DEVICES];
std::mutex g_scratch_mu;

// Device address of the current device's scratch array.
tp_status scratch_address(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) {
    (void)hipGetLastError();
    return fail(TP_E_DEVICE, "no usable HIP device for the static scratch");
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  ScratchAddr& sa = g_scratch[dev];
  if (!sa.tried) {
    sa.tried = true;
    sa.err = hipGetSymbolAddress(&sa.ptr, HIP_SYMBOL(scratch));
    if (sa.err != hipSuccess || sa.ptr == nullptr) {
      (void)hipGetLastError();
      sa.ptr = nullptr;
      if (sa.err == hipSuccess) sa.err = hipErrorInvalidSymbol;
    }
  }
  if (!sa.ptr) return fail(TP_E_DEVICE, "address of the static scratch on device %d: %s", dev, hipGetErrorString(sa.err));
  *ptr = sa.ptr;
  return TP_OK;
}

}  // namespace

namespace tproj {
// Status helpers shared with the other entry-point files of the library.
tp_status api_fail(tp_status s, const char* msg) { return fail(s, "%s", msg); }
tp_status api_ok() { return ok(); }
}  // namespace tproj

extern "C" {

int tp_abi_version(void) { return TPROJ_ABI_VERSION; }

const char* tp_status_string(int s) {
  switch (s) {   // an int: a caller may pass any code
    case TP_OK: return "ok";
    case TP_E_NULL: return "required pointer is NULL";
    case TP_E_SHAPE: return "invalid shape";
    case TP_E_VALUE: return "invalid value";
    case TP_E_DEVICE: return "no usable HIP device";
    case TP_E_LAUNCH: return "kernel launch failed";
    case TP_E_WORKSPACE: return "workspace too small";
  }
  return "unknown status";
}

const char* tp_last_error_detail(void) { return g_detail.c_str(); }

tp_status tp_timing_enable(int on) {
  std::lock_guard<std::mutex> lk(g_kt_mu);
  g_kt_on = on != 0;
  return ok();
}

tp_status tp_timing_read(int kernel_class, double* total_ms, int64_t* launches) {
  if (!total_ms || !launches) return fail(TP_E_NULL, "total_ms and launches must not be NULL");
  if (kernel_class < 0 || kernel_class >= TP_KT_COUNT) return fail(TP_E_VALUE, "unknown kernel class %d", kernel_class);
  std::lock_guard<std::mutex> lk(g_kt_mu);
  double sum = 0.0;
  int64_t n = 0;
  tp_status st = TP_OK;
  std::vector<TimedLaunch> keep;
  for (const TimedLaunch& t : g_kt) {
    if (t.cls != kernel_class) {
      keep.push_back(t);
      continue;
    }
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(t.ev.b);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, t.ev.a, t.ev.b);
    if (e != hipSuccess && st == TP_OK) st = fail(TP_E_LAUNCH, "event timing failed: %s", hipGetErrorString(e));
    (void)hipEventDestroy(t.ev.a);
    (void)hipEventDestroy(t.ev.b);
    sum += ms;
    ++n;
  }
  g_kt.swap(keep);
  *total_ms = sum;
  *launches = n;
  return st == TP_OK ? ok() : st;
}

tp_status tp_validate(const tp_geom* geom) {
  TRY(check_geom(geom));
  return ok();
}

size_t tp_workspace_size(const tp_geom* geom, int op) {
  if (check_geom(geom) != TP_OK) return (size_t)-1;
  if (op < TP_OP_PROJECT || op > TP_OP_BACKPROJECT_2D_BACKWARD) return (size_t)-1;
  return workspace_need(geom, op);
}

}  // extern "C"

namespace {
// Workspace of the 2D -> 2D ops: the periodic extension of the complex source
// (Ec) and of the real one (Er), the per-image maxima (mx) and the partial
// sums of the accumulation, each 256-byte aligned and present only when the
// op uses it.
struct Ws2 {
  float2* ec = nullptr;
  float* er = nullptr;
  float* mx = nullptr;
  void* parts = nullptr;
  size_t bytes = 0;
};

Ws2 ws2_layout(const tp_geom* g, int op, void* base) {
  const tproj::KGeom k = kgeom(g);
  const size_t ne = (size_t)g->Bv * tproj::e2_size(g->D);
  const bool ec = op != TP_OP_BACKPROJECT_2D;
  const bool er = op == TP_OP_BACKPROJECT_2D_BACKWARD;
  const bool bp = op == TP_OP_PROJECT_2D_BACKWARD || op == TP_OP_BACKPROJECT_2D;
  // offsets first; pointers only into a real base (no arithmetic on NULL)
  size_t off = 0, o_ec = 0, o_er = 0, o_mx = 0, o_parts = 0;
  if (ec) { o_ec = off; off += align_up(ne * sizeof(float2)); }
  if (er) { o_er = off; off += align_up(ne * sizeof(float)); }
  if (bp) {
    o_mx = off;
    off += align_up((size_t)g->B * g->P * sizeof(float));
    o_parts = off;
    off += align_up(tproj::twod_bp_parts_bytes(k, op == TP_OP_BACKPROJECT_2D));
  }
  Ws2 w;
  w.bytes = off;
  if (base) {
    char* p = (char*)base;
    if (ec) w.ec = (float2*)(p + o_ec);
    if (er) w.er = (float*)(p + o_er);
    if (bp) {
      w.mx = (float*)(p + o_mx);
      w.parts = p + o_parts;
    }
  }
  return w;
}

size_t workspace_need(const tp_geom* geom, int op) {
  if (op >= TP_OP_PROJECT_2D) return ws2_layout(geom, op, nullptr).bytes;
  const size_t gather = gather_plan(geom).ws_bytes;
  if (op == TP_OP_PROJECT || op == TP_OP_BACKPROJECT_BACKWARD) return gather;
  // the back-projection's part, then the gradients' (they may run at once)
  if (op == TP_OP_PROJECT_BACKWARD) return align_up(bwd_plan(geom, false).ws_bytes) + gather;
  return bwd_plan(geom, true).ws_bytes;
}
}  // namespace

extern "C" {

tp_status project_3d_to_2d(const tp_geom* geom, const void* vol, const float* rot, const float* shifts, void* out,
                           void* workspace, size_t ws_bytes, void* stream) {
  TRY(check_geom(geom));
  TRY(check_shifts(geom, shifts));
  TRY(check_ptr(vol, "vol", 8));
  TRY(check_ptr(rot, "rot", 4));
  TRY(check_opt(shifts, "shifts", 4));
  TRY(check_ptr(out, "out", 8));
  TRY(check_opt(workspace, "workspace", 8));
  TRY(check_workspace(geom, TP_OP_PROJECT, workspace, ws_bytes));
  TRY(check_device());
  const tproj::KGeom k = kgeom(geom);
  hipStream_t st = (hipStream_t)stream;
  TRY(run_forward(geom, k, (const float2*)vol, rot, shifts, (float2*)out, workspace, ws_bytes, st));
  return ok();
}

tp_status project_3d_to_2d_noalloc(const tp_geom* geom, const void* vol, const float* rot, const float* shifts,
                                   void* out, void* stream) {
  TRY(check_geom(geom));
  TRY(check_shifts(geom, shifts));
  TRY(check_ptr(vol, "vol", 8));
  TRY(check_ptr(rot, "rot", 4));
  TRY(check_opt(shifts, "shifts", 4));
  TRY(check_ptr(out, "out", 8));
  const size_t need = workspace_need(geom, TP_OP_PROJECT);
  if (need > TP_NOALLOC_SCRATCH_BYTES)
    return fail(TP_E_WORKSPACE, "this geometry needs %zu bytes of scratch, more than the %zu bytes of the static "
                "array of project_3d_to_2d_noalloc (use project_3d_to_2d with a workspace)",
                need, (size_t)TP_NOALLOC_SCRATCH_BYTES);
  TRY(check_device());
  void* ws = nullptr;
  TRY(scratch_address(&ws));
  const tproj::KGeom k = kgeom(geom);
  hipStream_t st = (hipStream_t)stream;
  TRY(run_forward(geom, k, (const float2*)vol, rot, shifts, (float2*)out, ws, TP_NOALLOC_SCRATCH_BYTES, st,
                  /*may_alloc=*/false));
  return ok();
}

tp_status project_3d_to_2d_backward(const tp_geom* geom, const void* grad_out, const void* vol, const float* rot,
                                    const float* shifts, void* grad_vol, float* grad_rot, float* grad_shifts,
                                    void* workspace, size_t ws_bytes, void* stream) {
  TRY(check_geom(geom));
  TRY(check_shifts(geom, shifts));
  TRY(check_ptr(grad_out, "grad_out", 8));
  TRY(check_ptr(rot, "rot", 4));
  TRY(check_opt(shifts, "shifts", 4));
  TRY(check_opt(grad_vol, "grad_vol", 8));
  TRY(check_opt(grad_rot, "grad_rot", 4));
  TRY(check_opt(grad_shifts, "grad_shifts", 4));
  TRY(check_opt(workspace, "workspace", 8));
  if ((grad_rot || grad_shifts) && !vol) return fail(TP_E_NULL, "vol is NULL but rotation/shift grads are requested");
  TRY(check_opt(vol, "vol", 8));
  if (grad_shifts && !shifts) return fail(TP_E_NULL, "grad_shifts requested without shifts");
  TRY(check_workspace(geom, TP_OP_PROJECT_BACKWARD, workspace, ws_bytes));
  TRY(check_device());
  const tproj::KGeom k = kgeom(geom);
  hipStream_t st = (hipStream_t)stream;
  const bool grads = grad_rot || grad_shifts;
  if (grad_vol && grads && worth_splitting(geom, 20, st)) {
    // gradients on the side stream (workspace after the scatter's part),
    // the scatter on the caller's stream, then the caller's stream waits
    const size_t off = align_up(bwd_plan(geom, false).ws_bytes);
    void* ws2 = workspace ? (char*)workspace + off : nullptr;
    const size_t n2 = ws_bytes > off ? ws_bytes - off : 0;
    std::lock_guard<std::mutex> lk(g_side_mu);
    SideStream* ss = side_stream();
    if (ss) {
      // the scatter first (its kernels are queued ahead), the gradients from
      // the start of the call, so that they overlap the scatter's set-up and
      // band-maximum pass
      hipError_t e = hipEventRecord(ss->fork, st);
      if (e != hipSuccess) return fail(TP_E_LAUNCH, "stream fork failed: %s", hipGetErrorString(e));
      TRY(run_bwd(geom, k, (const float2*)grad_out, nullptr, rot, shifts, (float2*)grad_vol, nullptr, workspace,
                  ws_bytes, st));
      e = hipStreamWaitEvent(ss->s, ss->fork, 0);
      if (e != hipSuccess) return fail(TP_E_LAUNCH, "stream fork failed: %s", hipGetErrorString(e));
      const tp_status sg = run_grads(geom, k, (const float2*)vol, nullptr, (const float2*)grad_out, nullptr, rot,
                                     shifts, grad_rot, grad_shifts, ws2, n2, ss->s);
      e = hipEventRecord(ss->join, ss->s);
      if (e == hipSuccess) e = hipStreamWaitEvent(st, ss->join, 0);
      if (e != hipSuccess) return fail(TP_E_LAUNCH, "stream join failed: %s", hipGetErrorString(e));
      if (sg != TP_OK) return sg;
      return ok();
    }
  }
  // one after the other on the caller's stream (the band maxima on the side
  // stream when nothing else uses it)
  if (grad_vol)
    TRY(run_bwd(geom, k, (const float2*)grad_out, nullptr, rot, shifts, (float2*)grad_vol, nullptr, workspace,
                ws_bytes, st, !grads));
  if (grads)
    TRY(run_grads(geom, k, (const float2*)vol, nullptr, (const float2*)grad_out, nullptr, rot, shifts, grad_rot,
                  grad_shifts, workspace, ws_bytes, st));
  return ok();
}

tp_status backproject_2d_to_3d(const tp_geom* geom, const void* images, const float* weights, const float* rot,
                               const float* shifts, void* data_vol, float* weight_vol, void* workspace,
                               size_t ws_bytes, void* stream) {
  TRY(check_geom(geom));
  TRY(check_shifts(geom, shifts));
  TRY(check_ptr(images, "images", 8));
  TRY(check_ptr(rot, "rot", 4));
  TRY(check_opt(shifts, "shifts", 4));
  TRY(check_ptr(data_vol, "data_vol", 8));
  if ((weights == nullptr) != (weight_vol == nullptr))
    return fail(TP_E_NULL, "weights and weight_vol must both be given or both be NULL");
  TRY(check_opt(weights, "weights", 4));
  TRY(check_opt(weight_vol, "weight_vol", 4));
  TRY(check_opt(workspace, "workspace", 8));
  TRY(check_workspace(geom, TP_OP_BACKPROJECT, workspace, ws_bytes));
  TRY(check_device());
  const tproj::KGeom k = kgeom(geom);
  hipStream_t st = (hipStream_t)stream;
  TRY(run_bwd(geom, k, (const float2*)images, weights, rot, shifts, (float2*)data_vol, weight_vol, workspace,
              ws_bytes, st, true));
  return ok();
}

tp_status backproject_2d_to_3d_backward(const tp_geom* geom, const void* grad_data_vol,
                                        const float* grad_weight_vol, const void* images, const float* weights,
                                        const float* rot, const float* shifts, void* grad_images,
                                        float* grad_weights, float* grad_rot, float* grad_shifts, void* workspace,
                                        size_t ws_bytes, void* stream) {
  TRY(check_geom(geom));
  TRY(check_shifts(geom, shifts));
  TRY(check_ptr(grad_data_vol, "grad_data_vol", 8));
  TRY(check_ptr(rot, "rot", 4));
  TRY(check_opt(shifts, "shifts", 4));
  TRY(check_opt(grad_weight_vol, "grad_weight_vol", 4));
  TRY(check_opt(images, "images", 8));
  TRY(check_opt(weights, "weights", 4));
  TRY(check_opt(grad_images, "grad_images", 8));
  TRY(check_opt(grad_weights, "grad_weights", 4));
  TRY(check_opt(grad_rot, "grad_rot", 4));
  TRY(check_opt(grad_shifts, "grad_shifts", 4));
  TRY(check_opt(workspace, "workspace", 8));
  if ((grad_rot || grad_shifts) && !images) return fail(TP_E_NULL, "images is NULL but rotation/shift grads are requested");
  if (grad_rot && grad_weight_vol && !weights)
    return fail(TP_E_NULL, "weights is NULL but grad_weight_vol and grad_rot are given");
  if (grad_shifts && !shifts) return fail(TP_E_NULL, "grad_shifts requested without shifts");
  TRY(check_workspace(geom, TP_OP_BACKPROJECT_BACKWARD, workspace, ws_bytes));
  TRY(check_device());
  const tproj::KGeom k = kgeom(geom);
  hipStream_t st = (hipStream_t)stream;
  if (grad_images)
    TRY(run_forward(geom, k, (const float2*)grad_data_vol, rot, shifts, (float2*)grad_images, workspace, ws_bytes, st));
  if (grad_weights) {
    if (grad_weight_vol)
      TRY(run_forward_real(geom, k, grad_weight_vol, rot, grad_weights, workspace, ws_bytes, st));
    else
      LAUNCH(tproj::launch_zero(grad_weights, img_elems(geom), st), "zero grad_weights");
  }
  if (grad_rot || grad_shifts) {
    const bool wch = grad_weight_vol != nullptr && weights != nullptr;
    TRY(run_grads(geom, k, (const float2*)grad_data_vol, wch ? grad_weight_vol : nullptr, (const float2*)images,
                  wch ? weights : nullptr, rot, shifts, grad_rot, grad_shifts, workspace, ws_bytes, st));
  }
  return ok();
}

// ---------------------------------------------------------------------------
// 2D -> 2D
// ---------------------------------------------------------------------------
tp_status project_2d_to_2d(const tp_geom* geom, const void* src, const float* rot, const float* shifts, void* out,
                           void* workspace, size_t ws_bytes, void* stream) {
  TRY(check_geom(geom));
  TRY(check_shifts(geom, shifts));
  TRY(check_ptr(src, "src", 8));
  TRY(check_ptr(rot, "rot", 4));
  TRY(check_opt(shifts, "shifts", 4));
  TRY(check_ptr(out, "out", 8));
  TRY(check_opt(workspace, "workspace", 8));
  TRY(check_workspace(geom, TP_OP_PROJECT_2D, workspace, ws_bytes));
  TRY(check_device());
  const tproj::KGeom k = kgeom(geom);
  hipStream_t st = (hipStream_t)stream;
  const Ws2 w = ws2_layout(geom, TP_OP_PROJECT_2D, workspace);
  LAUNCH(tproj::launch2_expand_c(k, (const float2*)src, w.ec, st), "2D source extension");
  LAUNCH(tproj::launch2_gather_c(k, geom->interp, w.ec, rot, shifts, (float2*)out, st), "2D projection");
  return ok();
}

tp_status project_2d_to_2d_backward(const tp_geom* geom, const void* grad_out, const void* src, const float* rot,
                                    const float* shifts, void* grad_src, float* grad_rot, float* grad_shifts,
                                    void* workspace, size_t ws_bytes, void* stream) {
  TRY(check_geom(geom));
  TRY(check_shifts(geom, shifts));
  TRY(check_ptr(grad_out, "grad_out", 8));
  TRY(check_ptr(rot, "rot", 4));
  TRY(check_opt(shifts, "shifts", 4));
  TRY(check_opt(grad_src, "grad_src", 8));
  TRY(check_opt(grad_rot, "grad_rot", 4));
  TRY(check_opt(grad_shifts, "grad_shifts", 4));
  TRY(check_opt(workspace, "workspace", 8));
  if ((grad_rot || grad_shifts) && !src) return fail(TP_E_NULL, "src is NULL but rotation/shift grads are requested");
  TRY(check_opt(src, "src", 8));
  if (grad_shifts && !shifts) return fail(TP_E_NULL, "grad_shifts requested without shifts");
  TRY(check_workspace(geom, TP_OP_PROJECT_2D_BACKWARD, workspace, ws_bytes));
  TRY(check_device());
  const tproj::KGeom k = kgeom(geom);
  hipStream_t st = (hipStream_t)stream;
  const Ws2 w = ws2_layout(geom, TP_OP_PROJECT_2D_BACKWARD, workspace);
  if (grad_src)
    LAUNCH(tproj::launch2_bp(k, geom->interp, (const float2*)grad_out, nullptr, rot, shifts, w.mx, w.parts,
                             (float2*)grad_src, nullptr, st),
           "2D accumulation");
  if (grad_rot || grad_shifts) {
    if (grad_rot) LAUNCH(tproj::launch_zero(grad_rot, 4 * (int64_t)geom->Br * geom->P, st), "zero grad_rot");
    if (grad_shifts) LAUNCH(tproj::launch_zero(grad_shifts, 2 * (int64_t)geom->Bs * geom->P, st), "zero grad_shifts");
    LAUNCH(tproj::launch2_expand_c(k, (const float2*)src, w.ec, st), "2D source extension");
    LAUNCH(tproj::launch2_grad(k, geom->interp, w.ec, nullptr, (const float2*)grad_out, nullptr, rot, shifts, grad_rot,
                               grad_shifts, st),
           "2D rotation/shift grads");
  }
  return ok();
}

tp_status backproject_2d_to_2d(const tp_geom* geom, const void* images, const float* weights, const float* rot,
                               const float* shifts, void* data, float* weight_out, void* workspace,
                               size_t ws_bytes, void* stream) {
  TRY(check_geom(geom));
  TRY(check_shifts(geom, shifts));
  TRY(check_ptr(images, "images", 8));
  TRY(check_ptr(rot, "rot", 4));
  TRY(check_opt(shifts, "shifts", 4));
  TRY(check_opt(weights, "weights", 4));
  TRY(check_ptr(data, "data", 8));
  TRY(check_opt(weight_out, "weight_out", 4));
  TRY(check_opt(workspace, "workspace", 8));
  if ((weights == nullptr) != (weight_out == nullptr))
    return fail(TP_E_NULL, "weights and weight_out must both be given or both be NULL");
  TRY(check_workspace(geom, TP_OP_BACKPROJECT_2D, workspace, ws_bytes));
  TRY(check_device());
  const tproj::KGeom k = kgeom(geom);
  hipStream_t st = (hipStream_t)stream;
  const Ws2 w = ws2_layout(geom, TP_OP_BACKPROJECT_2D, workspace);
  LAUNCH(tproj::launch2_bp(k, geom->interp, (const float2*)images, weights, rot, shifts, w.mx, w.parts, (float2*)data,
                           weight_out, st),
         "2D accumulation");
  return ok();
}

tp_status backproject_2d_to_2d_backward(const tp_geom* geom, const void* grad_data, const float* grad_weight,
                                        const void* images, const float* weights, const float* rot,
                                        const float* shifts, void* grad_images, float* grad_weights,
                                        float* grad_rot, float* grad_shifts, void* workspace, size_t ws_bytes,
                                        void* stream) {
  TRY(check_geom(geom));
  TRY(check_shifts(geom, shifts));
  TRY(check_ptr(grad_data, "grad_data", 8));
  TRY(check_ptr(rot, "rot", 4));
  TRY(check_opt(shifts, "shifts", 4));
  TRY(check_opt(grad_weight, "grad_weight", 4));
  TRY(check_opt(images, "images", 8));
  TRY(check_opt(weights, "weights", 4));
  TRY(check_opt(grad_images, "grad_images", 8));
  TRY(check_opt(grad_weights, "grad_weights", 4));
  TRY(check_opt(grad_rot, "grad_rot", 4));
  TRY(check_opt(grad_shifts, "grad_shifts", 4));
  TRY(check_opt(workspace, "workspace", 8));
  if ((grad_rot || grad_shifts) && !images) return fail(TP_E_NULL, "images is NULL but rotation/shift grads are requested");
  if (grad_rot && grad_weight && !weights) return fail(TP_E_NULL, "weights is NULL but grad_weight and grad_rot are given");
  if (grad_shifts && !shifts) return fail(TP_E_NULL, "grad_shifts requested without shifts");
  TRY(check_workspace(geom, TP_OP_BACKPROJECT_2D_BACKWARD, workspace, ws_bytes));
  TRY(check_device());
  const tproj::KGeom k = kgeom(geom);
  hipStream_t st = (hipStream_t)stream;
  const Ws2 w = ws2_layout(geom, TP_OP_BACKPROJECT_2D_BACKWARD, workspace);
  LAUNCH(tproj::launch2_expand_c(k, (const float2*)grad_data, w.ec, st), "2D source extension");
  if (grad_weight) LAUNCH(tproj::launch2_expand_r(k, grad_weight, w.er, st), "2D weight extension");
  if (grad_images)
    LAUNCH(tproj::launch2_gather_c(k, geom->interp, w.ec, rot, shifts, (float2*)grad_images, st), "2D projection");
  if (grad_weights) {
    if (grad_weight) LAUNCH(tproj::launch2_gather_r(k, geom->interp, w.er, rot, grad_weights, st), "2D weight projection");
    else LAUNCH(tproj::launch_zero(grad_weights, img_elems(geom), st), "zero grad_weights");
  }
  if (grad_rot || grad_shifts) {
    if (grad_rot) LAUNCH(tproj::launch_zero(grad_rot, 4 * (int64_t)geom->Br * geom->P, st), "zero grad_rot");
    if (grad_shifts) LAUNCH(tproj::launch_zero(grad_shifts, 2 * (int64_t)geom->Bs * geom->P, st), "zero grad_shifts");
    const bool wch = grad_weight != nullptr && weights != nullptr;
    LAUNCH(tproj::launch2_grad(k, geom->interp, w.ec, wch ? w.er : nullptr, (const float2*)images,
                               wch ? weights : nullptr, rot, shifts, grad_rot, grad_shifts, st),
           "2D rotation/shift grads");
  }
  return ok();
}

}  // extern "C"
