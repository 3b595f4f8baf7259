// Steps either side of the Fourier-slice path, for gfx950: the real-space
// front end of a volume (zero padding for oversampling, centre to index 0,
// 3D real-to-complex FFT), the back end of projections (2D complex-to-real
// FFT, index 0 back to the centre), the per-image weight (CTF) multiply, and
// the finishing division of an accumulated reconstruction by its weights.
//
// The pages use the PyTorch rfft layout for every Fourier array, name CTF
// correction as the use of the weight channel, and compare cubic
// interpolation against oversampling by zero padding (torch-projectors
// pages: Spanish "Resumen tecnico" 2 and 4, Dutch Methodologie and
// Resultaten, French "Resume technique" 2 and 4).  The FFTs themselves are
// library calls (hipFFT plans, cached per shape and device, with the work
// area taken from the caller's workspace); the element-wise steps are the
// kernels below.
#include <hip/hip_runtime.h>
#include <hipfft/hipfft.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <map>
#include <mutex>
#include <tuple>

#include "tproj.h"
#include "tproj_spectral.h"

namespace tproj {
tp_status api_fail(tp_status s, const char* msg);
tp_status api_ok();
}  // namespace tproj

namespace {

// ---------------------------------------------------------------------------
// kernels
// ---------------------------------------------------------------------------

// Padded, index-shifted copy of a real volume: dst is [Bv][N][N][N] with
//   dst[j] = src[(j + N/2) mod N - (N - D)/2]   per axis, 0 outside [0, D):
// the input centred in a box of N = pad * D (zero padding), then its centre
// N/2 moved to index 0.
__global__ void __launch_bounds__(256) k_pad_ifftshift(const float* __restrict__ src, float* __restrict__ dst, int D,
                                                       int N, int64_t total) {
  const int off = (N - D) / 2, h = N / 2;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int x = (int)(i % N);
    const int y = (int)((i / N) % N);
    const int z = (int)((i / ((int64_t)N * N)) % N);
    const int64_t b = i / ((int64_t)N * N * N);
    const int sx = (x + h) % N - off, sy = (y + h) % N - off, sz = (z + h) % N - off;
    float v = 0.f;
    if (sx >= 0 && sx < D && sy >= 0 && sy < D && sz >= 0 && sz < D)
      v = src[((b * D + sz) * D + sy) * (int64_t)D + sx];
    dst[i] = v;
  }
}

// Spectrum [n][H][H/2+1] times (-1)^(iy + ix) / H^2: after the unnormalised
// complex-to-real FFT this gives the normalised inverse with index 0 moved
// to the centre H/2 (a shift by H/2 in both axes is that sign pattern).
__global__ void __launch_bounds__(256) k_spectrum_centre(const float2* __restrict__ in, float2* __restrict__ out,
                                                         int H, float scale, int64_t total) {
  const int W = H / 2 + 1;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int ix = (int)(i % W);
    const int iy = (int)((i / W) % H);
    const float s = ((ix + iy) & 1) ? -scale : scale;
    const float2 v = in[i];
    out[i] = make_float2(s * v.x, s * v.y);
  }
}

// out[i] = images[i] * weights[i mod nw]
__global__ void __launch_bounds__(256) k_weight_images(const float2* __restrict__ img, const float* __restrict__ w,
                                                       float2* __restrict__ out, int64_t total, int64_t nw) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const float a = w[i % nw];
    const float2 v = img[i];
    out[i] = make_float2(a * v.x, a * v.y);
  }
}

// out[i] = data[i] / (weights[i] + lambda) where that is > 0, else 0.
__global__ void __launch_bounds__(256) k_finish(const float2* __restrict__ data, const float* __restrict__ w,
                                                float lambda, float2* __restrict__ out, int64_t total) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const float d = w[i] + lambda;
    const float2 v = data[i];
    out[i] = d > 0.f ? make_float2(v.x / d, v.y / d) : make_float2(0.f, 0.f);
  }
}

unsigned grid_for(int64_t n) {
  const int64_t b = (n + 255) / 256;
  return (unsigned)(b < 1 ? 1 : (b > 65536 ? 65536 : b));
}

size_t align256(size_t n) { return (n + 255) / 256 * 256; }

// ---------------------------------------------------------------------------
// FFT plans: one per (kind, size, batch, device), created on first use with
// automatic work-area allocation off.  Creating a plan is the one place where
// device memory is allocated on the library's behalf (hipFFT keeps its
// tables there), so a first call for a new shape should not happen under
// graph capture; executing one uses the caller's workspace.  The mutex keeps
// the set-stream / set-work-area / exec triple of one call together.  At most
// MAX_PLANS plans are kept: a new one beyond that replaces the least recently
// used, whose device is first synchronised so that no queued transform still
// reads its tables.
// ---------------------------------------------------------------------------
struct Plan {
  hipfftHandle h = nullptr;
  size_t work = 0;
  uint64_t last_use = 0;
};
constexpr size_t MAX_PLANS = 16;
std::mutex g_plan_mu;
std::map<std::tuple<int, int, int64_t, int>, Plan> g_plans;
uint64_t g_plan_clock = 0;

// Drops the least recently used plan.  Caller holds g_plan_mu.
void evict_plan() {
  auto lru = g_plans.begin();
  for (auto it = g_plans.begin(); it != g_plans.end(); ++it)
    if (it->second.last_use < lru->second.last_use) lru = it;
  const int pdev = std::get<3>(lru->first);
  int cur = -1;
  (void)hipGetDevice(&cur);
  if (pdev != cur) (void)hipSetDevice(pdev);
  (void)hipDeviceSynchronize();
  hipfftDestroy(lru->second.h);
  if (pdev != cur && cur >= 0) (void)hipSetDevice(cur);
  (void)hipGetLastError();
  g_plans.erase(lru);
}

enum { KIND_R2C_3D = 0, KIND_C2R_2D = 1 };

// Returns nullptr (and sets *err) on failure.  Caller holds g_plan_mu.
Plan* get_plan(int kind, int n, int64_t batch, const char** err) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    *err = "no usable HIP device";
    return nullptr;
  }
  const auto key = std::make_tuple(kind, n, batch, dev);
  auto it = g_plans.find(key);
  if (it != g_plans.end()) {
    it->second.last_use = ++g_plan_clock;
    return &it->second;
  }
  if (batch > 0x7fffffff) {
    *err = "FFT batch too large";
    return nullptr;
  }
  Plan p;
  if (hipfftCreate(&p.h) != HIPFFT_SUCCESS) {
    *err = "hipfftCreate failed";
    return nullptr;
  }
  hipfftResult r = hipfftSetAutoAllocation(p.h, 0);
  if (r == HIPFFT_SUCCESS) {
    if (kind == KIND_R2C_3D) {
      int dims[3] = {n, n, n};
      r = hipfftMakePlanMany(p.h, 3, dims, nullptr, 1, 0, nullptr, 1, 0, HIPFFT_R2C, (int)batch, &p.work);
    } else {
      int dims[2] = {n, n};
      r = hipfftMakePlanMany(p.h, 2, dims, nullptr, 1, 0, nullptr, 1, 0, HIPFFT_C2R, (int)batch, &p.work);
    }
  }
  if (r != HIPFFT_SUCCESS) {
    hipfftDestroy(p.h);
    *err = "hipFFT plan creation failed";
    return nullptr;
  }
  while (g_plans.size() >= MAX_PLANS) evict_plan();
  p.last_use = ++g_plan_clock;
  return &(g_plans[key] = p);
}

tp_status fail(tp_status s, const char* fmt, ...) {
  char buf[256];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  return tproj::api_fail(s, buf);
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

tp_status check_volume_args(int D, int pad, int Bv) {
  if (D < 2 || D % 2 != 0 || D > 1024) return fail(TP_E_SHAPE, "D must be even, 2 <= D <= 1024 (got %d)", D);
  if (pad < 1 || (int64_t)pad * D > 1024) return fail(TP_E_SHAPE, "pad must be >= 1 with pad * D <= 1024 (got %d)", pad);
  if (Bv < 1) return fail(TP_E_SHAPE, "Bv must be >= 1 (got %d)", Bv);
  return TP_OK;
}

tp_status check_images_args(int H, int64_t n) {
  if (H < 2 || H % 2 != 0 || H > 4096) return fail(TP_E_SHAPE, "H must be even, 2 <= H <= 4096 (got %d)", H);
  if (n < 0 || n > 0x7fffffff) return fail(TP_E_SHAPE, "image count out of range (got %lld)", (long long)n);
  return TP_OK;
}

}  // namespace

extern "C" {

size_t tp_volume_rfft_workspace(int D, int pad, int Bv) {
  if (check_volume_args(D, pad, Bv) != TP_OK) return (size_t)-1;
  const int N = pad * D;
  std::lock_guard<std::mutex> lk(g_plan_mu);
  const char* err = nullptr;
  Plan* p = get_plan(KIND_R2C_3D, N, Bv, &err);
  if (!p) {
    fail(TP_E_DEVICE, "%s", err);
    return (size_t)-1;
  }
  return align256((size_t)Bv * N * N * N * sizeof(float)) + p->work;
}

tp_status tp_volume_rfft(int D, int pad, int Bv, const float* vol, void* out, void* workspace, size_t ws_bytes,
                         void* stream) {
  tp_status s = check_volume_args(D, pad, Bv);
  if (s != TP_OK) return s;
  if (!vol || !out || !workspace) return fail(TP_E_NULL, "vol, out and workspace are required");
  if (!aligned(vol, 4) || !aligned(out, 8) || !aligned(workspace, 256))
    return fail(TP_E_VALUE, "misaligned pointer (vol 4 B, out 8 B, workspace 256 B)");
  const int N = pad * D;
  const size_t real_bytes = align256((size_t)Bv * N * N * N * sizeof(float));
  hipStream_t st = (hipStream_t)stream;
  std::lock_guard<std::mutex> lk(g_plan_mu);
  const char* err = nullptr;
  Plan* p = get_plan(KIND_R2C_3D, N, Bv, &err);
  if (!p) return fail(TP_E_DEVICE, "%s", err);
  if (ws_bytes < real_bytes + p->work)
    return fail(TP_E_WORKSPACE, "workspace %zu B < %zu B", ws_bytes, real_bytes + p->work);
  float* padded = (float*)workspace;
  void* fftwork = (char*)workspace + real_bytes;
  const int64_t total = (int64_t)Bv * N * N * N;
  hipLaunchKernelGGL(k_pad_ifftshift, dim3(grid_for(total)), dim3(256), 0, st, vol, padded, D, N, total);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TP_E_LAUNCH, "pad/shift kernel: %s", hipGetErrorString(e));
  if (hipfftSetStream(p->h, st) != HIPFFT_SUCCESS || (p->work && hipfftSetWorkArea(p->h, fftwork) != HIPFFT_SUCCESS))
    return fail(TP_E_LAUNCH, "hipFFT stream / work area set-up failed");
  if (hipfftExecR2C(p->h, (hipfftReal*)padded, (hipfftComplex*)out) != HIPFFT_SUCCESS)
    return fail(TP_E_LAUNCH, "hipfftExecR2C failed");
  return tproj::api_ok();
}

size_t tp_images_irfft_workspace(int H, int64_t n) {
  if (check_images_args(H, n) != TP_OK) return (size_t)-1;
  if (n == 0) return 0;
  std::lock_guard<std::mutex> lk(g_plan_mu);
  const char* err = nullptr;
  Plan* p = get_plan(KIND_C2R_2D, H, n, &err);
  if (!p) {
    fail(TP_E_DEVICE, "%s", err);
    return (size_t)-1;
  }
  return align256((size_t)n * H * (H / 2 + 1) * sizeof(float2)) + p->work;
}

tp_status tp_images_irfft(int H, int64_t n, const void* images, float* out, void* workspace, size_t ws_bytes,
                          void* stream) {
  tp_status s = check_images_args(H, n);
  if (s != TP_OK) return s;
  if (n == 0) return tproj::api_ok();
  if (!images || !out || !workspace) return fail(TP_E_NULL, "images, out and workspace are required");
  if (!aligned(images, 8) || !aligned(out, 4) || !aligned(workspace, 256))
    return fail(TP_E_VALUE, "misaligned pointer (images 8 B, out 4 B, workspace 256 B)");
  const size_t spec_bytes = align256((size_t)n * H * (H / 2 + 1) * sizeof(float2));
  hipStream_t st = (hipStream_t)stream;
  std::lock_guard<std::mutex> lk(g_plan_mu);
  const char* err = nullptr;
  Plan* p = get_plan(KIND_C2R_2D, H, n, &err);
  if (!p) return fail(TP_E_DEVICE, "%s", err);
  if (ws_bytes < spec_bytes + p->work)
    return fail(TP_E_WORKSPACE, "workspace %zu B < %zu B", ws_bytes, spec_bytes + p->work);
  float2* spec = (float2*)workspace;
  void* fftwork = (char*)workspace + spec_bytes;
  const int64_t total = n * H * (int64_t)(H / 2 + 1);
  hipLaunchKernelGGL(k_spectrum_centre, dim3(grid_for(total)), dim3(256), 0, st, (const float2*)images, spec, H,
                     1.0f / ((float)H * (float)H), total);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TP_E_LAUNCH, "spectrum kernel: %s", hipGetErrorString(e));
  if (hipfftSetStream(p->h, st) != HIPFFT_SUCCESS || (p->work && hipfftSetWorkArea(p->h, fftwork) != HIPFFT_SUCCESS))
    return fail(TP_E_LAUNCH, "hipFFT stream / work area set-up failed");
  if (hipfftExecC2R(p->h, (hipfftComplex*)spec, (hipfftReal*)out) != HIPFFT_SUCCESS)
    return fail(TP_E_LAUNCH, "hipfftExecC2R failed");
  return tproj::api_ok();
}

tp_status tp_weight_images(int64_t n, int64_t nw, const void* images, const float* weights, void* out, void* stream) {
  if (n < 0 || nw < 1 || (n > 0 && n % nw != 0))
    return fail(TP_E_SHAPE, "need n >= 0, nw >= 1 and nw dividing n (n %lld, nw %lld)", (long long)n, (long long)nw);
  if (n == 0) return tproj::api_ok();
  if (!images || !weights || !out) return fail(TP_E_NULL, "images, weights and out are required");
  if (!aligned(images, 8) || !aligned(out, 8) || !aligned(weights, 4)) return fail(TP_E_VALUE, "misaligned pointer");
  hipLaunchKernelGGL(k_weight_images, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream, (const float2*)images,
                     weights, (float2*)out, n, nw);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TP_E_LAUNCH, "weight kernel: %s", hipGetErrorString(e));
  return tproj::api_ok();
}

tp_status tp_finish_reconstruction(int64_t n, const void* data, const float* weights, float lambda, void* out,
                                   void* stream) {
  if (n < 0) return fail(TP_E_SHAPE, "n must be >= 0");
  if (!(lambda >= 0.f) || lambda == __builtin_huge_valf()) return fail(TP_E_VALUE, "lambda must be finite and >= 0");
  if (n == 0) return tproj::api_ok();
  if (!data || !weights || !out) return fail(TP_E_NULL, "data, weights and out are required");
  if (!aligned(data, 8) || !aligned(out, 8) || !aligned(weights, 4)) return fail(TP_E_VALUE, "misaligned pointer");
  hipLaunchKernelGGL(k_finish, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream, (const float2*)data, weights,
                     lambda, (float2*)out, n);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TP_E_LAUNCH, "finishing kernel: %s", hipGetErrorString(e));
  return tproj::api_ok();
}

}  // extern "C"
