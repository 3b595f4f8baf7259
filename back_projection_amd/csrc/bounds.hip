// The fixed-point bounds of the back-projection kernels (fixed_point_bound.h)
// exported for checking: host evaluations of the same source, and a kernel
// that evaluates them on the GPU.
#include <hip/hip_runtime.h>

#include <cmath>

#include "fixed_point_bound.h"
#include "tproj.h"
#include "tproj_bounds.h"

namespace tproj {
tp_status api_fail(tp_status s, const char* msg);
tp_status api_ok();
}  // namespace tproj

namespace {

template <int NT>
__device__ float bound_of(int kind, float o, float kmax, int D, const float* R) {
  if (kind == 0) return tproj::weight_sum_bound3<NT>(o, R);
  if (kind == 1) return tproj::contrib_bound3<NT>(o, R);
  return tproj::weight_sum_bound_2d<NT>(o, kmax, D, R);
}

__global__ void __launch_bounds__(256) k_bounds(int kind, int interp, float o, float kmax, int D,
                                                const float* __restrict__ rot, int64_t n, float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int stride = kind == 2 ? 4 : 9;
  float R[9];
  for (int a = 0; a < stride; ++a) R[a] = rot[i * stride + a];
  out[i] = interp == 1 ? bound_of<4>(kind, o, kmax, D, R) : bound_of<2>(kind, o, kmax, D, R);
}

struct DevBuf {
  void* p = nullptr;
  ~DevBuf() {
    if (p) (void)hipFree(p);
  }
};

}  // namespace

extern "C" {

float tp_weight_sum_bound_3d(int interp, float oversampling, const float* rot) {
  if (!rot) return NAN;
  return interp == 1 ? tproj::weight_sum_bound3<4>(oversampling, rot) : tproj::weight_sum_bound3<2>(oversampling, rot);
}

float tp_contrib_bound_3d(int interp, float oversampling, const float* rot) {
  if (!rot) return NAN;
  return interp == 1 ? tproj::contrib_bound3<4>(oversampling, rot) : tproj::contrib_bound3<2>(oversampling, rot);
}

float tp_weight_sum_bound_2d(int interp, float oversampling, float kmax, int D, const float* rot) {
  if (!rot || D <= 0) return NAN;
  return interp == 1 ? tproj::weight_sum_bound_2d<4>(oversampling, kmax, D, rot)
                     : tproj::weight_sum_bound_2d<2>(oversampling, kmax, D, rot);
}

tp_status tp_bounds_device(int kind, int interp, float oversampling, float kmax, int D, const float* rot, int64_t n,
                           float* out) {
  if (kind < 0 || kind > 2 || (interp != 0 && interp != 1) || n < 0 || n > ((int64_t)1 << 24) ||
      (kind == 2 && D <= 0))
    return tproj::api_fail(TP_E_VALUE, "tp_bounds_device: kind must be 0-2, interp 0 or 1, 0 <= n <= 2^24 (and D > 0 "
                                       "for kind 2)");
  if (n == 0) return tproj::api_ok();
  if (!rot || !out) return tproj::api_fail(TP_E_NULL, "tp_bounds_device: rot and out are required");
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
    (void)hipGetLastError();
    return tproj::api_fail(TP_E_DEVICE, "tp_bounds_device: no usable HIP device");
  }
  const size_t rb = (size_t)n * (kind == 2 ? 4 : 9) * sizeof(float), ob = (size_t)n * sizeof(float);
  DevBuf dr, dout;
  if (hipMalloc(&dr.p, rb) != hipSuccess || hipMalloc(&dout.p, ob) != hipSuccess ||
      hipMemcpy(dr.p, rot, rb, hipMemcpyHostToDevice) != hipSuccess) {
    (void)hipGetLastError();
    return tproj::api_fail(TP_E_LAUNCH, "tp_bounds_device: allocation or copy failed");
  }
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(k_bounds, dim3((unsigned)blocks), dim3(256), 0, nullptr, kind, interp, oversampling, kmax, D,
                     (const float*)dr.p, n, (float*)dout.p);
  if (hipGetLastError() != hipSuccess || hipMemcpy(out, dout.p, ob, hipMemcpyDeviceToHost) != hipSuccess) {
    (void)hipGetLastError();
    return tproj::api_fail(TP_E_LAUNCH, "tp_bounds_device: launch or copy back failed");
  }
  return tproj::api_ok();
}

}  // extern "C"
