// Microbenchmarks of the bandwidths the projection kernels' rooflines rest on
// (libtproj_probes.so; measurement only, not part of the projection library):
//   tpp_stream_read  HBM stream read (16-byte loads, grid-stride)
//   tpp_l2_gather    8-byte reads at hashed indices of a small, cache-resident
//                    buffer (the tap access pattern without LDS staging)
//   tpp_lds_taps     4x4x4 tap reads or 64-bit atomics per lane from a 16^3
//                    tile in LDS with the projection kernels' padded strides
//                    (1, 17, 276 entries), under controlled bank keys
// Each kernel folds what it reads into one float per thread (sink), so that
// nothing is optimised away.  Argument checks on the host; -1 on bad input,
// else the HIP status of the launch.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "tproj_probes.h"

namespace {

constexpr int THREADS = 256;
constexpr int TILE = 4416;   // 16 * 276 entries

__device__ __forceinline__ unsigned mix(unsigned x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return x;
}

__global__ void __launch_bounds__(THREADS) k_stream_read(const float4* __restrict__ src, size_t n4,
                                                         float* __restrict__ sink) {
  float acc = 0.f;
  const size_t stride = (size_t)gridDim.x * THREADS;
  for (size_t i = (size_t)blockIdx.x * THREADS + threadIdx.x; i < n4; i += stride) {
    const float4 v = src[i];
    acc += (v.x + v.y) + (v.z + v.w);
  }
  sink[(size_t)blockIdx.x * THREADS + threadIdx.x] = acc;
}

__global__ void __launch_bounds__(THREADS) k_l2_gather(const float2* __restrict__ buf, unsigned mask, int iters,
                                                       float* __restrict__ sink) {
  float acc = 0.f;
  const unsigned t = blockIdx.x * THREADS + threadIdx.x;
  for (int it = 0; it < iters; ++it) {
    // a random base per lane, then 16 consecutive-row taps (4 rows of 4)
    const unsigned base = mix(t * 7919u + (unsigned)it * 104729u) & mask;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const float2 v = buf[(base + (unsigned)(b * 128 + a)) & mask];
        acc += v.x + v.y;
      }
  }
  sink[t] = acc;
}

// x, y, z in [0, 13) with (x + 17 y + 276 z) & 15 == want
__device__ __forceinline__ void pick_key(unsigned h, int want, int& x, int& y, int& z) {
  z = (int)((h >> 16) % 13u);
  y = (int)((h >> 8) % 13u);
  int r = (want - y - 4 * z) & 15;
  if (r >= 13) {
    if (y + (r - 12) < 13) {
      y += r - 12;
      r = 12;
    } else {
      y -= 16 - r;
      r = 0;
    }
  }
  x = r;
}

// rank of this lane's key among the wavefront's keys (ties by lane)
__device__ __forceinline__ int key_rank(int key) {
  const int lane = threadIdx.x & 63;
  const unsigned long long below = (1ull << lane) - 1ull;
  unsigned long long less = 0ull, eq = ~0ull;
#pragma unroll
  for (int j = 3; j >= 0; --j) {
    const bool bit = (key >> j) & 1;
    const unsigned long long bj = __ballot(bit);
    if (bit) {
      less |= eq & ~bj;
      eq &= bj;
    } else {
      eq &= ~bj;
    }
  }
  return __popcll(less) + __popcll(eq & below);
}

// mode 0: random bases; 1: random bases, lanes permuted by rank of the bank
// key (rank r to lane (r % 8) * 8 + r / 8); 2: every 16-lane group holds 16
// distinct keys.  ATOMIC: ds_add_u64 instead of reads.
template <int MODE, bool ATOMIC>
__global__ void __launch_bounds__(THREADS) k_lds_taps(int iters, float* __restrict__ sink) {
  __shared__ unsigned long long tile[TILE];
  for (int i = threadIdx.x; i < TILE; i += THREADS) tile[i] = (unsigned long long)i;
  __syncthreads();
  const int lane = threadIdx.x & 63;
  unsigned long long acc = 0ull;
  for (int it = 0; it < iters; ++it) {
    const unsigned h = mix(blockIdx.x * 7919u + threadIdx.x * 131u + (unsigned)it * 977u);
    int x = (int)(h % 13u), y = (int)((h >> 8) % 13u), z = (int)((h >> 16) % 13u);
    if constexpr (MODE == 2) pick_key(h, lane & 15, x, y, z);
    if constexpr (MODE == 1) {
      const int r = key_rank((x + 17 * y + 276 * z) & 15);
      const int dest = (((r & 7) << 3) | (r >> 3)) << 2;
      x = __builtin_amdgcn_ds_permute(dest, x);
      y = __builtin_amdgcn_ds_permute(dest, y);
      z = __builtin_amdgcn_ds_permute(dest, z);
    }
    // x, y, z <= 12: the 4^3 footprint ends at 15 + 17 * 15 + 276 * 15 < TILE
    unsigned long long* base = tile + z * 276 + y * 17 + x;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          if constexpr (ATOMIC) atomicAdd(&base[c * 276 + b * 17 + a], (unsigned long long)(it + 1));
          else acc += base[c * 276 + b * 17 + a];
        }
  }
  if constexpr (ATOMIC) {
    __syncthreads();
    acc = tile[threadIdx.x];
  }
  sink[blockIdx.x * THREADS + threadIdx.x] = (float)acc;
}

}  // namespace

extern "C" {

int tpp_stream_read(const void* src, size_t bytes, float* sink, int blocks, void* stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 != 0 || blocks < 1 || blocks > 65535) return -1;
  hipLaunchKernelGGL(k_stream_read, dim3(blocks), dim3(THREADS), 0, (hipStream_t)stream, (const float4*)src,
                     bytes / 16, sink);
  return (int)hipGetLastError();
}

int tpp_l2_gather(const void* buf, int log2_entries, float* sink, int iters, int blocks, void* stream) {
  if (!buf || !sink || log2_entries < 10 || log2_entries > 26 || iters < 1 || blocks < 1 || blocks > 65535)
    return -1;
  hipLaunchKernelGGL(k_l2_gather, dim3(blocks), dim3(THREADS), 0, (hipStream_t)stream, (const float2*)buf,
                     (1u << log2_entries) - 1u, iters, sink);
  return (int)hipGetLastError();
}

int tpp_lds_taps(float* sink, int mode, int atomic, int iters, int blocks, void* stream) {
  if (!sink || mode < 0 || mode > 2 || iters < 1 || blocks < 1 || blocks > 65535) return -1;
  const hipStream_t st = (hipStream_t)stream;
#define TPP_LDS(M, A) hipLaunchKernelGGL((k_lds_taps<M, A>), dim3(blocks), dim3(THREADS), 0, st, iters, sink)
  if (atomic) {
    if (mode == 0) TPP_LDS(0, true);
    else if (mode == 1) TPP_LDS(1, true);
    else TPP_LDS(2, true);
  } else {
    if (mode == 0) TPP_LDS(0, false);
    else if (mode == 1) TPP_LDS(1, false);
    else TPP_LDS(2, false);
  }
#undef TPP_LDS
  return (int)hipGetLastError();
}

}  // extern "C"
