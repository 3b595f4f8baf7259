// Microbenchmarks of the bandwidths the projection kernels' rooflines rest on
// (libtproj_probes.so; measurement only, not part of the projection library):
//   tpp_stream_read  HBM stream read (16-byte loads, grid-stride)
//   tpp_l2_gather    8-byte reads at hashed indices of a small, cache-resident
//                    buffer (the tap access pattern without LDS staging)
//   tpp_lds_taps     4x4x4 tap reads or 64-bit atomics per lane from a 16^3
//                    tile in LDS with padded strides (1, 17, 276 entries)
//                    under controlled bank keys, or in the bank-split layout
//                    with per-lane rotated tap order
//   tpp_lds_width    LDS read (4, 8, 16 bytes per lane) and integer atomic
//                    (4, 8 bytes) rates by width, conflict-free
//   tpp_valu         FP32 FMA issue rate (independent chains, no packed
//                    math), alone or beside bank-split 64-bit LDS atomics
//                    whose values come from the FMAs (the scatter's mix);
//                    the issue rates of integer add, bitwise select,
//                    compare-and-select and 64-bit add chains
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

// Bank-split layout of a 16^3 tile of 8-byte entries: entry (x, y, z) at
// (x & 3) + 16 (x >> 2) + 64 y + 4 (z & 3) + 1024 (z >> 2), dense (4096
// entries), so that its bank pair (address mod 16) is (x & 3) + 4 (z & 3).
__device__ __forceinline__ int split_x(int x) { return (x & 3) + ((x >> 2) << 4); }
__device__ __forceinline__ int split_z(int z) { return ((z & 3) << 2) + ((z >> 2) << 10); }

// mode 0: random bases; 1: random bases, lanes permuted by rank of the bank
// key (rank r to lane (r % 8) * 8 + r / 8); 2: every 16-lane group holds 16
// distinct keys; 3: random bases in the bank-split layout, each lane visiting
// its footprint's x and z taps in the rotated order that puts its accesses in
// bank pair (lane mod 16) + the step's offset.  ATOMIC: ds_add_u64 instead of
// reads.
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
    if constexpr (MODE == 3) {
      // slot (lane & 3, (lane >> 2) & 3): x taps from rotation t, z taps from r
      const int t = ((lane & 3) - x) & 3, r = (((lane >> 2) & 3) - z) & 3;
      int xo[4], zo[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        xo[j] = split_x(x + ((j + t) & 3));
        zo[j] = split_z(z + ((j + r) & 3)) + 64 * y;
      }
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          unsigned long long* col = tile + xo[a] + zo[c];
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            if constexpr (ATOMIC) atomicAdd(&col[64 * b], (unsigned long long)(it + 1));
            else acc += col[64 * b];
          }
        }
      continue;
    }
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


// FP32 FMA issue: 8 independent chains per thread, 8 FMAs per chain per
// iteration (64 per iteration), compiled without packed math so that every
// FMA is one v_fma_f32 / v_fmac_f32.
__global__ void __launch_bounds__(THREADS) k_valu_fma(int iters, float* __restrict__ sink) {
  const unsigned t = blockIdx.x * THREADS + threadIdx.x;
  float a[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) a[j] = (float)((t + j) & 7) * 0.125f;
  const float m = 0.999f, c = 1e-3f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
      for (int j = 0; j < 8; ++j) a[j] = fmaf(a[j], m, c);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += a[j];
  sink[t] = s;
}

// Issue rate of one non-FP32 VALU instruction kind: 8 independent chains per
// thread, 64 operations per iteration; an empty asm statement after each
// operation keeps every step in a register, so the chains are not folded.
// KIND 0: 32-bit integer add (v_add_u32); 1: bitwise select (v_and_b32 +
// v_and_or_b32, two instructions); 2: compare and select (v_cmp +
// v_cndmask_b32, two instructions); 3: 64-bit add (v_lshl_add_u64).
template <int KIND>
__global__ void __launch_bounds__(THREADS) k_valu_int(int iters, float* __restrict__ sink) {
  const unsigned t = blockIdx.x * THREADS + threadIdx.x;
  unsigned a[8];
  unsigned long long q[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = mix(t * 8u + (unsigned)j);
    q[j] = ((unsigned long long)a[j] << 32) | (unsigned long long)(t + j);
  }
  const unsigned m = mix(t) | 0x0f0f0f0fu, c = 0x5555u + (t & 15u);
  const unsigned long long c64 = 0x0000000100000003ull + (unsigned long long)(t & 7u);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if constexpr (KIND == 0) a[j] = a[j] + c;
        if constexpr (KIND == 1) a[j] = (a[j] & m) | (a[(j + 1) & 7] & ~m);
        if constexpr (KIND == 2) a[j] = (int)a[j] < (int)c ? a[(j + 3) & 7] : m;
        if constexpr (KIND == 3) q[j] = q[j] + c64;
        if constexpr (KIND == 3) asm volatile("" : "+v"(q[j]));
        else asm volatile("" : "+v"(a[j]));
      }
  }
  unsigned s = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += a[j] + (unsigned)(q[j] >> 11);
  sink[t] = (float)s;
}

// The scatter's tap mix: per 4x4x4 footprint in a bank-split 16^3 tile of
// 8-byte entries (random bases, rotated per-lane tap order, as mode 3 of
// k_lds_taps), each tap's word comes from two magic-number FMAs packed with
// one 64-bit subtraction, plus EXTRA further FMAs into independent
// accumulators; ATOMIC = false forms the same words and tap indices in
// registers and drops them (an empty asm statement consumes each pair).
template <int EXTRA, bool ATOMIC>
__global__ void __launch_bounds__(THREADS) k_tap_mix(int iters, float* __restrict__ sink) {
  __shared__ unsigned long long tile[4096];
  for (int i = threadIdx.x; i < 4096; i += THREADS) tile[i] = 0ull;
  __syncthreads();
  const int lane = threadIdx.x & 63;
  unsigned long long acc = 0ull;
  float e[4] = {0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
    const unsigned h = mix(blockIdx.x * 7919u + threadIdx.x * 131u + (unsigned)it * 977u);
    const int x = (int)(h % 13u), y = (int)((h >> 8) % 13u), z = (int)((h >> 16) % 13u);
    const float f = (float)(h & 1023u) * (1.0f / 1024.0f);
    float w[4], u[4], v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      w[j] = f + 0.25f * (float)j;
      u[j] = 3.0f - f * (float)j;
      v[j] = f * (float)j - 2.0f;
    }
    const int t = ((lane & 3) - x) & 3, r = (((lane >> 2) & 3) - z) & 3;
    int xo[4], zo[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      xo[j] = split_x(x + ((j + t) & 3));
      zo[j] = split_z(z + ((j + r) & 3)) + 64 * y;
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        unsigned long long* col = tile + xo[a] + zo[c];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const unsigned long long lo = __float_as_uint(fmaf(w[a], u[b], 12582912.0f));
          const unsigned long long hi = __float_as_uint(fmaf(w[c], v[b], 12582912.0f));
          const unsigned long long word = ((hi << 32) | lo) - 0x4B4000004B400000ull;
#pragma unroll
          for (int k = 0; k < EXTRA; ++k) e[k & 3] = fmaf(e[k & 3], w[b], u[a]);
          if constexpr (ATOMIC) atomicAdd(&col[64 * b], word);
          else asm volatile("" ::"v"(word), "v"(xo[a] + zo[c]));   // word and address formed, then dropped
        }
      }
  }
  if constexpr (ATOMIC) {
    __syncthreads();
    acc = tile[threadIdx.x];
  }
  sink[blockIdx.x * THREADS + threadIdx.x] = (float)acc + e[0] + e[1] + e[2] + e[3];
}

// LDS access width: each lane reads (or, ATOMIC, adds to) 16 consecutive-lane
// words of W bytes per iteration (lane l, word j at (l + 64 j + 1024 it) W,
// wrapped to a 32 KB tile): every access pattern is conflict-free, so the
// rate is the LDS's rate for that instruction width.
template <int W, bool ATOMIC>
__global__ void __launch_bounds__(THREADS) k_lds_width(int iters, float* __restrict__ sink) {
  constexpr int TB = 32768;
  __shared__ __align__(16) unsigned char tile[TB];
  for (int i = threadIdx.x; i < TB / 4; i += THREADS) reinterpret_cast<float*>(tile)[i] = (float)(i & 255);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  float acc = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int off = ((lane + 64 * j + 1024 * it) * W) & (TB - 1);
      if constexpr (ATOMIC && W == 4) {
        atomicAdd(reinterpret_cast<unsigned int*>(tile + off), 1u);
      } else if constexpr (ATOMIC) {
        atomicAdd(reinterpret_cast<unsigned long long*>(tile + off), 1ull);
      } else if constexpr (W == 4) {
        acc += *reinterpret_cast<const float*>(tile + off);
      } else if constexpr (W == 8) {
        const float2 v = *reinterpret_cast<const float2*>(tile + off);
        acc += v.x + v.y;
      } else {
        const float4 v = *reinterpret_cast<const float4*>(tile + off);
        acc += (v.x + v.y) + (v.z + v.w);
      }
    }
  }
  if constexpr (ATOMIC) {
    __syncthreads();
    acc = *reinterpret_cast<const float*>(tile + 4 * threadIdx.x);
  }
  sink[blockIdx.x * THREADS + threadIdx.x] = acc;
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
  if (!sink || mode < 0 || mode > 3 || iters < 1 || blocks < 1 || blocks > 65535) return -1;
  const hipStream_t st = (hipStream_t)stream;
#define TPP_LDS(M, A) hipLaunchKernelGGL((k_lds_taps<M, A>), dim3(blocks), dim3(THREADS), 0, st, iters, sink)
  if (atomic) {
    if (mode == 0) TPP_LDS(0, true);
    else if (mode == 1) TPP_LDS(1, true);
    else if (mode == 2) TPP_LDS(2, true);
    else TPP_LDS(3, true);
  } else {
    if (mode == 0) TPP_LDS(0, false);
    else if (mode == 1) TPP_LDS(1, false);
    else if (mode == 2) TPP_LDS(2, false);
    else TPP_LDS(3, false);
  }
#undef TPP_LDS
  return (int)hipGetLastError();
}

int tpp_lds_width(float* sink, int width, int atomic, int iters, int blocks, void* stream) {
  if (!sink || (width != 4 && width != 8 && width != 16) || (atomic && width == 16) || iters < 1 || blocks < 1 ||
      blocks > 65535)
    return -1;
  const hipStream_t st = (hipStream_t)stream;
  const dim3 g(blocks), b(THREADS);
  if (atomic) {
    if (width == 4) hipLaunchKernelGGL((k_lds_width<4, true>), g, b, 0, st, iters, sink);
    else hipLaunchKernelGGL((k_lds_width<8, true>), g, b, 0, st, iters, sink);
  } else {
    if (width == 4) hipLaunchKernelGGL((k_lds_width<4, false>), g, b, 0, st, iters, sink);
    else if (width == 8) hipLaunchKernelGGL((k_lds_width<8, false>), g, b, 0, st, iters, sink);
    else hipLaunchKernelGGL((k_lds_width<16, false>), g, b, 0, st, iters, sink);
  }
  return (int)hipGetLastError();
}

int tpp_valu(float* sink, int mode, int iters, int blocks, void* stream) {
  if (!sink || mode < 0 || mode > 10 || iters < 1 || blocks < 1 || blocks > 65535) return -1;
  const hipStream_t st = (hipStream_t)stream;
#define TPP_MIX(E, A) hipLaunchKernelGGL((k_tap_mix<E, A>), dim3(blocks), dim3(THREADS), 0, st, iters, sink)
  switch (mode) {
    case 0: hipLaunchKernelGGL(k_valu_fma, dim3(blocks), dim3(THREADS), 0, st, iters, sink); break;
    case 1: TPP_MIX(0, true); break;
    case 2: TPP_MIX(0, false); break;
    case 3: TPP_MIX(2, true); break;
    case 4: TPP_MIX(2, false); break;
    case 5: TPP_MIX(6, true); break;
    case 6: TPP_MIX(6, false); break;
    case 7: hipLaunchKernelGGL((k_valu_int<0>), dim3(blocks), dim3(THREADS), 0, st, iters, sink); break;
    case 8: hipLaunchKernelGGL((k_valu_int<1>), dim3(blocks), dim3(THREADS), 0, st, iters, sink); break;
    case 9: hipLaunchKernelGGL((k_valu_int<2>), dim3(blocks), dim3(THREADS), 0, st, iters, sink); break;
    default: hipLaunchKernelGGL((k_valu_int<3>), dim3(blocks), dim3(THREADS), 0, st, iters, sink); break;
  }
#undef TPP_MIX
  return (int)hipGetLastError();
}

}  // extern "C"
