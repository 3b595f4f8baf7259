/*
 * tproj_probes.h -- C ABI of libtproj_probes.so: microbenchmarks of the
 * bandwidths behind the projection kernels' rooflines on gfx950 (HBM stream
 * read, cache-resident 8-byte gathers, LDS tap reads and 64-bit atomics).
 * Measurement only; the projection library does not use them.
 *
 * Every function launches one kernel on `stream` (a hipStream_t, NULL = the
 * default stream) and returns without waiting: -1 for invalid arguments
 * (nothing is launched), otherwise the hipError_t of the launch (0 = ok).
 * `sink` is a caller-allocated device array of blocks * 256 floats that the
 * kernel writes (one value per thread, so that its reads are not optimised
 * away).  Timing is the caller's (events around the call).
 */
#ifndef TPROJ_PROBES_H
#define TPROJ_PROBES_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` (a multiple of 16) from device buffer src with 16-byte loads,
 * grid-stride over `blocks` workgroups of 256 threads (1..65535).          */
int tpp_stream_read(const void* src, size_t bytes, float* sink, int blocks, void* stream);

/* Each of blocks * 256 threads, `iters` times, picks a hashed base index in
 * buf (2^log2_entries complex64 entries, log2_entries in 10..26; buf must
 * hold them) and reads 16 entries at base + 128 b + a (a, b < 4), indices
 * wrapped to the buffer: 128 B of taps per lane per iteration.            */
int tpp_l2_gather(const void* buf, int log2_entries, float* sink, int iters, int blocks, void* stream);

/* Each of blocks * 256 threads, `iters` times, picks a 4x4x4 footprint in a
 * 16^3 tile of 8-byte entries in LDS (strides 1, 17, 276) and reads its 64
 * entries (atomic = 0) or adds to them with 64-bit atomics (atomic = 1).
 * mode 0: random footprints; 1: random footprints with the lanes of each
 * wavefront permuted by the bank key of the footprint's first entry (rank r
 * to lane (r % 8) * 8 + r / 8, as the projection kernels do); 2: footprints
 * chosen so that every group of 16 consecutive lanes holds 16 distinct keys
 * (the conflict-free case).                                               */
int tpp_lds_taps(float* sink, int mode, int atomic, int iters, int blocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TPROJ_PROBES_H */
