/*
 * tproj_probes.h -- C ABI of libtproj_probes.so: microbenchmarks of the
 * bandwidths behind the projection kernels' rooflines on gfx950 (HBM stream
 * read, cache-resident 8-byte gathers, LDS tap reads and 64-bit atomics,
 * FP32 FMA issue alone and beside LDS atomics, integer VALU issue).
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
 * to lane (r % 8) * 8 + r / 8); 2: footprints chosen so that every group of
 * 16 consecutive lanes holds 16 distinct keys (the conflict-free case);
 * 3: random footprints in the bank-split layout (entry (x, y, z) at
 * (x & 3) + 16 (x >> 2) + 64 y + 4 (z & 3) + 1024 (z >> 2)), each lane
 * visiting its x and z taps in the rotated order that gives lane l the bank
 * pair (l mod 16) plus the step's common offset.                          */
int tpp_lds_taps(float* sink, int mode, int atomic, int iters, int blocks, void* stream);

/* LDS rate by access width: each of blocks * 256 threads, `iters` times,
 * reads 16 words of `width` bytes (4, 8 or 16) from a 32 KB tile, or with
 * atomic != 0 adds 1 to them with integer atomics (width 4 or 8), the lanes
 * of a wavefront at consecutive words (conflict-free).                     */
int tpp_lds_width(float* sink, int width, int atomic, int iters, int blocks, void* stream);

/* FP32 VALU issue, alone or beside LDS atomics.
 * mode 0: each of blocks * 256 threads runs 8 independent FMA chains, 64
 *         FMAs per iteration (128 flop), `iters` iterations.
 * modes 1-6: each thread, `iters` times, takes a random 4x4x4 footprint in
 *         a bank-split 16^3 tile of 8-byte entries (as tpp_lds_taps mode 3)
 *         and for each of its 64 taps forms a 64-bit word from two FMAs and
 *         one 64-bit subtraction, plus E further FMAs (E = 0 for modes 1-2,
 *         2 for 3-4, 6 for 5-6); odd modes add the words to the tile with
 *         64-bit LDS atomics, even modes form the words and tap indices and
 *         drop them (no LDS access).
 * modes 7-10: each thread runs 8 independent chains of one non-FP32 VALU
 *         operation, 64 per iteration: 7 a 32-bit integer add (one
 *         v_add_u32), 8 a bitwise select (v_and_b32 + v_and_or_b32), 9 a
 *         compare and select (v_cmp + v_cndmask_b32), 10 a 64-bit add (one
 *         v_lshl_add_u64).                                               */
int tpp_valu(float* sink, int mode, int iters, int blocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TPROJ_PROBES_H */
