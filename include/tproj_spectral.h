/* Steps either side of the Fourier-slice path (libtproj.so).
 *
 * The torch-projectors pages keep every Fourier array in the PyTorch rfft
 * layout (Spanish "Resumen tecnico" 2, French "Resume technique" 2), name CTF
 * correction as the use of the weight channel (French page 2), and set
 * cubic interpolation against oversampling by real-space zero padding, done
 * offline or on the fly with extra FFTs (Spanish page 4, Dutch Resultaten,
 * French page 4).  These entry points are the real-space front end of a
 * volume, the real-space back end of projections, the per-image weight
 * multiply and the finishing division of a reconstruction.
 *
 * Conventions are those of tproj.h: device pointers, stream-ordered work on
 * `stream` (a hipStream_t; NULL = the default stream), arguments checked
 * before anything is enqueued, tp_status results with tp_last_error_detail().
 * The FFTs are hipFFT plans cached per (kind, size, batch, device): creating
 * one (the first workspace query or call for a shape) allocates hipFFT's own
 * device tables, so that first use belongs outside graph capture; every call
 * takes its scratch from the caller's workspace.  Calls that share a plan
 * are serialised by a lock while they enqueue.  At most 16 plans are kept;
 * creating one more first waits for the device of the least recently used
 * plan to go idle and destroys that plan (callers that cycle through many
 * image counts pay this wait: a fixed batch size avoids it).
 */
#ifndef TPROJ_SPECTRAL_H
#define TPROJ_SPECTRAL_H

#include <stddef.h>
#include <stdint.h>

#include "tproj.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Volume front end.  vol [Bv][D][D][D] float32 (z, y, x), centre at index
 * D/2.  Per axis the volume is placed centred in a box of N = pad * D
 * (zeros around it: index i goes to i + (N - D)/2), index N/2 is moved to 0
 * (ifftshift), and the 3D real-to-complex DFT (unnormalised, forward sign)
 * is written to out [Bv][N][N][N/2+1] complex64, the layout the projection
 * entry points read (project with oversampling = pad for the same image
 * frequencies).  D even, pad >= 1, N <= 1024.  workspace: at least
 * tp_volume_rfft_workspace(D, pad, Bv) bytes, 256-byte aligned (the padded
 * real copy, then the FFT work area).  The input is not modified.          */
size_t tp_volume_rfft_workspace(int D, int pad, int Bv);
tp_status tp_volume_rfft(int D, int pad, int Bv, const float* vol, void* out, void* workspace, size_t ws_bytes,
                         void* stream);

/* Image back end.  images [n][H][H/2+1] complex64 (rfft2 layout, Hermitian
 * in the self-conjugate entries) -> out [n][H][H] float32: the normalised
 * inverse 2D DFT (1/H^2), index 0 moved to the centre H/2 (fftshift).
 * workspace: tp_images_irfft_workspace(H, n) bytes, 256-byte aligned (a
 * sign-modulated copy of the spectra, so the input is not modified, then the
 * FFT work area).  H even, n >= 0.                                         */
size_t tp_images_irfft_workspace(int H, int64_t n);
tp_status tp_images_irfft(int H, int64_t n, const void* images, float* out, void* workspace, size_t ws_bytes,
                          void* stream);

/* Weight (CTF) multiply: out[i] = images[i] * weights[i mod nw] for the n
 * complex64 entries of images (out may equal images); weights float32 of nw
 * entries, nw dividing n (a [P][H][H/2+1] set of per-image weights applied
 * to a [B][P][H][H/2+1] stack has nw = P * H * (H/2+1)).                   */
tp_status tp_weight_images(int64_t n, int64_t nw, const void* images, const float* weights, void* out, void* stream);

/* Reconstruction finishing: out[i] = data[i] / (weights[i] + lambda) where
 * weights[i] + lambda > 0, else 0; data, out complex64 and weights float32
 * of n entries each (a back-projected data volume and its weight volume);
 * lambda finite and >= 0 (a constant regulariser; 0 = plain division).
 * out may equal data.                                                      */
tp_status tp_finish_reconstruction(int64_t n, const void* data, const float* weights, float lambda, void* out,
                                   void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TPROJ_SPECTRAL_H */
