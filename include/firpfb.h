/*
 * firpfb.h -- polyphase filter-bank channelizer on AMD Instinct MI355X
 * (gfx950), built on the overlap-save library's FFT.
 *
 * The method is the one of the channelizer page ("GPU polyphase filter bank
 * channelizer"), sections 2.1 and 2.2: the wide-band input is split into K
 * sub-bands, each shifted down to baseband, low-pass filtered by a real
 * prototype h of Nh taps and decimated by D.  Section 2.2's design has 50 %
 * overlapping channels, D = K / 2; D = K is the critically sampled bank.
 * For channel c in [0, K) and output m of the stream,
 *     y_c(m) = sum_{p<Nh} h(p) xt(t_m - p) exp(-2 pi j c (t_m - p) / K),
 * where t_m = (m + 1) D - 1 is the stream time of the last sample of output
 * m's hop of D samples and xt is the stream (zeros before its first
 * sample, or a state the caller sets).  The library computes it the way
 * section 2.1 describes: K branch filters h_k(n) = h(n K + k) on the
 * decimated branches, a K-point FFT across the branches, and the baseband
 * phase.
 *
 * Data types.  Samples are complex64 (interleaved float32 re, im); taps are
 * float32.  Status codes are the FIR_OLS_* values of firols.h.  Streams
 * are hipStream_t values passed as void* (NULL: the null stream).  A plan
 * lives on the device that was current when it was created; every later
 * call must be made with that device current.  A plan carries one stream
 * (its state and stream time), so its calls must be ordered.
 */
#ifndef FIRPFB_H
#define FIRPFB_H

#include <stdint.h>

#include "firols.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct fir_pfb_plan_s *fir_pfb_plan_t;   /* opaque, library-owned */

/*
 * Create a channelizer for K channels, decimation D and Nh prototype taps.
 *   K   power of two, 64 <= K <= 1024.
 *   D   divides K (D = K / 2: section 2.2's 50 % overlap; D = K: critical).
 *   Nh  1 <= Nh <= 8 K.
 * FIR_OLS_ERR_UNSUPPORTED when the workgroup's input span (Nh rounded up
 * to 2, 4 or 8 taps per branch, times K, plus the hops of the transforms
 * one workgroup runs at once) does not fit its LDS.  Allocates the taps,
 * the FFT and phase tables and two state buffers of Nh - 1 samples; the
 * state starts at zero and the stream time at 0.  Synchronous.
 */
int fir_pfb_plan(fir_pfb_plan_t *out, int64_t K, int64_t D, int64_t Nh);

/*
 * Set the prototype low-pass filter (section 2.2: designed by the window
 * method; any real taps are accepted).
 *   h_host  host array of Nh float32 taps, copied before return.
 *   Nh      must equal the plan's Nh.
 * Returns after the taps are in place.  Leaves the state unchanged.
 */
int fir_pfb_set_taps(fir_pfb_plan_t p, const float *h_host, int64_t Nh, void *stream);

/*
 * Channelize one call's input.
 *   x_dev     device complex64 input, nsamples samples (8-byte aligned).
 *   y_dev     device complex64 output [nsamples / D][K]: row m holds the K
 *             channels of output m (time-major), channel c at column c.
 *   nsamples  >= 0, a multiple of D (each output consumes one hop of D
 *             samples); 0 is a no-op.
 * The two ranges must not overlap.  Stream-ordered and asynchronous; the
 * state becomes the last Nh - 1 samples of {state, x} and the stream time
 * advances by nsamples, so consecutive calls equal one call over the
 * concatenated input.  Enqueues kernel launches only, so a run of calls
 * may be captured into a HIP graph; the stream time and the state buffer
 * of each call are fixed at capture, so replays continue the stream when
 * the captured run has an even number of calls (Nh > 1) and a multiple of
 * K samples in all.
 */
int fir_pfb_execute(fir_pfb_plan_t p, const void *x_dev, void *y_dev, int64_t nsamples,
                    void *stream);

/*
 * Replace the state: s_dev holds the Nh - 1 samples before the next call
 * (oldest first; NULL for zeros) and t_next is the stream time of the next
 * call's first sample (>= 0; the baseband phase uses it modulo K).
 * Stream-ordered and asynchronous.
 */
int fir_pfb_set_state(fir_pfb_plan_t p, const void *s_dev, int64_t t_next, void *stream);

/*
 * Copy the state (Nh - 1 samples) to s_out_dev and return the stream time
 * of the next call's first sample in *t_next (either may be NULL).
 */
int fir_pfb_get_state(fir_pfb_plan_t p, void *s_out_dev, int64_t *t_next, void *stream);

/* Wait for the plan's device, then free its buffers.  NULL is a no-op. */
int fir_pfb_destroy(fir_pfb_plan_t p);

#ifdef __cplusplus
}
#endif

#endif /* FIRPFB_H */
