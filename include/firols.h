/*
 * firols.h -- overlap-save FIR filtering on AMD Instinct MI355X (gfx950).
 *
 * The method is the one of the page "一种基于GPU的高阶数字FIR滤波器频域并行
 * 处理实现方法" (a GPU frequency-domain parallel method for high-order FIR
 * filters), claim 1:
 *   step 1  H = N-point DFT of the M taps zero-padded to N, or H given
 *           directly, kept in GPU memory;
 *   step 2  the input of a call is cut into blocks B_i of L samples;
 *   step 3  E_0 = {S0, B_0}, E_i = {D_(i-1), B_i}, where D_i is the last
 *           M-1 samples of B_i; D_(k-1) becomes the state S0 of the next call;
 *   step 4  F_i = FFT_N(E_i), I_i = F_i * H, R_i = IFFT_N(I_i);
 *   step 5  R_i = {Z_i, Y_i}: the first M-1 points Z_i are dropped and the
 *           L points Y_i are the output;
 *   step 6  the next input is processed the same way.
 * With N = L + M - 1 every kept point equals the linear convolution of the
 * taps with the stream {S0, X}:
 *       y[t] = sum_{m<M} h[m] * xt[t-m],  xt[j] = S0[M-1+j] for j < 0.
 *
 * Data types.  Samples are complex64: interleaved (re, im) float32 pairs.
 * The state S0 of a channel is M-1 samples in time order (S0[0] oldest).
 * Channel c of a [nchan][chan_stride] array starts at element c*chan_stride.
 *
 * Status.  Every function returns FIR_OLS_OK (0) or a negative status.  A
 * call that returns an error has enqueued nothing and changed nothing,
 * except FIR_OLS_ERR_HIP after a launch, which reports what the HIP runtime
 * said.  No function aborts or prints.
 *
 * Devices and streams.  A plan lives on the HIP device that was current
 * when it was created; every later call must be made with that device
 * current.  Stream arguments are hipStream_t values passed as void*; NULL
 * means the device's null stream.  A plan holds one filter state, so calls
 * on one plan must be ordered (one stream, or streams the caller orders).
 * Different plans are independent.
 */
#ifndef FIROLS_H
#define FIROLS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct fir_ols_plan_s *fir_ols_plan_t;   /* opaque, library-owned */

enum {
    FIR_OLS_OK = 0,
    FIR_OLS_ERR_INVALID_ARG = -1,  /* null handle/pointer, bad size or stride */
    FIR_OLS_ERR_UNSUPPORTED = -2,  /* size outside what the kernels cover */
    FIR_OLS_ERR_NO_FILTER = -3,    /* execute before set_taps/set_freq_response */
    FIR_OLS_ERR_ALIAS = -4,        /* input and output memory overlap */
    FIR_OLS_ERR_ALIGN = -5,        /* device pointer not aligned to its element (8 bytes; 4 for real rows) */
    FIR_OLS_ERR_OOM = -6,          /* device allocation failed */
    FIR_OLS_ERR_HIP = -7,          /* HIP runtime error (launch, copy, sync) */
    FIR_OLS_ERR_DEVICE = -8,       /* current device is not the plan's device */
    FIR_OLS_ERR_TIMEOUT = -9       /* a kernel's bounded wait ran out (fir_ols_check) */
};

/*
 * Create a plan for M taps and N-point blocks (claim 1, steps 1-2: N is the
 * transform length, the block length is L = N - M + 1).
 *   out    receives the handle (set to NULL on error).
 *   M      taps, 1 <= M <= N.
 *   N      power of two, 8 <= N <= 2^20 (1048576).
 *   nchan  independent channels sharing the filter, nchan >= 1; each has
 *          its own state.
 * Allocates the frequency response (aligned to 256 bytes, the page's
 * alignment rule in step 1), the twiddle tables and two state buffers of
 * nchan*(M-1) samples on the current device; for N = 65536 also a scratch
 * area of 512 KB for the synchronization flags of the two-workgroup kernel
 * that filters the blocks whose L outputs are all valid, plus N samples
 * (512 KB) per workgroup that fits on the device at once for the one-
 * workgroup kernel that filters a call's partial last block (129 x 512 KB
 * on a 256-CU MI355X); for N > 65536 a scratch area of 128 MiB (blocks of
 * N samples, at least one) through which the blocks of a call pass in
 * batches.  The state starts at zero.
 * No filter is set yet.  Synchronous.
 */
int fir_ols_plan(fir_ols_plan_t *out, int64_t M, int64_t N, int64_t nchan);

/*
 * Set the filter from its taps (claim 1, step 1, first case): the taps are
 * zero-padded to N and transformed on the GPU (for N >= 65536 a radix-N/32768
 * decimation with float64 phases, then 32768-point transforms); H is kept
 * scaled by 1/N so the inverse transform of step 4 needs no separate
 * scaling.
 *   h_host      host array: M float32 taps (is_complex == 0) or M
 *               interleaved complex64 taps (is_complex != 0); copied
 *               before return, the caller keeps ownership.
 *   M           must equal the plan's M.
 *   stream      stream the work is ordered on (after earlier executes).
 * Returns after H is in place.  Leaves the state unchanged.
 */
int fir_ols_set_taps(fir_ols_plan_t p, const float *h_host, int64_t M,
                     int is_complex, void *stream);

/*
 * Set the filter from its frequency response (claim 1, step 1, second
 * case).
 *   H_host  host array of N interleaved complex64 values: the unscaled
 *           forward DFT (kernel exp(-2 pi j q m / N)) of the zero-padded
 *           taps, bin 0 first.  Copied before return.
 *   N       must equal the plan's N.
 * The library applies the 1/N factor itself.  H is not checked for being
 * the response of an M-tap filter; if it is not, each output is the
 * circular convolution of its block E_i with IDFT(H) at index M-1+t.
 * Returns after H is in place.  Leaves the state unchanged.
 */
int fir_ols_set_freq_response(fir_ols_plan_t p, const float *H_host,
                              int64_t N, void *stream);

/*
 * Filter one call's input (claim 1, steps 2-5, with the state carry of
 * step 3).
 *   x_dev        device complex64 input, [nchan][chan_stride]; the first
 *                nsamples of every channel are read.
 *   y_dev        device complex64 output, same layout; the first nsamples
 *                of every channel are written, nothing else is touched.
 *   nsamples     samples per channel in this call, >= 0.  Any count is
 *                accepted: the last block may be partial (it is padded
 *                with zeros, which only reach dropped outputs).  0 is a
 *                no-op that leaves the state as it is.
 *   chan_stride  elements between channel starts, >= nsamples.
 *   stream       the call is enqueued on it and returns without waiting.
 * Both pointers must be 8-byte aligned and the two ranges must not
 * overlap (in-place filtering would let one block overwrite the overlap
 * another block still reads).  The state of every channel becomes the last
 * M-1 samples of {S0, x} of that channel.
 * The call enqueues kernel launches only (no allocation, copy, fill or
 * synchronization): one for N <= 32768; for N = 65536 a flag-clearing
 * kernel and the two-workgroup kernel per batch of up to 65536 full
 * blocks, and one launch for a partial last block; three per batch of
 * blocks for N > 65536.  So a run of calls may be captured into a HIP graph;
 * replays then carry the state like the calls they were captured from,
 * provided the captured run has an even number of calls with M > 1 (the
 * two state buffers alternate, and the plan's record of which one is
 * current changes at capture time, not at replay).
 */
int fir_ols_execute(fir_ols_plan_t p, const void *x_dev, void *y_dev,
                    int64_t nsamples, int64_t chan_stride, void *stream);

/*
 * Real-valued input (the samples of page 2's data are real float32): two real
 * streams filtered by a real filter at once.  Channel c of the plan is the
 * pair of real rows 2c and 2c + 1:
 *   x_dev, y_dev  device float32 [2 nchan][row_stride] (4-byte aligned).
 * Row 2c goes in as the real and row 2c + 1 as the imaginary part of one
 * complex stream; with real taps the real and imaginary parts of the
 * output are the two filtered rows, written to rows 2c and 2c + 1 of y.  A
 * real sample then moves 8 bytes (4 read, 4 written) against 16 for a
 * complex one.  The state is the plan's complex state (real part: row 2c's
 * last M-1 samples, imaginary part: row 2c + 1's), so fir_ols_set_state
 * and fir_ols_get_state hold the two rows' states packed the same way.
 * Stream-ordered and asynchronous like fir_ols_execute.
 * FIR_OLS_ERR_UNSUPPORTED unless the filter was set by fir_ols_set_taps
 * with real taps (any N); FIR_OLS_ERR_ALIGN for pointers not 4-byte
 * aligned; other errors as fir_ols_execute.
 */
int fir_ols_execute_real(fir_ols_plan_t p, const void *x_dev, void *y_dev,
                         int64_t nsamples, int64_t row_stride, void *stream);

/*
 * fir_ols_execute for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, layout, results, state carry and errors as
 * fir_ols_execute (complex64 input), and the same kernels; the call
 * allocates nothing.  The split (N = 65536) and multi-pass (N > 65536)
 * kernels work in a fixed array of device memory inside the library,
 * fir_ols_static_scratch_bytes() = 64 MiB, instead of the plan's own
 * scratch area; each GPU the call runs on holds its own copy of that array
 * until the process ends.  At N = 65536 the first 512 KB hold the flags of
 * the two-workgroup kernel and the rest 127 slots of 512 KB for the one-
 * workgroup kernel of partial last blocks (at most 127 of its workgroups
 * run); above 65536 the blocks go through the array in batches of as many
 * as it holds.  Plans with N <= 32768 use no scratch.  A plan whose block
 * would not fit the array gets FIR_OLS_ERR_UNSUPPORTED (no N the library
 * accepts needs more than 8 MiB).  Every call on one GPU shares that GPU's
 * array, whatever the plan: calls that may overlap in time on one GPU
 * (different streams, different threads) race on it and give wrong
 * results; order them on one stream.  The array's contents are whatever
 * the last call left; the kernels write every value before they read it.
 */
int fir_ols_execute_static(fir_ols_plan_t p, const void *x_dev, void *y_dev,
                           int64_t nsamples, int64_t chan_stride, void *stream);

/* Size in bytes of the array fir_ols_execute_static works in. */
int64_t fir_ols_static_scratch_bytes(void);

/*
 * Host-resident streaming (claim 1, steps 2 and 6: the samples arrive from
 * host memory in chunks and the filtered chunks go back to it).  Filters
 * nsamples per channel exactly as fir_ols_execute would, carrying the
 * state, but reads x from and writes y to host memory:
 *   x_host, y_host  host complex64 [nchan][chan_stride]; page-locked memory
 *                   (hipHostMalloc, or torch's pin_memory) lets the copies
 *                   run asynchronously and overlap the filtering; pageable
 *                   memory works but the runtime stages those copies.
 *   chunk           samples per channel per step (0: 2^22 / nchan rounded
 *                   up to whole blocks of L, about 32 MiB per staging slot),
 *                   clipped to nsamples.
 * The call cuts the stream into chunks and runs them through two device
 * staging slots owned by the plan ([nchan][chunk] complex64 each for input
 * and output, allocated on first use and grown when a larger chunk is
 * asked for): host-to-device copies on one internal stream, one
 * fir_ols_execute per chunk on `stream`, device-to-host copies on another
 * internal stream.  Everything is enqueued before the call returns; the
 * copies start after the work queued on `stream` before the call, and
 * `stream` passes the call only after the last output copy, so the caller
 * synchronizes `stream` before it reads y_host or reuses x_host.  Because
 * each chunk is a separate filtering call, the outputs equal those of
 * fir_ols_execute over the same chunks, bit for bit.  Not for HIP graph
 * capture (internal streams, first-use allocation).  Errors as
 * fir_ols_execute (FIR_OLS_ERR_ALIAS when the two host ranges overlap,
 * FIR_OLS_ERR_OOM when the staging slots cannot be allocated); a failure
 * after the first chunk was enqueued returns FIR_OLS_ERR_HIP with the
 * state advanced by the chunks already enqueued.
 */
int fir_ols_execute_host(fir_ols_plan_t p, const void *x_host, void *y_host,
                         int64_t nsamples, int64_t chan_stride, int64_t chunk,
                         void *stream);

/*
 * Replace the state (claim 1, step 3: S0 is the M-1 samples that preceded
 * the call).
 *   s0_dev  device complex64 [nchan][M-1], time order, or NULL for zeros.
 * Stream-ordered and asynchronous.  With M == 1 there is no state and the
 * call is a no-op.
 */
int fir_ols_set_state(fir_ols_plan_t p, const void *s0_dev, void *stream);

/*
 * Copy the current state out, e.g. to checkpoint a stream and resume it in
 * another plan with fir_ols_set_state.
 *   s0_out_dev  device complex64 [nchan][M-1].
 * Stream-ordered and asynchronous.
 */
int fir_ols_get_state(fir_ols_plan_t p, void *s0_out_dev, void *stream);

/*
 * Kernel-side errors of the calls enqueued so far.  For N = 65536 the
 * second workgroup of a block waits, bounded to 0.5 s, for the first to
 * park its half-spectrum (claim 1, step 4 split over two workgroups).  The
 * launch order means the first is always running, so the bound is not
 * reached in normal operation.  If it is, that wait gives up, the block's
 * outputs are written as quiet NaN, and the plan's device error word is
 * set.  fir_ols_check synchronizes `stream`, reads and clears that word,
 * and returns FIR_OLS_ERR_TIMEOUT if it was set (FIR_OLS_OK otherwise, or
 * FIR_OLS_ERR_HIP / FIR_OLS_ERR_DEVICE).  Calls through
 * fir_ols_execute_static report through the same word.  The environment
 * variable FIROLS_PAIR_HOLD_READY=1 at plan creation makes every such wait
 * run out after 10 us (a test of this path; never set it otherwise).
 */
int fir_ols_check(fir_ols_plan_t p, void *stream);

/*
 * Destroy a plan: waits for the plan's device to finish, then frees its
 * buffers.  NULL is a no-op.
 */
int fir_ols_destroy(fir_ols_plan_t p);

/*
 * Planner choice of N (claim 1, step 1 leaves the FFT length free): the
 * power of two N >= max(M, 256) that maximizes the predicted output rate
 * (N - M + 1) x blocks_per_second(N), from a table of block rates measured
 * on MI355X (one long single-channel call per N).  Returns N,
 * FIR_OLS_ERR_INVALID_ARG for M < 1, or FIR_OLS_ERR_UNSUPPORTED for
 * M > 2^20.  Pure host arithmetic: no device call.
 */
int64_t fir_ols_choose_n(int64_t M);

/* Block length L = N - M + 1 of a plan, or a negative status. */
int64_t fir_ols_block_length(fir_ols_plan_t p);

/* Static text for a status code. */
const char *fir_ols_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FIROLS_H */
