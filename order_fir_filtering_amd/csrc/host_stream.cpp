// Host-resident streaming: the input comes from host memory and the output
// goes back to it (the method page, claim 1, steps 2 and 6: the stream is
// cut into chunks on the host and the filtered chunks returned).  The
// chunks run through two device staging slots in a three-stage pipeline:
// host-to-device copy on one stream, the filtering call on the caller's
// stream, device-to-host copy on another stream, so the copies of one
// chunk overlap the filtering of the next.  Argument meaning and error
// behaviour are documented in include/firols.h.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "firols.h"
#include "plan.hpp"

namespace {

enum { EV_IN = 0, EV_COMP = 2, EV_OUT = 4, EV_START = 6, EV_END = 7 };

void free_slots(fir_ols_plan_s *p) {
    for (int s = 0; s < 2; ++s) {
        (void)hipFree(p->hs_x[s]);
        (void)hipFree(p->hs_y[s]);
        p->hs_x[s] = p->hs_y[s] = nullptr;
    }
    p->hs_chunk = 0;
}

// Streams and events on first use; staging slots of at least `chunk`
// samples per channel (reallocated, after the pipeline has drained, when
// a larger chunk is asked for).
int prepare(fir_ols_plan_s *p, int64_t chunk) {
    if (!p->hs_in) {
        // all or nothing: a failure leaves no stream or event behind
        bool ok = hipStreamCreateWithFlags(&p->hs_in, hipStreamNonBlocking) == hipSuccess &&
                  hipStreamCreateWithFlags(&p->hs_out, hipStreamNonBlocking) == hipSuccess;
        for (hipEvent_t &e : p->hs_ev)
            ok = ok && hipEventCreateWithFlags(&e, hipEventDisableTiming) == hipSuccess;
        if (!ok) {
            (void)hipGetLastError();
            release_host_stream(p);
            return FIR_OLS_ERR_HIP;
        }
    }
    if (chunk <= p->hs_chunk) return FIR_OLS_OK;
    // earlier calls may still read or write the old slots
    if (hipStreamSynchronize(p->hs_in) != hipSuccess ||
        hipStreamSynchronize(p->hs_out) != hipSuccess ||
        hipEventSynchronize(p->hs_ev[EV_END]) != hipSuccess)
        return FIR_OLS_ERR_HIP;
    free_slots(p);
    const size_t bytes = (size_t)p->nchan * (size_t)chunk * sizeof(float2);
    for (int s = 0; s < 2; ++s) {
        if (hipMalloc(&p->hs_x[s], bytes) != hipSuccess ||
            hipMalloc(&p->hs_y[s], bytes) != hipSuccess) {
            (void)hipGetLastError();
            free_slots(p);
            return FIR_OLS_ERR_OOM;
        }
    }
    p->hs_chunk = chunk;
    return FIR_OLS_OK;
}

}  // namespace

void release_host_stream(fir_ols_plan_s *p) {
    if (p->hs_in) (void)hipStreamSynchronize(p->hs_in);
    if (p->hs_out) (void)hipStreamSynchronize(p->hs_out);
    free_slots(p);
    for (hipEvent_t &e : p->hs_ev) {
        if (e) (void)hipEventDestroy(e);
        e = nullptr;
    }
    if (p->hs_in) (void)hipStreamDestroy(p->hs_in);
    if (p->hs_out) (void)hipStreamDestroy(p->hs_out);
    p->hs_in = p->hs_out = nullptr;
}

extern "C" int fir_ols_execute_host(fir_ols_plan_t p, const void *x_host, void *y_host,
                                    int64_t nsamples, int64_t chan_stride, int64_t chunk,
                                    void *stream) {
    if (!p || nsamples < 0 || chunk < 0) return FIR_OLS_ERR_INVALID_ARG;
    if (!p->has_filter) return FIR_OLS_ERR_NO_FILTER;
    if (nsamples == 0) return FIR_OLS_OK;
    if (!x_host || !y_host || chan_stride < nsamples) return FIR_OLS_ERR_INVALID_ARG;
    if (chan_stride > ((int64_t)1 << 50) / p->nchan) return FIR_OLS_ERR_INVALID_ARG;
    const int64_t span = ((p->nchan - 1) * chan_stride + nsamples) * (int64_t)sizeof(float2);
    const uintptr_t xa = (uintptr_t)x_host, ya = (uintptr_t)y_host;
    if (xa < ya + (uintptr_t)span && ya < xa + (uintptr_t)span) return FIR_OLS_ERR_ALIAS;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != p->device) return FIR_OLS_ERR_DEVICE;
    if (chunk == 0) {
        // about 32 MiB per staging slot, in whole blocks, at least one block
        int64_t want = ((int64_t)1 << 22) / p->nchan;
        if (want < 1) want = 1;
        chunk = (want + p->L - 1) / p->L * p->L;
    }
    if (chunk > nsamples) chunk = nsamples;
    if (chunk > ((int64_t)1 << 40) / p->nchan) return FIR_OLS_ERR_INVALID_ARG;
    int st = prepare(p, chunk);
    if (st != FIR_OLS_OK) return st;

    hipStream_t sc = (hipStream_t)stream;
    hipEvent_t *ev = p->hs_ev;
    const size_t hpitch = (size_t)chan_stride * sizeof(float2);
    const size_t dpitch = (size_t)p->hs_chunk * sizeof(float2);
    // the first copies wait for what the caller queued before this call
    if (hipEventRecord(ev[EV_START], sc) != hipSuccess ||
        hipStreamWaitEvent(p->hs_in, ev[EV_START], 0) != hipSuccess)
        return FIR_OLS_ERR_HIP;
    int k = 0;
    for (int64_t c0 = 0; c0 < nsamples; c0 += chunk, ++k) {
        const int s = k & 1;
        const int64_t n = nsamples - c0 < chunk ? nsamples - c0 : chunk;
        const size_t w = (size_t)n * sizeof(float2);
        // slot s is free once the output copy of chunk k - 2 is done (that
        // copy itself waited for the filtering of chunk k - 2)
        if (hipStreamWaitEvent(p->hs_in, ev[EV_OUT + s], 0) != hipSuccess ||
            hipMemcpy2DAsync(p->hs_x[s], dpitch, (const char *)x_host + c0 * sizeof(float2), hpitch,
                             w, (size_t)p->nchan, hipMemcpyHostToDevice, p->hs_in) != hipSuccess ||
            hipEventRecord(ev[EV_IN + s], p->hs_in) != hipSuccess ||
            hipStreamWaitEvent(sc, ev[EV_IN + s], 0) != hipSuccess ||
            hipStreamWaitEvent(sc, ev[EV_OUT + s], 0) != hipSuccess)
            return FIR_OLS_ERR_HIP;
        st = fir_ols_execute(p, p->hs_x[s], p->hs_y[s], n, p->hs_chunk, sc);
        if (st != FIR_OLS_OK) return st;
        if (hipEventRecord(ev[EV_COMP + s], sc) != hipSuccess ||
            hipStreamWaitEvent(p->hs_out, ev[EV_COMP + s], 0) != hipSuccess ||
            hipMemcpy2DAsync((char *)y_host + c0 * sizeof(float2), hpitch, p->hs_y[s], dpitch, w,
                             (size_t)p->nchan, hipMemcpyDeviceToHost, p->hs_out) != hipSuccess ||
            hipEventRecord(ev[EV_OUT + s], p->hs_out) != hipSuccess)
            return FIR_OLS_ERR_HIP;
    }
    // the caller's stream passes this call only after the last output copy
    if (hipEventRecord(ev[EV_END], p->hs_out) != hipSuccess ||
        hipStreamWaitEvent(sc, ev[EV_END], 0) != hipSuccess)
        return FIR_OLS_ERR_HIP;
    return FIR_OLS_OK;
}
